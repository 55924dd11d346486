// Per-block top-r selection and group construction.
//
// "HTTM: Head-wise Temporal Token Merging for Faster VGGT", key design 1: the
// r matched sources with the highest similarity merge into their destination;
// a merged token stands for its destination and those sources.  Ties go to
// the smaller source position.
//
// One workgroup (8 waves) per (stream, head, block) works in registers and LDS:
//   1. if 0 < r < |S|: radix select (four 8-bit LDS histogram passes) of the
//      r-th smallest key (descending score as an unsigned key); sources with a
//      smaller key merge, sources equal to it merge in ascending source order
//      until r are taken;
//   2. every block position gets a group: its own index for a destination,
//      the matched destination for a merged source, and |D| for the other
//      sources (they follow as singletons);
//   3. a stable counting sort by group gives the CSR: positions are visited
//      in ascending original token id (block position order for frame-major
//      blocks; for frame-minor blocks the frame-major enumeration of the same
//      block), each wave ranks its contiguous segment of that enumeration 64
//      at a time (lanes with equal groups are found with one ballot per key
//      bit), and a scan over (group, wave) turns per-wave counts into
//      offsets, so members ascend by token id inside a group (the order of
//      the means' sums).
// Everything is integer work after the float-to-key transform, so the result
// is deterministic.  Extra workgroups fill the special-token slots.
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = kMaxBlock / kThreads;     // sources per thread
constexpr int kMaxGroups = kMaxBlock / 2 + 1;  // destinations (stride >= 2) + the singleton class
constexpr int kGroupBits = 12;                 // 2^12 > kMaxGroups - 1
static_assert((1 << kGroupBits) >= kMaxGroups, "group id bits");

struct SelArgs {
  Geo g;
  int st0;  // first stream handled by this launch
  const int32_t* match[2];
  const float* score[2];
  Csr csr[2];
};

// Exclusive scan of one value per thread over the 512-thread block.
__device__ __forceinline__ uint32_t scan512(uint32_t v, uint32_t* sh /* >= kWaves + 1 */, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t acc = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = sh[w];
      sh[w] = acc;
      acc += t;
    }
    sh[kWaves] = acc;
  }
  __syncthreads();
  total = sh[kWaves];
  const uint32_t r = sh[wave] + x - v;
  __syncthreads();  // sh may be reused right after
  return r;
}

// Lanes of this wave whose (valid) key equals mine: one ballot per key bit.
__device__ __forceinline__ uint64_t match_any(uint32_t key, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < kGroupBits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__global__ __launch_bounds__(kThreads) void block_select(SelArgs a) {
  __shared__ int32_t sGrp[kMaxBlock];                      // source -> group
  __shared__ uint16_t sCnt[kWaves][kMaxGroups + 7];        // per-wave counts, then starts
  __shared__ uint32_t sHist[256];
  __shared__ uint32_t sSh[kWaves + 1];
  __shared__ uint32_t sRes[2];
  const Geo& g = a.g;
  const int per_head = g.nblocks + 1;
  const int st = a.st0 + blockIdx.x / (g.heads * per_head);
  const int rem_ = blockIdx.x % (g.heads * per_head);
  const int head = rem_ / per_head;
  const int b = rem_ % per_head;
  const Csr c = a.csr[st];
  const size_t tokbase = (size_t)head * g.N;
  const size_t slotbase = (size_t)head * (g.nslots[st] + 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (b == g.nblocks) {
    // special tokens: one slot each, after the patch slots; then the end marker
    const int nspec = g.F * g.nsp;
    const int slot_sp0 = g.nslots[st] - nspec;
    for (int e = tid; e < nspec; e += kThreads) {
      const int tok = (e / g.nsp) * g.T + (e % g.nsp);
      c.members[tokbase + g.P + e] = tok;
      c.off[slotbase + slot_sp0 + e] = g.P + e;
      c.group[tokbase + tok] = slot_sp0 + e;
    }
    if (tid == 0) c.off[slotbase + g.nslots[st]] = g.N;
    return;
  }

  const BlockInfo bi = block_info(g, b, st);
  const int s = g.s[st];
  const int nd = bi.nd, ns = bi.ns, r = bi.r;
  const int32_t* match = a.match[st] + (size_t)head * g.nsrc[st] + bi.src0;
  const float* score = a.score[st] + (size_t)head * g.nsrc[st] + bi.src0;

  // 1. which sources merge (thread t owns sources t*kPer .. t*kPer + kPer - 1)
  const int k0 = tid * kPer;
  int mk[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int k = k0 + e;
    const int m = k < ns ? match[k] : 0;
    mk[e] = (unsigned)m < (unsigned)nd ? m : 0;
  }
  uint32_t selbits = 0;
  if (r >= ns) {
    selbits = (1u << kPer) - 1u;
  } else if (r > 0) {
    uint32_t key[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) key[e] = k0 + e < ns ? ~float_key(score[k0 + e] + 0.0f) : 0u;
    uint32_t prefix = 0, want = (uint32_t)r;  // want-th smallest among keys matching prefix
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) sHist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const bool in = k0 + e < ns && (pass == 0 || (key[e] >> (shift + 8)) == prefix);
        if (in) atomicAdd(&sHist[(key[e] >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t h[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h[j] = sHist[4 * lane + j];
          sum += h[j];
        }
        uint32_t x = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const uint32_t y = __shfl_up(x, d);
          if (lane >= d) x += y;
        }
        uint32_t below = x - sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (below < want && below + h[j] >= want) {
            sRes[0] = 4 * lane + j;
            sRes[1] = want - below;
          }
          below += h[j];
        }
      }
      __syncthreads();
      prefix = (prefix << 8) | sRes[0];
      want = sRes[1];
      __syncthreads();  // sRes / sHist reused by the next pass
    }
    // keys below the threshold merge; equal keys take the remaining `want` in source order
    uint32_t eq = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) eq += (k0 + e < ns && key[e] == prefix) ? 1u : 0u;
    uint32_t tot;
    uint32_t rank = scan512(eq, sSh, tot);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (k0 + e >= ns) continue;
      bool take = key[e] < prefix;
      if (key[e] == prefix) {
        take = rank < want;
        ++rank;
      }
      selbits |= take ? (1u << e) : 0u;
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    if (k0 + e < ns) sGrp[k0 + e] = ((selbits >> e) & 1u) ? mk[e] : nd;
  const int G = nd + 1;  // destinations and the singleton class
  for (int i = tid; i < kWaves * G; i += kThreads) sCnt[i / G][i % G] = 0;
  __syncthreads();

  // 2-3a. group of every position; per-wave stable ranks.  Wave w owns the
  // contiguous enumeration indices [w*pw, (w+1)*pw); index u is the u-th
  // token of the block in ascending token id, at block position pos(u).
  const int pw = ceil_div(bi.n, kThreads) * 64;  // multiple of 64, kWaves * pw >= n
  const int chunks = pw / 64;
  auto pos = [&](int u) { return g.order ? (u % bi.run) * bi.nf + u / bi.run : u; };
  int grp[kPer], lrank[kPer];
#pragma unroll
  for (int ch = 0; ch < kPer; ++ch) {
    if (ch >= chunks) break;  // uniform over the workgroup
    const int u = wave * pw + ch * 64 + lane;
    const bool valid = u < bi.n;
    const int i = valid ? pos(u) : 0;
    int gi = 0;
    if (valid) gi = (i % s == 0) ? i / s : sGrp[i - i / s - 1];
    const uint64_t eqm = match_any((uint32_t)gi, valid);
    const uint64_t lt = (1ull << lane) - 1ull;
    int rk = 0;
    if (valid) {
      rk = (int)sCnt[wave][gi] + __popcll(eqm & lt);
    }
    // the highest lane of each class advances the wave's running count
    if (valid && (eqm >> lane) == 1ull) sCnt[wave][gi] = (uint16_t)(rk + 1);
    grp[ch] = gi;
    lrank[ch] = rk;
  }
  __syncthreads();

  // 3b. starts[w][g] = gstart[g] + sum_{w' < w} cnt[w'][g]; destination offsets
  const int gper = ceil_div(G, kThreads);
  const int gb = tid * gper, ge = min(G, gb + gper);
  uint32_t local = 0;
  for (int gg = gb; gg < ge; ++gg)
    for (int w = 0; w < kWaves; ++w) local += sCnt[w][gg];
  uint32_t gtot;
  uint32_t acc = scan512(local, sSh, gtot);
  for (int gg = gb; gg < ge; ++gg) {
    if (gg < nd) c.off[slotbase + bi.slot0 + gg] = bi.start + (int)acc;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t n = sCnt[w][gg];
      sCnt[w][gg] = (uint16_t)acc;
      acc += n;
    }
  }
  __syncthreads();

  // 3c. scatter
  const int first_single = nd + r;
#pragma unroll
  for (int ch = 0; ch < kPer; ++ch) {
    if (ch >= chunks) break;
    const int u = wave * pw + ch * 64 + lane;
    if (u >= bi.n) continue;
    const int i = pos(u);
    const int gi = grp[ch];
    const int p = (int)sCnt[wave][gi] + lrank[ch];
    const int tok = block_token(g, bi, i);
    c.members[tokbase + bi.start + p] = tok;
    int slot;
    if (gi < nd) {
      slot = bi.slot0 + gi;
    } else {
      slot = bi.slot0 + nd + (p - first_single);
      c.off[slotbase + slot] = bi.start + p;
    }
    c.group[tokbase + tok] = slot;
  }
}

}  // namespace

hipError_t launch_select(const Geo& g, const int32_t* match_q, const float* score_q,
                         const int32_t* match_k, const float* score_k, Csr q, Csr k, int streams,
                         hipStream_t stream) {
  if ((streams & 3) == 0) return hipSuccess;
  SelArgs a;
  a.g = g;
  a.st0 = (streams & 1) ? 0 : 1;
  const int nst = (streams & 1) + ((streams >> 1) & 1);
  a.match[0] = match_q;
  a.match[1] = match_k;
  a.score[0] = score_q;
  a.score[1] = score_k;
  a.csr[0] = q;
  a.csr[1] = k;
  const int grid = nst * g.heads * (g.nblocks + 1);
  hipLaunchKernelGGL(block_select, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace httm
