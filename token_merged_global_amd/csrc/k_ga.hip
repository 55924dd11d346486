// Geometry-aware three-class partition and global matching.
//
// "LiteVGGT: Boosting Vanilla VGGT via Geometry-aware Cached Token Merging",
// key design 1: a geometry score per token (here its token-variance half:
// the variance of the features in the token's 3x3 neighbourhood on its
// frame's patch grid); key design 2: per frame, the highest-score patches are
// protected, destinations are every unprotected patch of the first frame and
// the lowest-score unprotected patch of each 2x2 cell in the other frames,
// the rest are sources; key design 3: every source joins its most similar
// destination (cosine) over the whole sequence and each destination's group
// is merged by the mean.  Like HTTM's matching this runs per head and per
// stream (Q and K).
//
// The groups are handed to the rest of the layer in the same form as the
// block-local matching produces: per head a CSR of members (ascending token
// ids inside a group) over `bound` slots, slots past the head's group count
// empty, and the group (slot) of every token.
//
// Pipeline: ga_variance -> ga_roles (per frame: radix top-k, 2x2 minima) ->
// ga_scan (per-frame offsets) -> ga_slots (anchor slots, destination and
// source lists) -> ga_match (MFMA cosine argmax of sources against all
// destinations; member counts per slot) -> ga_offsets (slot offsets) ->
// ga_place (every token into its slot's range, any order) -> ga_rank (each
// member's place inside its range = members with a smaller id).  No sort
// and no memset: the result does not depend on the order of the atomics.
#include "common.h"
#include "kernels.h"
#include "sim_tile.h"

namespace httm {

namespace {

#define HTTM_DISPATCH_T(dtype, ...) \
  do {                              \
    if ((dtype) == 1) {             \
      typedef uint16_t T;           \
      __VA_ARGS__;                  \
    } else {                        \
      typedef float T;              \
      __VA_ARGS__;                  \
    }                               \
  } while (0)

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x) { Row8<T>::load(p, x); }

constexpr int kRoleSrc = 0, kRoleDst = 1, kRoleProtect = 2, kRoleSpecial = 3;

// fp32 sum of the available cells (centre, and left / right when present),
// left to right, for 8 channels.
__device__ __forceinline__ void row3(const float* l, const float* c, const float* r, bool hl, bool hr, float* o) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float t = hl ? __fadd_rn(l[e], c[e]) : c[e];
    o[e] = hr ? __fadd_rn(t, r[e]) : t;
  }
}

// Variance map: one thread per patch.  Per channel octet: the three rows'
// sums (x and x*x) left to right, then top to bottom; var = s2/cnt -
// (s1/cnt)^2 summed over channels in ascending order, divided by 64.
template <typename T>
__global__ __launch_bounds__(256) void ga_variance(const T* __restrict__ q, const T* __restrict__ k, int heads,
                                                   int N, int Tf, int nsp, int H, int W,
                                                   float* __restrict__ var) {
  const int HW = H * W;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int f = blockIdx.y;
  const int sh = blockIdx.z, st = sh / heads, head = sh % heads;
  if (j < nsp) var[((size_t)st * heads + head) * N + (size_t)f * Tf + j] = 0.f;  // specials: no score
  if (j >= HW) return;
  const T* X = (st == 0 ? q : k) + (size_t)head * N * kD;
  const int y = j / W, xx = j - y * W;
  const bool hl = xx > 0, hr = xx + 1 < W, hu = y > 0, hd = y + 1 < H;
  const float cnt = (float)((1 + hl + hr) * (1 + hu + hd));
  const T* base = X + ((size_t)f * Tf + nsp) * kD;
  float acc = 0.f;
  for (int c8 = 0; c8 < 8; ++c8) {
    float s1[8], s2[8];
    for (int dy = -1; dy <= 1; ++dy) {
      if ((dy < 0 && !hu) || (dy > 0 && !hd)) continue;
      const T* row = base + (size_t)((y + dy) * W + xx) * kD + c8 * 8;
      float a[8], b[8], c[8], a2[8], b2[8], c2[8];
      load8(row, b);
      if (hl) load8(row - kD, a);
      if (hr) load8(row + kD, c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a2[e] = hl ? __fmul_rn(a[e], a[e]) : 0.f;
        b2[e] = __fmul_rn(b[e], b[e]);
        c2[e] = hr ? __fmul_rn(c[e], c[e]) : 0.f;
      }
      float h1[8], h2[8];
      row3(a, b, c, hl, hr, h1);
      row3(a2, b2, c2, hl, hr, h2);
      if (dy < 0 || (dy == 0 && !hu)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s1[e] = h1[e];
          s2[e] = h2[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s1[e] = __fadd_rn(s1[e], h1[e]);
          s2[e] = __fadd_rn(s2[e], h2[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float m = s1[e] / cnt;
      acc = __fadd_rn(acc, __fsub_rn(s2[e] / cnt, __fmul_rn(m, m)));
    }
  }
  var[((size_t)st * heads + head) * N + (size_t)f * Tf + nsp + j] = acc / 64.0f;
}

constexpr int kRoleThreads = 256;

// Exclusive prefix over the workgroup's threads (thread order) and the total.
__device__ __forceinline__ int wg_excl_scan(int x, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kRoleThreads / 64; ++w) {
    const int t = wsum[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + inc - x;
}

// Roles of one frame: the k_protect largest scores are protected (ties to
// the smaller patch), then destinations (first frame: every other patch;
// other frames: the lowest-score unprotected patch of each 2x2 cell, ties to
// the smaller patch), sources for the rest.  Counts anchors (non-sources,
// specials included), destinations and sources per frame.
__global__ __launch_bounds__(kRoleThreads) void ga_roles(const float* __restrict__ var, int heads, int N, int Tf,
                                                          int nsp, int H, int W, int F, int k_protect,
                                                          uint8_t* __restrict__ role, int32_t* __restrict__ fcnt) {
  __shared__ uint32_t sKey[kMaxFrameHW];
  __shared__ uint8_t sRole[kMaxFrameHW];
  __shared__ uint32_t sHist[256];
  __shared__ uint32_t sSel[2];
  __shared__ int wsum[kRoleThreads / 64];
  __shared__ int sCnt[2];
  const int HW = H * W;
  const int f = blockIdx.x, sh = blockIdx.y, st = sh / heads, head = sh % heads;
  const int tid = threadIdx.x;
  const size_t tok0 = (size_t)f * Tf + nsp;
  const float* V = var + ((size_t)st * heads + head) * N + tok0;
  for (int j = tid; j < HW; j += kRoleThreads) sKey[j] = float_key(V[j] + 0.0f);
  if (tid < 2) sCnt[tid] = 0;
  __syncthreads();
  // radix select of the k-th largest key, 8 bits at a time
  uint32_t prefix = 0, kk = (uint32_t)k_protect;
  const bool any = k_protect > 0 && k_protect < HW;
  for (int pass = 0; pass < 4 && any; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kRoleThreads) sHist[i] = 0;
    __syncthreads();
    const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (32 - 8 * pass));
    for (int j = tid; j < HW; j += kRoleThreads) {
      const uint32_t key = sKey[j];
      if ((key & hmask) == prefix) atomicAdd(&sHist[(key >> shift) & 0xFF], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t above = 0;
      int b = 255;
      for (; b > 0; --b) {
        if (above + sHist[b] >= kk) break;
        above += sHist[b];
      }
      sSel[0] = prefix | ((uint32_t)b << shift);
      sSel[1] = kk - above;
    }
    __syncthreads();
    prefix = sSel[0];
    kk = sSel[1];
    __syncthreads();
  }
  // protected: key above the threshold, or equal and among the first kk equal keys by patch
  const int per = ceil_div(HW, kRoleThreads);
  const int j0 = tid * per, j1 = min(HW, j0 + per);
  int eq = 0;
  if (any)
    for (int j = j0; j < j1; ++j) eq += sKey[j] == prefix;
  int total;
  int rank = wg_excl_scan(eq, wsum, total);
  for (int j = j0; j < j1; ++j) {
    bool prot;
    if (k_protect <= 0) prot = false;
    else if (k_protect >= HW) prot = true;
    else if (sKey[j] > prefix) prot = true;
    else if (sKey[j] == prefix) prot = (uint32_t)(rank++) < kk;
    else prot = false;
    sRole[j] = prot ? kRoleProtect : (f == 0 ? kRoleDst : kRoleSrc);
  }
  __syncthreads();
  if (f > 0) {
    const int cw = (W + 1) / 2, ncell = cw * ((H + 1) / 2);
    for (int c = tid; c < ncell; c += kRoleThreads) {
      const int cy = (c / cw) * 2, cx = (c % cw) * 2;
      int best = -1;
      uint32_t bk = 0;
      for (int dy = 0; dy < 2; ++dy)
        for (int dx = 0; dx < 2; ++dx) {
          const int y = cy + dy, x = cx + dx;
          if (y >= H || x >= W) continue;
          const int j = y * W + x;
          if (sRole[j] == kRoleProtect) continue;
          if (best < 0 || sKey[j] < bk || (sKey[j] == bk && j < best)) {
            best = j;
            bk = sKey[j];
          }
        }
      if (best >= 0) sRole[best] = kRoleDst;
    }
  }
  __syncthreads();
  uint8_t* R = role + ((size_t)st * heads + head) * N + (size_t)f * Tf;
  int nd = 0, ns = 0;
  for (int j = tid; j < HW; j += kRoleThreads) {
    const uint8_t r = sRole[j];
    R[nsp + j] = r;
    nd += r == kRoleDst;
    ns += r == kRoleSrc;
  }
  for (int j = tid; j < nsp; j += kRoleThreads) R[j] = kRoleSpecial;
  if (nd) atomicAdd(&sCnt[0], nd);
  if (ns) atomicAdd(&sCnt[1], ns);
  __syncthreads();
  if (tid == 0) {
    int32_t* c = fcnt + (((size_t)st * heads + head) * F + f) * 3;
    c[0] = Tf - sCnt[1];  // anchors: every token that is not a source
    c[1] = sCnt[0];
    c[2] = sCnt[1];
  }
}

// Per (stream, head): exclusive prefixes of the per-frame counts, and totals.
__global__ __launch_bounds__(256) void ga_scan(const int32_t* __restrict__ fcnt, int F, int heads,
                                               int32_t* __restrict__ foff, int32_t* __restrict__ tot,
                                               int32_t* __restrict__ lenk) {
  __shared__ int wsum[4];
  const int sh = blockIdx.x;
  const int32_t* c = fcnt + (size_t)sh * F * 3;
  int32_t* o = foff + (size_t)sh * F * 3;
  const int per = ceil_div(F, 256);
  const int f0 = threadIdx.x * per, f1 = min(F, f0 + per);
  for (int t = 0; t < 3; ++t) {
    int loc = 0;
    for (int f = f0; f < f1; ++f) loc += c[f * 3 + t];
    int total;
    int acc = wg_excl_scan(loc, wsum, total);
    for (int f = f0; f < f1; ++f) {
      o[f * 3 + t] = acc;
      acc += c[f * 3 + t];
    }
    if (threadIdx.x == 0) {
      tot[sh * 3 + t] = total;
      if (t == 0 && sh >= heads) lenk[sh - heads] = total;  // keys per head: the key stream's groups
    }
  }
}

// Per (stream, head, frame): slots of the anchors in token order, the
// destination list (with each destination's slot) and the source list.
__global__ __launch_bounds__(kRoleThreads) void ga_slots(const uint8_t* __restrict__ role, int heads, int N, int Tf,
                                                          int F, int bound, const int32_t* __restrict__ foff,
                                                          int32_t* __restrict__ slot, int32_t* __restrict__ dst_list,
                                                          int32_t* __restrict__ dst_slot,
                                                          int32_t* __restrict__ src_list, int32_t* __restrict__ gdst,
                                                          float* __restrict__ gscore, int32_t* __restrict__ cnt,
                                                          int32_t* __restrict__ fill) {
  __shared__ int wsum[kRoleThreads / 64];
  const int f = blockIdx.x, sh = blockIdx.y;
  const size_t hb = (size_t)sh * N;
  const uint8_t* R = role + hb + (size_t)f * Tf;
  const int32_t* o = foff + ((size_t)sh * F + f) * 3;
  const int per = ceil_div(Tf, kRoleThreads);
  const int t0 = threadIdx.x * per, t1 = min(Tf, t0 + per);
  int na = 0, nd = 0, ns = 0;
  for (int t = t0; t < t1; ++t) {
    const uint8_t r = R[t];
    na += r != kRoleSrc;
    nd += r == kRoleDst;
    ns += r == kRoleSrc;
  }
  int tot_a, tot_d, tot_s;
  int ra = o[0] + wg_excl_scan(na, wsum, tot_a);
  int rd = o[1] + wg_excl_scan(nd, wsum, tot_d);
  int rs = o[2] + wg_excl_scan(ns, wsum, tot_s);
  for (int t = t0; t < t1; ++t) {
    const uint8_t r = R[t];
    const int tok = f * Tf + t;
    if (r != kRoleSrc) {
      slot[hb + tok] = ra;
      gdst[hb + tok] = -1;
      gscore[hb + tok] = 0.f;
      cnt[(size_t)sh * bound + ra] = 1;  // the anchor; ga_match adds the sources
      fill[(size_t)sh * bound + ra] = 0;
      if (r == kRoleDst) {
        dst_list[hb + rd] = tok;
        dst_slot[hb + rd] = ra;
        ++rd;
      }
      ++ra;
    } else {
      slot[hb + tok] = -1;
      src_list[hb + rs++] = tok;
    }
  }
}

// Global match, bf16: per (stream, head, 256 sources) like the block-local
// similarity kernel, with source and destination rows taken from the lists.
constexpr int kSrcPerWg = 256, kDstTile = 64;
struct GaMatchArgs {
  const void* x[2];
  int heads, N, chunks;
  const int32_t* tot;       // [2][h][3]: anchors, destinations, sources
  const int32_t* dst_list;  // [2][h][N]
  const int32_t* dst_slot;
  const int32_t* src_list;
  int32_t* gdst;            // [2][h][N] matched destination token (sources)
  int32_t* gslot;           // [2][h][N] its slot
  float* gscore;            // [2][h][N] cosine
  int32_t* cnt;             // [2][h][bound] members per slot (atomic adds)
  int bound;
};

__global__ __launch_bounds__(256) void ga_match_bf16(GaMatchArgs a) {
  __shared__ u32x4 sD[2][kDstTile * 8];
  __shared__ __attribute__((aligned(16))) float sInv[2][kDstTile];
  const int chunk = blockIdx.x % a.chunks, sh = blockIdx.x / a.chunks;
  const int st = sh / a.heads, head = sh % a.heads;
  const int nd = a.tot[sh * 3 + 1], ns = a.tot[sh * 3 + 2];
  if (chunk * kSrcPerWg >= ns || nd == 0) return;
  const size_t hb = (size_t)sh * a.N;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x[st]) + (size_t)head * a.N * kD;
  const int32_t* DL = a.dst_list + hb;
  const int32_t* SL = a.src_list + hb;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lg = lane >> 4, l16 = lane & 15;
  bf16x8 bs[4][2];
  float off[4], invs[4];
  int ksrc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int kidx = chunk * kSrcPerWg + wave * 64 + c * 16 + l16;
    ksrc[c] = kidx;
    const int tok = SL[kidx < ns ? kidx : 0];
    const uint16_t* row = X + (size_t)tok * kD;
    float ss = 0.f;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(row + kc * 32 + lg * 8);
      bs[c][kc] = __builtin_bit_cast(bf16x8, u);
      ss = sumsq8(bs[c][kc], ss);
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    off[c] = __builtin_amdgcn_sqrtf(ss) * (1.0f + 0x1p-10f);
    invs[c] = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
  }
  uint32_t best[4] = {0u, 0u, 0u, 0u}, bestT[4] = {0u, 0u, 0u, 0u};
  int bt[4] = {0, 0, 0, 0};
  const int lrow = tid >> 2, lch = (tid & 3) * 2;
  const int ntiles = ceil_div(nd, kDstTile);
  u32x4 pre[2];
  auto load_tile = [&](int t) {
    int d = t * kDstTile + lrow;
    d = d < nd ? d : 0;
    const u32x4* row = reinterpret_cast<const u32x4*>(X + (size_t)DL[d] * kD);
    pre[0] = row[lch];
    pre[1] = row[lch + 1];
  };
  load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        ss = sumsq8(__builtin_bit_cast(bf16x8, pre[c]), ss);
        sD[buf][lrow * 8 + ((lch + c) ^ swz(lrow))] = pre[c];
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      if ((tid & 3) == 0) sInv[buf][lrow] = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
    }
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);
    uint32_t tm[4];
    if ((t + 1) * kDstTile > nd)
      tile_keys<true>(sD[buf], sInv[buf], bs, off, lg, l16, nd - t * kDstTile, tm);
    else
      tile_keys<false>(sD[buf], sInv[buf], bs, off, lg, l16, kDstTile, tm);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t tT = tm[c] & ~15u;
      if (t == 0 || tT > bestT[c]) {
        best[c] = tm[c];
        bestT[c] = tT;
        bt[c] = t;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = 15 - (int)(best[c] & 15u);
    int d = bt[c] * kDstTile + (i >> 2) * 16 + 4 * lg + (i & 3);
    uint32_t kb = bestT[c];
    {
      const uint32_t ko = (uint32_t)__shfl_xor((int)kb, 16);
      const int dob = __shfl_xor(d, 16);
      take_better(kb, d, ko, dob);
    }
    {
      const uint32_t ko = (uint32_t)__shfl_xor((int)kb, 32);
      const int dob = __shfl_xor(d, 32);
      take_better(kb, d, ko, dob);
    }
    if (lg == 0 && ksrc[c] < ns) {
      const int dd = d < nd ? d : 0;
      const size_t o = hb + SL[ksrc[c]];
      const int ds = a.dst_slot[hb + dd];
      a.gdst[o] = DL[dd];
      a.gslot[o] = ds;
      a.gscore[o] = (__uint_as_float(kb) - off[c]) * invs[c] + 0.0f;
      atomicAdd(&a.cnt[(size_t)sh * a.bound + ds], 1);
    }
  }
}

// fp32 inputs: one thread per source, destinations through LDS, fp32 dots.
__global__ __launch_bounds__(256) void ga_match_f32(GaMatchArgs a) {
  __shared__ float sD[kDstTile][kD + 1];
  __shared__ float sInv[kDstTile];
  const int chunk = blockIdx.x % a.chunks, sh = blockIdx.x / a.chunks;
  const int st = sh / a.heads, head = sh % a.heads;
  const int nd = a.tot[sh * 3 + 1], ns = a.tot[sh * 3 + 2];
  if (chunk * kSrcPerWg >= ns || nd == 0) return;
  const size_t hb = (size_t)sh * a.N;
  const float* X = reinterpret_cast<const float*>(a.x[st]) + (size_t)head * a.N * kD;
  const int32_t* DL = a.dst_list + hb;
  const int tid = threadIdx.x;
  const int kidx = chunk * kSrcPerWg + tid;
  const int stok = a.src_list[hb + (kidx < ns ? kidx : 0)];
  float xs[kD];
  float ss = 0.f;
  for (int c = 0; c < kD; ++c) {
    xs[c] = X[(size_t)stok * kD + c];
    ss = fmaf(xs[c], xs[c], ss);
  }
  const float inv_src = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
  float bestv = -INFINITY;
  int bidx = 0;
  for (int t0 = 0; t0 < nd; t0 += kDstTile) {
    __syncthreads();
    for (int e = tid; e < kDstTile * kD; e += blockDim.x) {
      const int r = e / kD, c = e % kD;
      const int d = t0 + r < nd ? t0 + r : 0;
      sD[r][c] = X[(size_t)DL[d] * kD + c];
    }
    __syncthreads();
    if (tid < kDstTile) {
      float qn = 0.f;
      for (int c = 0; c < kD; ++c) qn = fmaf(sD[tid][c], sD[tid][c], qn);
      sInv[tid] = 1.0f / fmaxf(sqrtf(qn), 1e-12f);
    }
    __syncthreads();
    const int nt = min(kDstTile, nd - t0);
    for (int r = 0; r < nt; ++r) {
      float dot = 0.f;
      for (int c = 0; c < kD; ++c) dot = fmaf(xs[c], sD[r][c], dot);
      const float v = dot * sInv[r];
      if (v > bestv) {
        bestv = v;
        bidx = t0 + r;
      }
    }
  }
  if (kidx < ns) {
    const size_t o = hb + stok;
    const int ds = a.dst_slot[hb + bidx];
    a.gdst[o] = DL[bidx];
    a.gslot[o] = ds;
    a.gscore[o] = bestv * inv_src + 0.0f;
    atomicAdd(&a.cnt[(size_t)sh * a.bound + ds], 1);
  }
}

// Slot offsets of one (stream, head): exclusive prefix of the member counts
// over the anchors' slots, N for the empty slots past them and at `bound`.
// 256 threads x 16 slots per chunk.
constexpr int kOffPer = 16;
__global__ __launch_bounds__(kRoleThreads) void ga_offsets(const int32_t* __restrict__ cnt,
                                                            const int32_t* __restrict__ tot, int heads, int N,
                                                            int bound, int32_t* __restrict__ off_q,
                                                            int32_t* __restrict__ off_k) {
  __shared__ int wsum[kRoleThreads / 64];
  const int sh = blockIdx.x, st = sh / heads, head = sh % heads;
  const int ng = tot[sh * 3 + 0];
  const int32_t* c = cnt + (size_t)sh * bound;
  int32_t* o = (st == 0 ? off_q : off_k) + (size_t)head * (bound + 1);
  int carry = 0;
  for (int c0 = 0; c0 < bound; c0 += kRoleThreads * kOffPer) {
    const int s0 = c0 + threadIdx.x * kOffPer;
    int v[kOffPer], local = 0;
#pragma unroll
    for (int j = 0; j < kOffPer; ++j) {
      v[j] = s0 + j < ng ? c[s0 + j] : 0;
      local += v[j];
    }
    int total;
    int acc = carry + wg_excl_scan(local, wsum, total);
#pragma unroll
    for (int j = 0; j < kOffPer; ++j) {
      if (s0 + j < bound) o[s0 + j] = s0 + j < ng ? acc : N;
      acc += v[j];
    }
    carry += total;
  }
  if (threadIdx.x == 0) o[bound] = N;
}

// Every token into its slot's member range (position from an atomic
// counter: any order), and its slot in the token -> slot map.
__global__ __launch_bounds__(256) void ga_place(const uint8_t* __restrict__ role, const int32_t* __restrict__ slot,
                                                const int32_t* __restrict__ gslot, int heads, int N, int bound,
                                                const int32_t* __restrict__ off_q, const int32_t* __restrict__ off_k,
                                                int32_t* __restrict__ fill, int32_t* __restrict__ tmp,
                                                int32_t* __restrict__ grp_q, int32_t* __restrict__ grp_k) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)2 * heads * N) return;
  const int sh = (int)(i / N), tok = (int)(i - (int64_t)sh * N);
  const int st = sh / heads, head = sh % heads;
  const int s = role[i] == kRoleSrc ? gslot[i] : slot[i];
  const int32_t* o = (st == 0 ? off_q : off_k) + (size_t)head * (bound + 1);
  const int pos = o[s] + atomicAdd(&fill[(size_t)sh * bound + s], 1);
  if (pos < N) tmp[(size_t)sh * N + pos] = tok;  // always: the counts sum to N
  (st == 0 ? grp_q : grp_k)[(size_t)head * N + tok] = s;
}

// Members in ascending token order: the member at position p of its slot's
// range moves to range start + (members of the range with a smaller id).
__global__ __launch_bounds__(256) void ga_rank(const int32_t* __restrict__ tmp, int heads, int N, int bound,
                                               const int32_t* __restrict__ off_q, const int32_t* __restrict__ off_k,
                                               const int32_t* __restrict__ grp_q, const int32_t* __restrict__ grp_k,
                                               int32_t* __restrict__ mem_q, int32_t* __restrict__ mem_k) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)2 * heads * N) return;
  const int sh = (int)(i / N);
  const int st = sh / heads, head = sh % heads;
  const int32_t* T = tmp + (size_t)sh * N;
  const int tok = T[i - (int64_t)sh * N];
  const int s = (st == 0 ? grp_q : grp_k)[(size_t)head * N + tok];
  const int32_t* o = (st == 0 ? off_q : off_k) + (size_t)head * (bound + 1);
  const int a = o[s], b = o[s + 1];
  int rank = 0;
  for (int q = a; q < b; ++q) rank += T[q] < tok;
  if (a + rank < N) (st == 0 ? mem_q : mem_k)[(size_t)head * N + a + rank] = tok;
}

}  // namespace

hipError_t launch_ga_partition(int dtype, const GaShape& s, const void* q, const void* k, const GaBuffers& b,
                               hipStream_t stream) {
  const int HW = s.H * s.W;
  const int SH = 2 * s.heads;
  {
    const dim3 grid((unsigned)ceil_div(HW > s.nsp ? HW : s.nsp, 256), (unsigned)s.F, (unsigned)SH);
    HTTM_DISPATCH_T(dtype, hipLaunchKernelGGL(ga_variance<T>, grid, dim3(256), 0, stream, (const T*)q, (const T*)k,
                                              s.heads, s.N, s.Tf, s.nsp, s.H, s.W, b.var));
  }
  hipLaunchKernelGGL(ga_roles, dim3((unsigned)s.F, (unsigned)SH), dim3(kRoleThreads), 0, stream, b.var, s.heads, s.N,
                     s.Tf, s.nsp, s.H, s.W, s.F, s.k_protect, b.role, b.fcnt);
  hipLaunchKernelGGL(ga_scan, dim3((unsigned)SH), dim3(256), 0, stream, b.fcnt, s.F, s.heads, b.foff, b.tot, b.lenk);
  hipLaunchKernelGGL(ga_slots, dim3((unsigned)s.F, (unsigned)SH), dim3(kRoleThreads), 0, stream, b.role, s.heads, s.N,
                     s.Tf, s.F, s.bound, b.foff, b.slot, b.dst_list, b.dst_slot, b.src_list, b.gdst, b.gscore, b.cnt,
                     b.fill);
  GaMatchArgs a;
  a.x[0] = q;
  a.x[1] = k;
  a.heads = s.heads;
  a.N = s.N;
  a.chunks = ceil_div(s.max_src, kSrcPerWg);
  a.tot = b.tot;
  a.dst_list = b.dst_list;
  a.dst_slot = b.dst_slot;
  a.src_list = b.src_list;
  a.gdst = b.gdst;
  a.gslot = b.gslot;
  a.gscore = b.gscore;
  a.cnt = b.cnt;
  a.bound = s.bound;
  if (dtype == 1)
    hipLaunchKernelGGL(ga_match_bf16, dim3((unsigned)(SH * a.chunks)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(ga_match_f32, dim3((unsigned)(SH * a.chunks)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(ga_offsets, dim3((unsigned)SH), dim3(kRoleThreads), 0, stream, b.cnt, b.tot, s.heads, s.N,
                     s.bound, b.off_q, b.off_k);
  const unsigned grid = (unsigned)(((int64_t)SH * s.N + 255) / 256);
  hipLaunchKernelGGL(ga_place, dim3(grid), dim3(256), 0, stream, b.role, b.slot, b.gslot, s.heads, s.N, s.bound,
                     b.off_q, b.off_k, b.fill, b.tmp, b.grp_q, b.grp_k);
  hipLaunchKernelGGL(ga_rank, dim3(grid), dim3(256), 0, stream, b.tmp, s.heads, s.N, s.bound, b.off_q, b.off_k,
                     b.grp_q, b.grp_k, b.mem_q, b.mem_k);
  return hipGetLastError();
}

}  // namespace httm
