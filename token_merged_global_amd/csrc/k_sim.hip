// Per-head, block-local cosine similarity with a fused argmax epilogue.
//
// "HTTM: Head-wise Temporal Token Merging for Faster VGGT", key design 1:
// Sim = RowNorm(S) RowNorm(D)^T per head; every source keeps only its most
// similar destination.  Key design 2: matching runs only inside a merge block.
//
// For each (stream in {Q, K}, head, block, chunk of 256 sources) one workgroup
// of 4 waves streams the block's destination rows through LDS in tiles of 64
// and multiplies them against the 64 source rows each wave holds in registers,
// with v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 accumulation).
// Rows are gathered straight from the [h][N][64] input through the temporal
// reordering, so no reordered copy is ever written.
//
// Argmax epilogue.  Lane (g, l16) of a 16x16 output tile holds destinations
// 4g..4g+3 of source column l16, so per 64-destination tile a lane sees 16
// candidates of each of its 4 source columns, in ascending destination order.
// Each candidate becomes v = dot * inv|d| + |s| (1 + 2^-10) with one FMA: the
// offset makes every v positive, so its bit pattern orders like its value.
// The low 4 bits of the pattern are replaced by 15 - (candidate position), and
// one unsigned max3 tree then yields the maximum and its first position at
// once (2.5 VALU ops per score).  The replaced bits bound the error of the
// decision and of the reported cosine by 16 ulp of v (< 4e-6 for |v| < 4|s|):
// candidates closer than that are near-ties.  Tiles are compared without the
// position bits, so an earlier tile keeps a tie; the 4 lanes of a source are
// combined last, ties going to the smaller destination.
#include "common.h"
#include "kernels.h"
#include "sim_tile.h"

namespace httm {

namespace {

constexpr int kSrcPerWave = 64;
constexpr int kSrcPerWg = 256;
constexpr int kDstTile = 64;

struct SimArgs {
  Geo g;
  const void* x[2];
  int32_t* match[2];
  float* score[2];
  int32_t chunks[2];
  int32_t wgs[2];  // workgroups per stream
  int32_t total;
};

// Workgroup -> (stream, head, block, source chunk).  The hardware hands
// workgroup ids to the 8 XCDs round-robin; XCD x = id % 8 takes the
// (head, block) pairs [x*HB/8, (x+1)*HB/8) with both streams, the longer
// K-stream chunks first, so every XCD gets an equal share of the work and the
// chunks of one block (which read the same destination rows) share its L2.
__device__ __forceinline__ bool decode(const SimArgs& a, int bid, int& st, int& head, int& b, int& chunk) {
  const int hb_total = a.g.heads * a.g.nblocks;
  const int x = bid & 7, j = bid >> 3;
  const int hb0 = (int)((int64_t)x * hb_total / 8), hb1 = (int)((int64_t)(x + 1) * hb_total / 8);
  const int nk = (hb1 - hb0) * a.chunks[1];
  int hb;
  if (j < nk) {
    st = 1;
    hb = hb0 + j / a.chunks[1];
    chunk = j % a.chunks[1];
  } else {
    const int jq = j - nk;
    if (jq >= (hb1 - hb0) * a.chunks[0]) return false;
    st = 0;
    hb = hb0 + jq / a.chunks[0];
    chunk = jq % a.chunks[0];
  }
  b = hb % a.g.nblocks;
  head = hb / a.g.nblocks;
  return true;
}

__global__ __launch_bounds__(256) void sim_argmax_bf16(SimArgs a) {
  __shared__ u32x4 sD[2][kDstTile * 8];
  __shared__ __attribute__((aligned(16))) float sInv[2][kDstTile];
  int st, head, b, chunk;
  if (!decode(a, blockIdx.x, st, head, b, chunk)) return;
  const Geo& g = a.g;
  const BlockInfo bi = block_info(g, b, st);
  const int s = g.s[st];
  if (chunk * kSrcPerWg >= bi.ns) return;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x[st]) + (size_t)head * g.N * kD;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lg = lane >> 4, l16 = lane & 15;
  const float rcp_run = div_rcp(block_divisor(g, bi)), rcp_s1 = div_rcp(s - 1);

  // Source operands: column tile c holds source chunk*256 + wave*64 + 16c + l16,
  // channels 32kc + 8lg .. +8 for k-chunk kc.
  bf16x8 bs[4][2];
  float off[4], invs[4];
  int ksrc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int k = chunk * kSrcPerWg + wave * kSrcPerWave + c * 16 + l16;
    ksrc[c] = k;
    const int kk = k < bi.ns ? k : 0;
    const int pos = kk + div_small(kk, rcp_s1) + 1;  // src_pos(kk, s)
    const int tok = block_token_r(g, bi, pos, rcp_run);
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
    // hardware sqrt / rsq (1 ulp): the offset only has to exceed |s| dot d^,
    // which its 2^-10 margin guarantees
    off[c] = __builtin_amdgcn_sqrtf(ss) * (1.0f + 0x1p-10f);
    invs[c] = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
  }

  uint32_t best[4] = {0u, 0u, 0u, 0u}, bestT[4] = {0u, 0u, 0u, 0u};
  int bt[4] = {0, 0, 0, 0};

  // Tile loader: thread loads row tid/4 of the tile, 16-byte chunks 2*(tid%4) and +1.
  const int lrow = tid >> 2, lch = (tid & 3) * 2;
  const int ntiles = ceil_div(bi.nd, kDstTile);
  u32x4 pre[2];
  auto load_tile = [&](int t) {
    int d = t * kDstTile + lrow;
    d = d < bi.nd ? d : 0;
    const int tok = block_token_r(g, bi, d * s, rcp_run);
    const u32x4* row = reinterpret_cast<const u32x4*>(X + (size_t)tok * kD);
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
    // destination rows past nd (last tile only) must not win: their keys are 0
    if ((t + 1) * kDstTile > bi.nd)
      tile_keys<true>(sD[buf], sInv[buf], bs, off, lg, l16, bi.nd - t * kDstTile, tm);
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
    if (lg == 0 && ksrc[c] < bi.ns) {
      const size_t o = (size_t)head * g.nsrc[st] + bi.src0 + ksrc[c];
      a.match[st][o] = d < bi.nd ? d : 0;
      a.score[st][o] = (__uint_as_float(kb) - off[c]) * invs[c] + 0.0f;
    }
  }
}

// fp32 inputs: one thread per source, destinations staged through LDS, fp32
// FMA dot products.  Used for fp32 layers (small correctness workloads).
__global__ __launch_bounds__(256) void sim_argmax_f32(SimArgs a) {
  __shared__ float sD[kDstTile][kD + 1];
  __shared__ float sInv[kDstTile];
  int st, head, b, chunk;
  if (!decode(a, blockIdx.x, st, head, b, chunk)) return;
  const Geo& g = a.g;
  const BlockInfo bi = block_info(g, b, st);
  const int s = g.s[st];
  if (chunk * kSrcPerWg >= bi.ns) return;
  const float* X = reinterpret_cast<const float*>(a.x[st]) + (size_t)head * g.N * kD;
  const int tid = threadIdx.x;
  const int k = chunk * kSrcPerWg + tid;
  const int kk = k < bi.ns ? k : 0;
  float xs[kD];
  const float* srow = X + (size_t)block_token(g, bi, src_pos(kk, s)) * kD;
  float ss = 0.f;
  for (int c = 0; c < kD; ++c) {
    xs[c] = srow[c];
    ss = fmaf(xs[c], xs[c], ss);
  }
  const float inv_src = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  for (int t0 = 0; t0 < bi.nd; t0 += kDstTile) {
    __syncthreads();
    for (int e = tid; e < kDstTile * kD; e += blockDim.x) {
      const int r = e / kD, c = e % kD;
      const int d = t0 + r < bi.nd ? t0 + r : 0;
      sD[r][c] = X[(size_t)block_token(g, bi, d * s) * kD + c];
    }
    __syncthreads();
    if (tid < kDstTile) {
      float q = 0.f;
      for (int c = 0; c < kD; ++c) q = fmaf(sD[tid][c], sD[tid][c], q);
      sInv[tid] = 1.0f / fmaxf(sqrtf(q), 1e-12f);
    }
    __syncthreads();
    const int nt = min(kDstTile, bi.nd - t0);
    for (int r = 0; r < nt; ++r) {
      float dot = 0.f;
      for (int c = 0; c < kD; ++c) dot = fmaf(xs[c], sD[r][c], dot);
      const float v = dot * sInv[r];
      if (v > best) {
        best = v;
        bidx = t0 + r;
      }
    }
  }
  if (k < bi.ns) {
    const size_t o = (size_t)head * g.nsrc[st] + bi.src0 + k;
    a.match[st][o] = bidx < bi.nd ? bidx : 0;
    a.score[st][o] = best * inv_src + 0.0f;
  }
}

}  // namespace

hipError_t launch_sim(const Geo& g, int dtype, const void* q, const void* k, int32_t* match_q,
                      float* score_q, int32_t* match_k, float* score_k, int streams, hipStream_t stream) {
  SimArgs a;
  a.g = g;
  a.x[0] = q;
  a.x[1] = k;
  a.match[0] = match_q;
  a.match[1] = match_k;
  a.score[0] = score_q;
  a.score[1] = score_k;
  // largest source count of any block shape
  for (int st = 0; st < 2; ++st) {
    int mx = 0;
    for (int b = 0; b < g.nblocks; ++b) {
      const BlockInfo bi = block_info(g, b, st);
      mx = bi.ns > mx ? bi.ns : mx;
    }
    a.chunks[st] = ((streams >> st) & 1) ? (mx > 0 ? ceil_div(mx, kSrcPerWg) : 1) : 0;
    a.wgs[st] = g.heads * g.nblocks * a.chunks[st];
  }
  if (a.chunks[0] + a.chunks[1] == 0) return hipSuccess;
  a.total = a.wgs[0] + a.wgs[1];
  // 8 XCD slices of ceil(HB/8) (head, block) pairs at most
  const int hb = g.heads * g.nblocks;
  const int per_xcd = ceil_div(hb, 8) * (a.chunks[0] + a.chunks[1]);
  const int grid = 8 * per_xcd;
  if (dtype == 1) {
    hipLaunchKernelGGL(sim_argmax_bf16, dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(sim_argmax_f32, dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace httm
