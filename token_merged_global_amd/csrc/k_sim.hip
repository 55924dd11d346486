// Per-head, block-local cosine similarity with a fused argmax epilogue.
//
// "HTTM: Head-wise Temporal Token Merging for Faster VGGT", key design 1:
// Sim = RowNorm(S) RowNorm(D)^T per head; every source keeps only its most
// similar destination.  Key design 2: matching runs only inside a merge block.
//
// For each (stream in {Q, K}, head, block, chunk of 256 sources) one workgroup
// of 4 waves streams the block's destination rows through LDS in tiles of 64
// and multiplies them against the 256 source rows held in registers, with
// v_mfma_f32_32x32x16_bf16 (exact bf16 products, fp32 accumulation).  The
// products are never pre-normalised to bf16: the destination's inverse norm
// (fp32) scales the fp32 dot product in the epilogue, the source's inverse
// norm scales only the final maximum (it does not change the argmax).
// Rows are gathered straight from the [h][N][64] input through the temporal
// reordering, so no reordered copy is ever written.
#include "common.h"
#include "kernels.h"

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

__device__ __forceinline__ void decode(const SimArgs& a, int w, int& st, int& head, int& b, int& chunk) {
  st = 0;
  if (w >= a.wgs[0]) { st = 1; w -= a.wgs[0]; }
  chunk = w % a.chunks[st];
  const int bh = w / a.chunks[st];
  b = bh % a.g.nblocks;
  head = bh / a.g.nblocks;
}

// Spread consecutive logical workgroups (chunks of one block) over one XCD:
// hardware hands workgroup ids to the 8 XCDs round-robin.
__device__ __forceinline__ int xcd_logical(int bid, int total) {
  const int per = (total + 7) / 8;
  return (bid % 8) * per + bid / 8;
}

__global__ __launch_bounds__(256) void sim_argmax_bf16(SimArgs a) {
  __shared__ u32x4 sD[2][kDstTile * 8];
  __shared__ __attribute__((aligned(16))) float sInv[2][kDstTile];
  const int w = xcd_logical(blockIdx.x, a.total);
  if (w >= a.total) return;
  int st, head, b, chunk;
  decode(a, w, st, head, b, chunk);
  const Geo& g = a.g;
  const BlockInfo bi = block_info(g, b, st);
  const int s = g.s[st];
  if (chunk * kSrcPerWg >= bi.ns) return;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x[st]) + (size_t)head * g.N * kD;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, l32 = lane & 31;

  // Source operands: lane holds src (wave*64 + c*32 + l32), channels q*16 + 8*hf .. +8.
  bf16x8 bs[2][4];
  float invs[2];
  int ksrc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int k = chunk * kSrcPerWg + wave * kSrcPerWave + c * 32 + l32;
    ksrc[c] = k;
    const int kk = k < bi.ns ? k : 0;
    const int tok = block_token(g, bi, src_pos(kk, s));
    const uint16_t* row = X + (size_t)tok * kD;
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(row + q * 16 + hf * 8);
      bs[c][q] = __builtin_bit_cast(bf16x8, u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(u[e] << 16), hi = __uint_as_float(u[e] & 0xFFFF0000u);
        ss += lo * lo;
        ss += hi * hi;
      }
    }
    ss += __shfl_xor(ss, 32);
    invs[c] = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
  }

  float best[2] = {-INFINITY, -INFINITY};
  int bidx[2] = {0x7fffffff, 0x7fffffff};

  // Tile loader: thread loads row tid/4 of the tile, 16-byte chunks 2*(tid%4) and +1.
  const int lrow = tid >> 2, lch = (tid & 3) * 2;
  const int ntiles = ceil_div(bi.nd, kDstTile);
  u32x4 pre[2];
  auto load_tile = [&](int t) {
    int d = t * kDstTile + lrow;
    d = d < bi.nd ? d : 0;
    const int tok = block_token(g, bi, d * s);
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
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(pre[c][e] << 16), hi = __uint_as_float(pre[c][e] & 0xFFFF0000u);
          ss += lo * lo;
          ss += hi * hi;
        }
        sD[buf][lrow * 8 + ((lch + c) ^ (lrow & 7))] = pre[c];
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      if ((tid & 3) == 0) sInv[buf][lrow] = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
    }
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x16 acc[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
      const int arow = rt * 32 + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 ua = sD[buf][arow * 8 + ((2 * q + hf) ^ (arow & 7))];
        const bf16x8 av = __builtin_bit_cast(bf16x8, ua);
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bs[c][q], acc[c], 0, 0, 0);
      }
      float inv[16];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(&sInv[buf][rt * 32 + 8 * gq + 4 * hf]);
#pragma unroll
        for (int j = 0; j < 4; ++j) inv[gq * 4 + j] = v4[j];
      }
      const int rbase = t * kDstTile + rt * 32 + 4 * hf;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = rbase + 8 * (i >> 2) + (i & 3);
          const float v = acc[c][i] * inv[i];
          if (v > best[c] && row < bi.nd) {
            best[c] = v;
            bidx[c] = row;
          }
        }
      }
    }
  }

#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const float ov = __shfl_xor(best[c], 32);
    const int oi = __shfl_xor(bidx[c], 32);
    if (ov > best[c] || (ov == best[c] && oi < bidx[c])) {
      best[c] = ov;
      bidx[c] = oi;
    }
    if (hf == 0 && ksrc[c] < bi.ns) {
      const size_t o = (size_t)head * g.nsrc[st] + bi.src0 + ksrc[c];
      a.match[st][o] = bidx[c] < bi.nd ? bidx[c] : 0;  // all-NaN rows: destination 0
      a.score[st][o] = best[c] * invs[c] + 0.0f;
    }
  }
}

// fp32 inputs: one thread per source, destinations staged through LDS, fp32
// FMA dot products.  Used for fp32 layers (small correctness workloads).
__global__ __launch_bounds__(256) void sim_argmax_f32(SimArgs a) {
  __shared__ float sD[kDstTile][kD + 1];
  __shared__ float sInv[kDstTile];
  const int w = blockIdx.x;
  if (w >= a.total) return;
  int st, head, b, chunk;
  decode(a, w, st, head, b, chunk);
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
                      float* score_q, int32_t* match_k, float* score_k, hipStream_t stream) {
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
    a.chunks[st] = mx > 0 ? ceil_div(mx, kSrcPerWg) : 1;
    a.wgs[st] = g.heads * g.nblocks * a.chunks[st];
  }
  a.total = a.wgs[0] + a.wgs[1];
  if (dtype == 1) {
    const int grid = ((a.total + 7) / 8) * 8;
    hipLaunchKernelGGL(sim_argmax_bf16, dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(sim_argmax_f32, dim3(a.total), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace httm
