// Ragged flash attention over the merged sequences.
//
// "HTTM: Head-wise Temporal Token Merging for Faster VGGT", overall framework
// and settings: attention runs on the shortened Q~ / K~ / V~ (bf16,
// FlashAttention on the page's A100).  Q~ is ragged per head because the
// outlier budget is shared across heads (key design 3); K~ / V~ have the same
// length in every head.
//
// One workgroup = 128 query rows of one head (4 waves x 32 rows).  Key tiles
// of 64 rows of K~ and the matching 64 columns of V~^T (stored transposed by
// the merge kernel) are double-buffered in LDS.  Each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so a lane owns one query row
// (32 lanes x 2 halves), keeps that row's running max and sum in registers
// (online softmax, exp2 with log2(e) folded into the scale), and feeds its
// probabilities straight back as the B operand of O^T = V^T P^T: the key
// order of P's registers and of the V^T operand agree, so no cross-lane
// shuffle is needed apart from one max exchange between the two halves.
// The (head, tile) of a workgroup comes from the per-head lengths on the
// device, so the host never waits for them.
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kRowsPerWg = 128;
constexpr int kKeyTile = 64;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* vt;
  void* o;
  const int32_t* lenq;
  int heads, lk, k_rows, vt_pitch, lq_uniform;
  int total_wg;
  float scale_log2;  // scale * log2(e)
};

__device__ __forceinline__ int xcd_logical(int bid, int total) {
  const int per = (total + 7) / 8;
  return (bid % 8) * per + bid / 8;
}

// (head, first packed row of the head, head length, tile) of workgroup w.
__device__ __forceinline__ bool locate(const AttnArgs& a, int w, int& head, int& cu, int& L,
                                       int& tile) {
  int acc = 0;
  cu = 0;
  for (int h = 0; h < a.heads; ++h) {
    const int len = a.lenq ? a.lenq[h] : a.lq_uniform;
    const int nt = ceil_div(len, kRowsPerWg);
    if (w < acc + nt) {
      head = h;
      L = len;
      tile = w - acc;
      return true;
    }
    acc += nt;
    cu += len;
  }
  return false;
}

__global__ __launch_bounds__(256) void attn_bf16(AttnArgs a) {
  __shared__ u32x4 sK[2][kKeyTile * 8];
  __shared__ u32x4 sV[2][kD * 8];
  const int w = xcd_logical(blockIdx.x, a.total_wg);
  int head, cu, L, tile;
  if (!locate(a, w, head, cu, L, tile)) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int hf = lane >> 5, l32 = lane & 31;
  const uint16_t* Qp = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* Kp = reinterpret_cast<const uint16_t*>(a.k) + (size_t)head * a.k_rows * kD;
  const uint16_t* Vp = reinterpret_cast<const uint16_t*>(a.vt) + (size_t)head * kD * a.vt_pitch;

  const int qr = tile * kRowsPerWg + wave * 32 + l32;
  const bool valid = qr < L;
  const size_t qrow = (size_t)cu + (valid ? qr : L - 1);
  bf16x8 bq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    bq[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Qp + qrow * kD + c * 16 + hf * 8));

  f32x16 oacc[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  const int lrow = tid >> 2, lch = (tid & 3) * 2;
  const int ntiles = ceil_div(a.lk, kKeyTile);
  u32x4 pk[2], pv[2];
  auto load_tile = [&](int t) {
    int key = t * kKeyTile + lrow;
    key = key < a.lk ? key : a.lk - 1;
    const u32x4* kr = reinterpret_cast<const u32x4*>(Kp + (size_t)key * kD);
    pk[0] = kr[lch];
    pk[1] = kr[lch + 1];
    const u32x4* vr = reinterpret_cast<const u32x4*>(Vp + (size_t)lrow * a.vt_pitch + t * kKeyTile);
    pv[0] = vr[lch];
    pv[1] = vr[lch + 1];
  };
  load_tile(0);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      sK[buf][lrow * 8 + ((lch + c) ^ (lrow & 7))] = pk[c];
      sV[buf][lrow * 8 + ((lch + c) ^ (lrow & 7))] = pv[c];
    }
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    // S^T = K Q^T for two 32-key tiles
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kt][i] = 0.f;
      const int arow = kt * 32 + l32;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, sK[buf][arow * 8 + ((2 * c + hf) ^ (arow & 7))]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bq[c], sacc[kt], 0, 0, 0);
      }
    }
    // scale, mask the ragged key tail, running max
    const int kbase = t * kKeyTile + 4 * hf;
    float mt = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + kt * 32 + 8 * (i >> 2) + (i & 3);
        const float x = key < a.lk ? sacc[kt][i] * a.scale_log2 : -INFINITY;
        sacc[kt][i] = x;
        mt = fmaxf(mt, x);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mnew = fmaxf(mrun, mt);
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    mrun = mnew;
    lrun *= alpha;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(sacc[kt][i] - mnew);
        sacc[kt][i] = p;
        lrun += p;
      }
    // O^T += V^T P^T: 4 MFMAs of 16 keys; lane's keys for MFMA j are
    // kt*32 + 16*(j%2) + 4*hf + {0..3, 8..11} with kt = j/2.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kt = j >> 1, i0 = 8 * (j & 1);
      bf16x8 bp;
#pragma unroll
      for (int e = 0; e < 8; ++e) bp[e] = (__bf16)sacc[kt][i0 + e];
      const int ch0 = 4 * kt + 2 * (j & 1);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const int vrow = dt * 32 + l32;
        const u32x2* base = reinterpret_cast<const u32x2*>(&sV[buf][vrow * 8]);
        const u32x2 lo = base[2 * (ch0 ^ (vrow & 7)) + hf];
        const u32x2 hi = base[2 * ((ch0 + 1) ^ (vrow & 7)) + hf];
        u32x4 va;
        va[0] = lo[0];
        va[1] = lo[1];
        va[2] = hi[0];
        va[3] = hi[1];
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), bp, oacc[dt], 0, 0, 0);
      }
    }
  }

  lrun += __shfl_xor(lrun, 32);
  const float inv = 1.0f / lrun;
  if (valid) {
    uint16_t* Op = reinterpret_cast<uint16_t*>(a.o) + ((size_t)cu + qr) * kD;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 w2;
        const int i = gq * 4;
        w2[0] = (uint32_t)f2bf(oacc[dt][i] * inv) | ((uint32_t)f2bf(oacc[dt][i + 1] * inv) << 16);
        w2[1] = (uint32_t)f2bf(oacc[dt][i + 2] * inv) | ((uint32_t)f2bf(oacc[dt][i + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(Op + dt * 32 + 8 * gq + 4 * hf) = w2;
      }
  }
}

// fp32 inputs: one thread per query row, key tiles staged in LDS, fp32
// online softmax.  For fp32 layers (small correctness workloads).
__global__ __launch_bounds__(128) void attn_f32(AttnArgs a) {
  __shared__ float sK[kKeyTile][kD + 1];
  __shared__ float sV[kD][kKeyTile + 1];
  int head, cu, L, tile;
  if (!locate(a, blockIdx.x, head, cu, L, tile)) return;
  const float* Qp = reinterpret_cast<const float*>(a.q);
  const float* Kp = reinterpret_cast<const float*>(a.k) + (size_t)head * a.k_rows * kD;
  const float* Vp = reinterpret_cast<const float*>(a.vt) + (size_t)head * kD * a.vt_pitch;
  const int qr = tile * kRowsPerWg + threadIdx.x;
  const bool valid = qr < L;
  const size_t qrow = (size_t)cu + (valid ? qr : L - 1);
  float qv[kD], acc[kD];
  for (int c = 0; c < kD; ++c) {
    qv[c] = Qp[qrow * kD + c];
    acc[c] = 0.f;
  }
  float mrun = -INFINITY, lrun = 0.f;
  for (int t0 = 0; t0 < a.lk; t0 += kKeyTile) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKeyTile * kD; e += blockDim.x) {
      const int r = e / kD, c = e % kD;
      const int key = t0 + r < a.lk ? t0 + r : a.lk - 1;
      sK[r][c] = Kp[(size_t)key * kD + c];
      sV[e / kKeyTile][e % kKeyTile] = Vp[(size_t)(e / kKeyTile) * a.vt_pitch + t0 + e % kKeyTile];
    }
    __syncthreads();
    const int nt = min(kKeyTile, a.lk - t0);
    for (int r = 0; r < nt; ++r) {
      float s = 0.f;
      for (int c = 0; c < kD; ++c) s = fmaf(qv[c], sK[r][c], s);
      s *= a.scale_log2;
      const float mnew = fmaxf(mrun, s);
      const float alpha = exp2f(mrun - mnew);
      const float p = exp2f(s - mnew);
      lrun = lrun * alpha + p;
      for (int c = 0; c < kD; ++c) acc[c] = fmaf(acc[c], alpha, p * sV[c][r]);
      mrun = mnew;
    }
  }
  if (valid) {
    float* Op = reinterpret_cast<float*>(a.o) + ((size_t)cu + qr) * kD;
    for (int c = 0; c < kD; ++c) Op[c] = acc[c] / lrun;
  }
}

}  // namespace

hipError_t launch_attention(int dtype, const AttnShape& s, const void* q, const void* k,
                            const void* vt, const int32_t* lenq, void* o, hipStream_t stream) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.vt = vt;
  a.o = o;
  a.lenq = lenq;
  a.heads = s.heads;
  a.lk = s.lk;
  a.k_rows = s.k_rows;
  a.vt_pitch = s.vt_pitch;
  a.lq_uniform = s.lq_uniform;
  a.scale_log2 = s.scale * 1.4426950408889634f;
  // tiles over all heads <= capacity / 128 + heads
  const int64_t cap_tiles = (s.q_capacity + kRowsPerWg - 1) / kRowsPerWg + s.heads;
  a.total_wg = (int)cap_tiles;
  if (dtype == 1) {
    const int grid = ((a.total_wg + 7) / 8) * 8;
    hipLaunchKernelGGL(attn_bf16, dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_f32, dim3(a.total_wg), dim3(kRowsPerWg), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace httm
