// Ragged flash attention over the merged sequences.
//
// "HTTM: Head-wise Temporal Token Merging for Faster VGGT", overall framework
// and settings: attention runs on the shortened Q~ / K~ / V~ (bf16,
// FlashAttention on the page's A100).  Q~ is ragged per head because the
// outlier budget is shared across heads (key design 3); K~ / V~ have the same
// length in every head.
//
// One workgroup = 128 query rows of one head: 4 waves x 2 tiles of 16 rows,
// using v_mfma_f32_16x16x32_bf16 (the full-rate bf16 MFMA of gfx950).  Key
// tiles of 64 rows of K~ and the matching 64 columns of V~^T (stored
// transposed by the merge kernel) are copied global -> LDS directly
// (global_load_lds_dwordx4) into a double buffer.  S^T = K~ Q^T puts one query
// per lane column, so the running max enters the MFMA as its initial
// accumulator (acc = k.q - m, K~ pre-multiplied by scale * log2 e), the
// probabilities are exp2(acc), and the lane's probabilities are exactly the B
// operand of O^T = V~^T P^T.  Row max and row sum cross lanes with VALU lane
// swaps only; the sum adds the bf16-rounded probabilities (v_dot2) that the
// PV product uses.  The running max is raised only on the first tile or when
// a score exceeds it by more than 8 in log2 units, so accumulators are
// rescaled rarely; the final division makes the result exact.
// The (head, tile) of a workgroup comes from the per-head lengths on the
// device, so the host never waits for them.
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kKeyTile = 64;
constexpr int kRowsF32 = 128;  // fp32 kernel: one thread per query row

struct AttnArgs {
  const void* q;
  const void* k;
  const void* vt;
  void* o;
  const int32_t* lenq;
  int heads, lk, k_rows, vt_pitch, lq_uniform;
  int total_wg;
  float scale_log2;  // scale * log2(e), already applied to K~ by its producer
};

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_wave_base + 16*i (the base must be the same for the whole wave).
__device__ __forceinline__ void lds_copy16(const void* g, u32x4* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
// LDS tiles are rows of 128 bytes (eight 16-byte chunks); chunk c of row r is
// stored at chunk c ^ swz(r).  The LDS serves 256 bytes (64 four-byte banks)
// per cycle, i.e. 16 lanes of a 16-byte read: with this swizzle 16
// consecutive rows read at one logical chunk hit 16 distinct bank groups
// (rows of equal parity get distinct chunks, the two parities the two halves).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm_le() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ int xcd_logical(int bid, int total) {
  const int per = (total + 7) / 8;
  return (bid % 8) * per + bid / 8;
}

// (head, first packed row of the head, head length, tile) of workgroup w.
__device__ __forceinline__ bool locate(const AttnArgs& a, int w, int rows_per_wg, int& head, int& cu,
                                       int& L, int& tile) {
  int acc = 0;
  cu = 0;
  for (int h = 0; h < a.heads; ++h) {
    const int len = a.lenq ? a.lenq[h] : a.lq_uniform;
    const int nt = ceil_div(len, rows_per_wg);
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

__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Max over lanes {l, l^32} and {l, l^16} of a wave, with VALU lane swaps
// (no LDS round trip): after a swap of a register with itself, element 0
// holds one of the two lanes' values and element 1 the other.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16x16x32 form (full-rate bf16 MFMA on gfx950).  Per wave: QT query tiles of
// 16 rows.  S^T tile (16 keys x 16 queries): lane l holds query l%16 and keys
// 4*(l/16) + 0..3, so a lane's four scores share one query and the running
// max enters as the accumulator's initial value (acc = k.q - m).  PV chunk of
// 32 keys: lane's B operand holds keys 32*kc + 4g + {0..3} and
// 32*kc + 16 + 4g + {0..3} (g = l/16), exactly the probabilities it owns.
template <int QT, int NW>
__global__ __launch_bounds__(NW * 64) void attn16(AttnArgs a) {
  constexpr int kRowsPerWg = NW * QT * 16;
  __shared__ u32x4 sK[2][kKeyTile * 8];
  __shared__ u32x4 sV[2][kD * 8];
  const int w = xcd_logical(blockIdx.x, a.total_wg);
  int head, cu, L, tile;
  if (!locate(a, w, kRowsPerWg, head, cu, L, tile)) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const uint16_t* Qp = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* Kp = reinterpret_cast<const uint16_t*>(a.k) + (size_t)head * a.k_rows * kD;
  const uint16_t* Vp = reinterpret_cast<const uint16_t*>(a.vt) + (size_t)head * kD * a.vt_pitch;

  bf16x8 bq[QT][2];
  bool valid[QT];
  int qrow[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qr = tile * kRowsPerWg + (wave * QT + qt) * 16 + l16;
    valid[qt] = qr < L;
    qrow[qt] = qr;
    const size_t r = (size_t)cu + (valid[qt] ? qr : L - 1);
#pragma unroll
    for (int dc = 0; dc < 2; ++dc)
      bq[qt][dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Qp + r * kD + dc * 32 + g * 8));
  }
  f32x4 negm[QT];  // -running max, as the S accumulator's initial value
  float mrun[QT], lrun[QT];
  f32x4 oacc[QT][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = 0.f;
    lrun[qt] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) negm[qt][r] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[qt][dt][r] = 0.f;
  }

  const int ntiles = ceil_div(a.lk, kKeyTile);
  // Per-lane source of each copy round: row of the 64-row tile and the
  // logical 16-byte chunk that lands in this lane's LDS slot.
  int lrow[8 / NW], lchk[8 / NW];
#pragma unroll
  for (int rd = 0; rd < 8 / NW; ++rd) {
    const int p = (rd * NW + wave) * 64 + lane;
    lrow[rd] = p >> 3;
    lchk[rd] = (p & 7) ^ swz(p >> 3);
  }
  auto load_tile = [&](int t, int buf) {
#pragma unroll
    for (int rd = 0; rd < 8 / NW; ++rd) {
      int key = t * kKeyTile + lrow[rd];
      key = key < a.lk ? key : a.lk - 1;
      lds_copy16(Kp + (size_t)key * kD + lchk[rd] * 8, &sK[buf][(rd * NW + wave) * 64]);
      lds_copy16(Vp + (size_t)lrow[rd] * a.vt_pitch + t * kKeyTile + lchk[rd] * 8,
                 &sV[buf][(rd * NW + wave) * 64]);
    }
  };
  load_tile(0, 0);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    wait_vm_le<0>();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1, buf ^ 1);

    // S^T - m for 4 key tiles of 16
    f32x4 sacc[QT][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int arow = kt * 16 + l16;
#pragma unroll
      for (int dc = 0; dc < 2; ++dc) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, sK[buf][arow * 8 + ((4 * dc + g) ^ swz(arow))]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sacc[qt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[qt][dc], dc == 0 ? negm[qt] : sacc[qt][kt], 0, 0, 0);
      }
    }
    if ((t + 1) * kKeyTile > a.lk) {  // ragged key tail: only the last tile
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t * kKeyTile + kt * 16 + 4 * g + r >= a.lk) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) sacc[qt][kt][r] = -INFINITY;
          }
    }

    bf16x8 bp[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      // tree of max3 over the lane's 16 scores, then across the 4 lane rows
      const f32x4* sa = sacc[qt];
      const float m0 = max3(sa[0][0], sa[0][1], sa[0][2]), m1 = max3(sa[0][3], sa[1][0], sa[1][1]);
      const float m2 = max3(sa[1][2], sa[1][3], sa[2][0]), m3 = max3(sa[2][1], sa[2][2], sa[2][3]);
      const float m4 = max3(sa[3][0], sa[3][1], sa[3][2]);
      float mx = fmaxf(max3(m0, m1, m2), max3(m3, m4, sa[3][3]));
      mx = max_xor16(max_xor32(mx));
      // Raise the running max only on the first tile or when a score exceeds
      // it by more than 8 (log2 units); the final division makes it exact.
      const bool grow = (t == 0) || mx > 8.0f;
      if (__any(grow)) {
        float shift = 0.f;
        if (grow) {
          const float mnew = mrun[qt] + mx;
          shift = mx;
          mrun[qt] = mnew;
#pragma unroll
          for (int r = 0; r < 4; ++r) negm[qt][r] = -mnew;
        }
        if (t > 0) {
          const float alpha = __builtin_amdgcn_exp2f(-shift);
          lrun[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[qt][dt][r] *= alpha;
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[qt][kt][r] -= shift;
      }
      // probabilities (bf16) and their sum over the same rounded values,
      // in four independent partial sums
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
      float ls[4] = {lrun[qt], 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        bf16x8 pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pb[r] = (__bf16)__builtin_amdgcn_exp2f(sacc[qt][2 * kc][r]);
          pb[4 + r] = (__bf16)__builtin_amdgcn_exp2f(sacc[qt][2 * kc + 1][r]);
        }
        bp[qt][kc] = pb;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pb[e], pb[e + 1]};
          ls[e >> 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, ls[e >> 1], false);
        }
      }
      lrun[qt] = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int vrow = dt * 16 + l16;
        const u32x2* base = reinterpret_cast<const u32x2*>(&sV[buf][vrow * 8]);
        const int c0 = 4 * kc + (g >> 1), c1 = 4 * kc + 2 + (g >> 1);
        const u32x2 lo = base[2 * (c0 ^ swz(vrow)) + (g & 1)];
        const u32x2 hi = base[2 * (c1 ^ swz(vrow)) + (g & 1)];
        u32x4 va;
        va[0] = lo[0];
        va[1] = lo[1];
        va[2] = hi[0];
        va[3] = hi[1];
        const bf16x8 vb = __builtin_bit_cast(bf16x8, va);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, bp[qt][kc], oacc[qt][dt], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float inv = 1.0f / sum_xor16(sum_xor32(lrun[qt]));
    if (valid[qt]) {
      uint16_t* Op = reinterpret_cast<uint16_t*>(a.o) + ((size_t)cu + qrow[qt]) * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        u32x2 w2;
        w2[0] = (uint32_t)f2bf(oacc[qt][dt][0] * inv) | ((uint32_t)f2bf(oacc[qt][dt][1] * inv) << 16);
        w2[1] = (uint32_t)f2bf(oacc[qt][dt][2] * inv) | ((uint32_t)f2bf(oacc[qt][dt][3] * inv) << 16);
        *reinterpret_cast<u32x2*>(Op + dt * 16 + 4 * g) = w2;
      }
    }
  }
}

// fp32 inputs: one thread per query row, key tiles staged in LDS, fp32
// online softmax.  For fp32 layers (small correctness workloads).
__global__ __launch_bounds__(kRowsF32) void attn_f32(AttnArgs a) {
  __shared__ float sK[kKeyTile][kD + 1];
  __shared__ float sV[kD][kKeyTile + 1];
  int head, cu, L, tile;
  if (!locate(a, blockIdx.x, kRowsF32, head, cu, L, tile)) return;
  const float* Qp = reinterpret_cast<const float*>(a.q);
  const float* Kp = reinterpret_cast<const float*>(a.k) + (size_t)head * a.k_rows * kD;
  const float* Vp = reinterpret_cast<const float*>(a.vt) + (size_t)head * kD * a.vt_pitch;
  const int qr = tile * kRowsF32 + threadIdx.x;
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
      for (int c = 0; c < kD; ++c) s = fmaf(qv[c], sK[r][c], s);  // K~ carries scale*log2 e
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
  if (dtype == 1) {
    constexpr int kQT = 2, kNW = 4, kRows = kNW * kQT * 16;
    a.total_wg = (int)((s.q_capacity + kRows - 1) / kRows + s.heads);
    const int grid = ((a.total_wg + 7) / 8) * 8;
    hipLaunchKernelGGL((attn16<kQT, kNW>), dim3(grid), dim3(kNW * 64), 0, stream, a);
  } else {
    a.total_wg = (int)((s.q_capacity + kRowsF32 - 1) / kRowsF32 + s.heads);
    hipLaunchKernelGGL(attn_f32, dim3(a.total_wg), dim3(kRowsF32), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace httm
