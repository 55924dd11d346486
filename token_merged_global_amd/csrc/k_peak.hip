// Measured-peak micro-benchmarks: back-to-back bf16 (or FP8) MFMAs on every
// SIMD with no memory traffic in the loop.  Every lane holds 8 operand pairs of
// pseudo-random bf16 values and consecutive MFMAs read different pairs, so
// the matrix units switch as they do on real data (with constant operands
// the same loop ran ~20 % faster, at a clock the card does not hold under
// real data).  A launch long enough to reach the card's steady clock shows
// the MFMA rate this GPU sustains: the measured counterpart of the
// 2.5 PFLOP/s bf16 figure, against which kernel fractions are also reported.
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kPeakThreads = 256;
constexpr int kPeakChains = 8;  // independent accumulators per wave: the pipe never waits on a result

// 32-bit integer hash (xorshift-multiply rounds), the operand source.
__device__ __forceinline__ uint32_t peak_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Lane g (global thread id), pair j, element e: h = peak_hash(64 g + 8 j + e);
// a_j[e] = bf16(a * ((h & 0xffff) - 32768) / 32768),
// b_j[e] = bf16(b * ((h >> 16) - 32768) / 32768).  Step ii of every group of
// 8 iterations multiplies a_j by b_((j + ii) mod 8) into chain j.
__global__ __launch_bounds__(kPeakThreads) void mfma_peak(int iters, float av, float bv, float* out) {
  const uint32_t g = blockIdx.x * kPeakThreads + threadIdx.x;
  bf16x8 a[kPeakChains], b[kPeakChains];
#pragma unroll
  for (int j = 0; j < kPeakChains; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = peak_hash(g * 64u + (uint32_t)(8 * j + e));
      a[j][e] = (__bf16)(av * ((float)(int)(h & 0xffffu) - 32768.0f) * (1.0f / 32768.0f));
      b[j][e] = (__bf16)(bv * ((float)(int)(h >> 16) - 32768.0f) * (1.0f / 32768.0f));
    }
  f32x4 c[kPeakChains];
#pragma unroll
  for (int j = 0; j < kPeakChains; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; i += 8) {
#pragma unroll
    for (int ii = 0; ii < 8; ++ii)
#pragma unroll
      for (int j = 0; j < kPeakChains; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[(j + ii) & 7], c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPeakChains; ++j) s += (c[j][0] + c[j][1]) + (c[j][2] + c[j][3]);
  out[(size_t)blockIdx.x * kPeakThreads + threadIdx.x] = s;
}

typedef int peak_i32x8 __attribute__((ext_vector_type(8)));
constexpr int kPeakChains8 = 4;  // FP8: 16-register accumulators, so 4 chains

// FP8 form: v_mfma_scale_f32_32x32x64_f8f6f4 on e4m3 operands with unit
// scales.  Lane g holds 4 pairs (A_j, B_j) of 32 bytes: dword w of A_j is
// peak_hash(128 g + 16 j + w) and of B_j peak_hash(128 g + 16 j + 8 + w), each
// byte with bit 6 cleared (exponent field below 8: magnitudes at most 1.875,
// no NaN code).  Step s of every group of 4 iterations accumulates A_j times
// B_((j + s) mod 4) into chain j.
__global__ __launch_bounds__(kPeakThreads) void mfma_peak_fp8(int iters, float* out) {
  const uint32_t g = blockIdx.x * kPeakThreads + threadIdx.x;
  peak_i32x8 a[kPeakChains8], b[kPeakChains8];
#pragma unroll
  for (int j = 0; j < kPeakChains8; ++j)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      a[j][w] = (int)(peak_hash(g * 128u + (uint32_t)(16 * j + w)) & 0xBFBFBFBFu);
      b[j][w] = (int)(peak_hash(g * 128u + (uint32_t)(16 * j + 8 + w)) & 0xBFBFBFBFu);
    }
  f32x16 c[kPeakChains8];
#pragma unroll
  for (int j = 0; j < kPeakChains8; ++j) c[j] = f32x16{};
  for (int i = 0; i < iters; i += kPeakChains8) {
#pragma unroll
    for (int ii = 0; ii < kPeakChains8; ++ii)
#pragma unroll
      for (int j = 0; j < kPeakChains8; ++j)
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j], b[(j + ii) & 3], c[j], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPeakChains8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  out[(size_t)blockIdx.x * kPeakThreads + threadIdx.x] = s;
}

}  // namespace

double peak_flop_per_iter_wg_fp8() { return (double)(kPeakThreads / 64) * kPeakChains8 * (2.0 * 32 * 32 * 64); }

hipError_t launch_mfma_peak_fp8(int iters, int grid, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak_fp8, dim3(grid), dim3(kPeakThreads), 0, stream, iters, out);
  return hipGetLastError();
}

int peak_threads() { return kPeakThreads; }
double peak_flop_per_iter_wg() { return (double)(kPeakThreads / 64) * kPeakChains * (2.0 * 16 * 16 * 32); }

hipError_t launch_mfma_peak(int iters, int grid, float a, float b, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak, dim3(grid), dim3(kPeakThreads), 0, stream, iters, a, b, out);
  return hipGetLastError();
}

}  // namespace httm
