// Measured-peak micro-benchmark: back-to-back bf16 MFMAs on every SIMD with
// no memory traffic in the loop.  Every lane holds 8 operand pairs of
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

}  // namespace

int peak_threads() { return kPeakThreads; }
double peak_flop_per_iter_wg() { return (double)(kPeakThreads / 64) * kPeakChains * (2.0 * 16 * 16 * 32); }

hipError_t launch_mfma_peak(int iters, int grid, float a, float b, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak, dim3(grid), dim3(kPeakThreads), 0, stream, iters, a, b, out);
  return hipGetLastError();
}

}  // namespace httm
