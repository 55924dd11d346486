// Measured-peak micro-benchmark: back-to-back bf16 MFMAs on every SIMD with
// no memory traffic in the loop.  A launch long enough to reach the card's
// steady clock under matrix load shows the MFMA rate this GPU sustains, the
// measured counterpart of the 2.5 PFLOP/s bf16 figure (which assumes
// 2.4 GHz): fractions of the attention and similarity kernels are reported
// against both.
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kPeakThreads = 256;
constexpr int kPeakChains = 8;  // independent accumulators per wave: the pipe never waits on a result

// Every lane's operands are a (8 x bf16) and b (8 x bf16); each
// v_mfma_f32_16x16x32_bf16 adds 32 a b to every accumulator element, so a
// thread ends with 8 chains x 4 elements x 32 a b x iters.
__global__ __launch_bounds__(kPeakThreads) void mfma_peak(int iters, float av, float bv, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)av;
    b[e] = (__bf16)bv;
  }
  f32x4 c[kPeakChains];
#pragma unroll
  for (int j = 0; j < kPeakChains; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kPeakChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
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
