// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geo.h"

// Runs the statement with T = uint16_t (bf16 bits, dtype 1) or T = float.
#define HTTM_DISPATCH(dtype, ...) \
  do {                            \
    if ((dtype) == 1) {           \
      typedef uint16_t T;         \
      __VA_ARGS__;                \
    } else {                      \
      typedef float T;            \
      __VA_ARGS__;                \
    }                             \
  } while (0)

namespace httm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 8 consecutive channels of a row as fp32, from fp32 or bf16 storage.
template <typename T>
struct Row8;

template <>
struct Row8<float> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = x[i]; b[i] = x[4 + i]; }
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
  }
};

template <>
struct Row8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(a[i] << 16);
      x[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* x) {
    u32x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = (uint32_t)f2bf(x[2 * i]) | ((uint32_t)f2bf(x[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4*>(p) = a;
  }
};

// Orderable key of a float: unsigned order equals float order (-0 < +0 is
// avoided by callers, who add +0.0f first).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Prefix sums over per-head lengths with one head per lane of the calling
// wave (heads <= 64; every lane of the wave calls it with the same
// arguments): one load per lane and shuffle scans instead of a serial walk.
// Lane h gets its head's length and the rows and tiles (tiles of tile_rows
// rows, 0: none) of heads 0..h-1 and 0..h; totals in every lane.
struct HeadPrefix {
  int len, rows_before, tiles_before, tiles_upto, rows_total, tiles_total;
};
__device__ __forceinline__ HeadPrefix head_prefix(const int32_t* lenq, int lq_uniform, int heads, int tile_rows) {
  const int lane = threadIdx.x & 63;
  HeadPrefix p;
  p.len = lane < heads ? (lenq ? lenq[lane] : lq_uniform) : 0;
  const int t = tile_rows > 0 ? ceil_div(p.len, tile_rows) : 0;
  int r = p.len, u = t;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int r2 = __shfl_up(r, d), u2 = __shfl_up(u, d);
    if (lane >= d) {
      r += r2;
      u += u2;
    }
  }
  p.rows_before = r - p.len;
  p.tiles_before = u - t;
  p.tiles_upto = u;
  p.rows_total = __shfl(r, 63);
  p.tiles_total = __shfl(u, 63);
  return p;
}

}  // namespace httm
