// Cosine-argmax tile of 64 destinations against 64 sources per wave, shared
// by the block-local similarity kernel and the geometry-aware global match.
// Argmax keys: see the similarity kernel's header comment.
#pragma once
#include "common.h"

namespace httm {
namespace {

// 16-byte chunk c of LDS row r sits at chunk c ^ swz(r): the 16 consecutive
// rows one A-operand read touches land in distinct bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// max(a, b, c) on unsigned values as one v_max3_u32 (written out: from the
// plain form the compiler emitted two v_max_u32 for a quarter of the trees).
__device__ __forceinline__ uint32_t umax3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_max3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// acc + sum of squares of 8 bf16 values, two per v_dot2.
__device__ __forceinline__ float sumsq8(const bf16x8 x, float acc) {
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2 p = {x[e], x[e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}

// Order of (key without position bits, destination): larger key, then smaller destination.
__device__ __forceinline__ void take_better(uint32_t& kb, int& db, uint32_t ko, int dob) {
  if (ko > kb || (ko == kb && dob < db)) {
    kb = ko;
    db = dob;
  }
}

// Keys of destination block dt (16 rows of the tile) for the 4 source
// columns, folded into tm: key = score bits with the low 4 bits replaced by
// 15 - (position of the candidate among the lane's 16), so one unsigned max
// keeps the larger score and, on equal bits, the smaller destination.
template <bool MASK>
__device__ __forceinline__ void tile_keys16(const f32x4 (&acc)[4], const f32x4 inv4, const float (&off)[4], int dt,
                                          int lg, int nvalid, uint32_t (&tm)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t key[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = fmaf(acc[c][r], inv4[r], off[c]);
      key[r] = (__float_as_uint(v) & ~15u) | (uint32_t)(15 - (4 * dt + r));
      if (MASK && dt * 16 + 4 * lg + r >= nvalid) key[r] = 0u;
    }
    if (dt == 0) {
      tm[c] = umax3(key[0], key[1], key[2] > key[3] ? key[2] : key[3]);
    } else {
      tm[c] = umax3(tm[c], key[0], key[1]);
      tm[c] = umax3(tm[c], key[2], key[3]);
    }
  }
}

// One 64-destination tile: the 8 MFMAs of block dt + 1 are issued between
// the key updates of block dt, so matrix and vector work overlap in a wave.
template <bool MASK>
__device__ __forceinline__ void tile_argmax(const u32x4* sDb, const float* sInvb, const bf16x8 (&bs)[4][2],
                                        const float (&off)[4], int lg, int l16, int nvalid, uint32_t (&tm)[4]) {
  f32x4 acc[2][4];
  auto mfma_block = [&](int dt, f32x4 (&o)[4]) {
    const int arow = dt * 16 + l16;
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, sDb[arow * 8 + ((0 + lg) ^ swz(arow))]);
    const bf16x8 a1 = __builtin_bit_cast(bf16x8, sDb[arow * 8 + ((4 + lg) ^ swz(arow))]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bs[c][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      o[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bs[c][1], o[c], 0, 0, 0);
    }
  };
  mfma_block(0, acc[0]);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    if (dt + 1 < 4) mfma_block(dt + 1, acc[(dt + 1) & 1]);
    const f32x4 inv4 = *reinterpret_cast<const f32x4*>(&sInvb[dt * 16 + 4 * lg]);
    tile_keys16<MASK>(acc[dt & 1], inv4, off, dt, lg, nvalid, tm);
    if (dt + 1 < 4) {
      // 8 MFMAs spread over the 40 key instructions
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
  }
}

// Keys of one 64-destination tile, each MFMA pair followed by its keys:
// tm[c] = max over the lane's 16 candidates of source column tile c
// (position bits included).  MASK: only destinations below nvalid
// (tile-relative) count.  The block-local similarity uses this order: with
// its short per-block loops the interleaved tile above measured 11 % slower
// there (500 frames, both streams).
template <bool MASK>
__device__ __forceinline__ void tile_keys(const u32x4* sDb, const float* sInvb, const bf16x8 (&bs)[4][2],
                                          const float (&off)[4], int lg, int l16, int nvalid, uint32_t (&tm)[4]) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int arow = dt * 16 + l16;
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, sDb[arow * 8 + ((0 + lg) ^ swz(arow))]);
    const bf16x8 a1 = __builtin_bit_cast(bf16x8, sDb[arow * 8 + ((4 + lg) ^ swz(arow))]);
    const f32x4 inv4 = *reinterpret_cast<const f32x4*>(&sInvb[dt * 16 + 4 * lg]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bs[c][0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bs[c][1], acc, 0, 0, 0);
      uint32_t key[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = fmaf(acc[r], inv4[r], off[c]);
        key[r] = (__float_as_uint(v) & ~15u) | (uint32_t)(15 - (4 * dt + r));
        if (MASK && dt * 16 + 4 * lg + r >= nvalid) key[r] = 0u;
      }
      if (dt == 0) {
        tm[c] = umax3(key[0], key[1], key[2] > key[3] ? key[2] : key[3]);
      } else {
        tm[c] = umax3(tm[c], key[0], key[1]);
        tm[c] = umax3(tm[c], key[2], key[3]);
      }
    }
  }
}

}  // namespace
}  // namespace httm
