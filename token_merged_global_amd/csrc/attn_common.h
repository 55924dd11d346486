// Pieces shared by the bf16 and FP8 attention kernels: the work-unit
// schedule (query tiles dealt to the XCDs, key splits, tail tiles), the
// partial-row layout of key splits, direct-to-LDS copies and lane swaps, and
// the store of a unit's rows.  Included by one kernel file each; everything
// has internal linkage.
#pragma once
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kKeyTile = 64;
constexpr int kRowsF32 = 128;  // fp32 kernel: one thread per query row
constexpr int kQT = 4;         // 16-row query tiles per wave
constexpr int kNW = 4;         // waves per workgroup
constexpr int kRows = kQT * kNW * 16;
constexpr float kTinySum = 8.673617379884035e-19f;  // 2^-60

struct AttnArgs {
  const void* q;
  const void* k;
  const void* vt;
  void* o;                 // normalized output rows (split == 1)
  float* opart;            // [split][q_capacity][64] partial numerators (split > 1)
  float* lpart;            // [split][q_capacity] partial row sums
  float* mpart;            // [split][q_capacity] reference of each partial
  const float* kmax;       // [heads] max |k~|
  const int32_t* lenk;     // [heads] keys per head when they vary (nullable: lk)
  int* fb_count;           // queued units for the exact kernel
  int* fb_list;
  const int32_t* lenq;
  int heads, lk, k_rows, vt_pitch, lq_uniform;
  int split;
  int tail_split;          // splits of an XCD's tail tiles (== split: no tail)
  int per_round;           // query tiles per full round of one XCD (split-S workgroups)
  int64_t q_capacity;
  int64_t tail_rows;       // partial rows reserved for splits >= split of tail tiles
  int total_wg;
  // FP8 scores only
  const uint8_t* k8;       // [heads][k_rows][64] e4m3 keys, scaled by 2^kexp[h]
  const int32_t* kexp;     // [heads] key scale exponents
  uint8_t* q8;             // [q_capacity][64] e4m3 queries as quantised (written by split 0; nullable)
  int32_t* qexp;           // [q_capacity] their scale exponents (nullable)
};

// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_wave_base + 16*i (the base must be the same for the whole wave).
__device__ __forceinline__ void lds_copy16(const void* g, u32x4* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
// The same through a buffer resource: a fixed per-lane byte offset voff and
// a wave-uniform soff (scalar register), so that advancing to the next tile
// costs no vector instruction.  Reads past the resource's `bytes` return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// A pointer every lane holds, as a wave-uniform (scalar) value.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void lds_copy16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                               u32x4* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff,
                                           soff, 0, 0);
}
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Two probabilities as one bf16 pair, each truncated to bf16 (its upper 16
// bits), in one v_perm_b32 instead of a rounding v_cvt_pk_bf16_f32.  The row
// sum adds the same truncated values, so the common part of their downward
// bias cancels in the normalisation and what remains spreads like rounding
// error (uniform over half an ulp either side).  Used by the FP8-score kernel,
// where it is faster; in the bf16 kernel's schedule it measured slower.
__device__ __forceinline__ uint32_t pack_bf16_trunc(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// LDS tiles are rows of 128 bytes (eight 16-byte chunks); chunk c of row r is
// stored at chunk c ^ swz(r).  The LDS serves 16 lanes of a 16-byte read per
// cycle (64 four-byte banks).  V~^T is read by 16 consecutive rows: swzV
// gives rows of equal parity distinct chunks.  K~ is read by the permuted
// rows 8(i/4) + 4p + i%4 of a 32-key chunk: swzK does the same for them.
__device__ __forceinline__ int swzV(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swzK(int row) { return ((row >> 1) & 1) | ((row >> 2) & 6); }

// Sums over lanes {l, l^32} and {l, l^16} with VALU lane swaps.
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

struct Unit {
  int head, cu, L, tile, split;
  int nsplit;  // key splits of this query tile
  int tord;    // slot among the tail tiles (-1: regular tile)
};

// Tail tiles per XCD at most (partial rows are reserved for this many).
constexpr int kMaxTailTiles = 16;

// The XCD share of U query tiles: tiles [u0, u0 + n), the first nr regular
// (split splits), the rest tail tiles (tail_split splits).
struct XcdShare {
  int u0, n, nr;
};
__device__ __forceinline__ XcdShare xcd_share(const AttnArgs& a, int U, int x) {
  XcdShare r;
  r.u0 = (int)((int64_t)x * U / 8);
  r.n = (int)((int64_t)(x + 1) * U / 8) - r.u0;
  const int t = a.per_round > 0 ? r.n % a.per_round : 0;
  r.nr = r.n - t;
  return r;
}

// Workgroup id -> unit (see Schedule above); false for workgroups past the
// work.  Every lane of the wave takes part (wave-wide scans over the heads).
__device__ __forceinline__ bool schedule(const AttnArgs& a, int bid, Unit& o) {
  const HeadPrefix hp = head_prefix(a.lenq, a.lq_uniform, a.heads, kRows);
  const int U = hp.tiles_total;
  const int x = bid & 7, j = bid >> 3;
  const XcdShare sh = xcd_share(a, U, x);
  int ug;
  if (j < a.split * sh.nr) {
    o.split = j / sh.nr;
    ug = sh.u0 + j % sh.nr;
    o.nsplit = a.split;
    o.tord = -1;
  } else {
    const int t = sh.n - sh.nr, jt = j - a.split * sh.nr;
    if (jt >= a.tail_split * t) return false;
    o.split = jt / t;
    o.tord = x * kMaxTailTiles + jt % t;
    ug = sh.u0 + sh.nr + jt % t;
    o.nsplit = a.tail_split;
  }
  // the head holding tile ug: heads whose tiles all lie below ug come first
  const int lane = threadIdx.x & 63;
  const int h = __popcll(__ballot(lane < a.heads && hp.tiles_upto <= ug));
  o.head = h;
  o.L = __shfl(hp.len, h);
  o.cu = __shfl(hp.rows_before, h);
  o.tile = ug - __shfl(hp.tiles_before, h);
  // every lane computed the same unit: keep it in scalar registers (buffer
  // resources and tile offsets built from it must be wave-uniform)
  o.head = __builtin_amdgcn_readfirstlane(o.head);
  o.cu = __builtin_amdgcn_readfirstlane(o.cu);
  o.L = __builtin_amdgcn_readfirstlane(o.L);
  o.tile = __builtin_amdgcn_readfirstlane(o.tile);
  o.split = __builtin_amdgcn_readfirstlane(o.split);
  o.nsplit = __builtin_amdgcn_readfirstlane(o.nsplit);
  o.tord = __builtin_amdgcn_readfirstlane(o.tord);
  return true;
}

// Row of the partial buffers for split s of packed row `row` (tile-relative
// row r) of a unit: splits below `split` are [split][q_capacity]; the extra
// splits of tail tiles follow as [tail_split - split][tail_rows].
__device__ __forceinline__ size_t part_row(const AttnArgs& a, int s, size_t row, int tord, int r) {
  if (s < a.split) return (size_t)s * a.q_capacity + row;
  return (size_t)a.split * a.q_capacity + (size_t)(s - a.split) * a.tail_rows + (size_t)tord * kRows + r;
}

// Write one unit's rows from O^T tiles (lane: query 16 qt + l16 of the
// wave's rows, channels 16 dt + 4 g .. + 3): normalized bf16 (split == 1) or
// fp32 partials with the row sum and the reference mref[qt] of the unit.
__device__ __forceinline__ void store_rows(const AttnArgs& a, const Unit& u, int qrow0, int L, int g,
                                           f32x4 (*oacc)[4], const float* lsum, const float* mref) {
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    if (qrow0 + qt * 16 >= L) continue;
    const size_t row = (size_t)u.cu + qrow0 + qt * 16;
    if (a.split == 1) {
      const float inv = 1.0f / lsum[qt];
      uint16_t* Op = reinterpret_cast<uint16_t*>(a.o) + row * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        u32x2 w2;
        w2[0] = (uint32_t)f2bf(oacc[qt][dt][0] * inv) | ((uint32_t)f2bf(oacc[qt][dt][1] * inv) << 16);
        w2[1] = (uint32_t)f2bf(oacc[qt][dt][2] * inv) | ((uint32_t)f2bf(oacc[qt][dt][3] * inv) << 16);
        *reinterpret_cast<u32x2*>(Op + dt * 16 + 4 * g) = w2;
      }
    } else {
      const size_t prow = part_row(a, u.split, row, u.tord, qrow0 - u.tile * kRows + qt * 16);
      float* Op = a.opart + prow * kD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) *reinterpret_cast<f32x4*>(Op + dt * 16 + 4 * g) = oacc[qt][dt];
      if (g == 0) {
        a.lpart[prow] = lsum[qt];
        a.mpart[prow] = mref[qt];  // the unit's softmax reference
      }
    }
  }
}

// Argument block of a launch (shared by both score types): `per_round` gives
// the fast kernel's query tiles per XCD round for a split count (0: no tail).
AttnArgs make_attn_args(int dtype, const AttnShape& s, const void* q, const void* k, const void* vt,
                        const int32_t* lenq, void* o, int (*per_round_of)(int)) {
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.vt = vt;
  a.o = o;
  a.opart = s.opart;
  a.lpart = s.lpart;
  a.mpart = s.mpart;
  a.kmax = s.kmax;
  a.fb_count = s.fb_count;
  a.fb_list = s.fb_list;
  a.lenq = lenq;
  a.heads = s.heads;
  a.lk = s.lk;
  a.lenk = s.lenk;
  a.k_rows = s.k_rows;
  a.vt_pitch = s.vt_pitch;
  a.lq_uniform = s.lq_uniform;
  a.split = dtype == 1 ? s.split : 1;
  const int per_round = dtype == 1 && a.split > 1 && s.tail_split > a.split && s.tail_rows > 0
                            ? (s.per_round > 0 ? s.per_round : per_round_of(a.split))
                            : 0;
  const bool tail = per_round > 0 && per_round - 1 <= kMaxTailTiles;
  a.tail_split = tail ? s.tail_split : a.split;
  a.per_round = tail ? per_round : 0;
  a.tail_rows = tail ? s.tail_rows : 0;
  a.q_capacity = s.q_capacity;
  a.k8 = s.k8;
  a.kexp = s.kexp;
  a.q8 = s.q8;
  a.qexp = s.qexp;
  AttnShape sh = s;
  sh.split = a.split;
  sh.tail_split = a.tail_split;
  sh.per_round = a.per_round;
  a.total_wg = (int)attention_workgroups(dtype, sh);
  return a;
}

// Query tiles per full round of one XCD for `split` key splits of the fast
// kernel `kern` on the current device (its resident workgroups / 8 XCDs /
// split), queried once per device; 0 disables tail splitting (query failed,
// or more tail tiles than reserved).  Each kernel keeps its own cache.
template <void (*kern)(AttnArgs)>
int per_round_for(int split) {
  constexpr int kDevs = 64;
  static std::atomic<int> slots[kDevs];  // resident workgroups per XCD + 1 (0: not known yet)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) {
    (void)hipGetLastError();
    return 0;
  }
  int v = slots[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int occ = 0, cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kNW * 64, 0) != hipSuccess || occ <= 0 ||
        cus <= 0 || cus % 8) {
      (void)hipGetLastError();
      occ = 0;
      cus = 0;
    }
    v = occ * cus / 8 + 1;
    slots[dev].store(v, std::memory_order_relaxed);
  }
  const int slots_xcd = v - 1;
  if (slots_xcd <= 0 || slots_xcd % split || slots_xcd / split - 1 > kMaxTailTiles) return 0;
  return slots_xcd / split;
}

}  // namespace

}  // namespace httm
