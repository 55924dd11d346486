// Memory-bound kernels of the layer: mean merge, query deviation, outlier
// restore, cached-index merge, unmerge, and the V transpose of the unmerged
// baseline.
//
// "HTTM: Head-wise Temporal Token Merging for Faster VGGT", key design 1: a
// merged token is the mean of its members, V follows K's groups, unmerge
// copies the merged output back to every member.  Key design 3: every
// query's L2 deviation to its merged token; outliers are subtracted from
// their merged token and restored as separate tokens.  "LiteVGGT", key
// design 3: x_d_up = (x_d + sum_{s in S_d} x_s) / (1 + |S_d|); cached merge
// indices are reused by later layers.
//
// All reductions are gathers over a CSR member list (no float atomics):
// sums run in member order (ascending token id) with separately rounded fp32
// operations, so results are deterministic and a mean or deviation equals
// the same sequence of IEEE operations written in any other language.  This
// file is compiled with -ffp-contract=off so that no add and multiply are
// fused into an FMA (the rounding helpers are inlined from headers, where a
// pragma in this file would not reach).  Division and square root use the
// plain operators, which HIP lowers to correctly rounded sequences
// (__fsqrt_rn would be the approximate native square root).
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kHist0Bins = 2048;  // first radix pass of the outlier select: bits 31..21
constexpr int kMergeQGroups = 32;  // query groups per merge_q workgroup (8 lanes each)

__device__ __forceinline__ float rn_div(float a, float b) { return a / b; }  // correctly rounded

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x) { Row8<T>::load(p, x); }
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* x) { Row8<T>::store(p, x); }

// Stored value of x in storage type T (what the attention MFMA reads).
template <typename T>
__device__ __forceinline__ float stored(float x) {
  if constexpr (sizeof(T) == 2) return bf2f(f2bf(x));
  return x;
}

// 8 consecutive lanes hold one row of T values (8 channels each): the row's
// L2 norm, valid in every lane of the group.
template <typename T>
__device__ __forceinline__ float row_norm8(const float* x) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float r = stored<T>(x[e]);
    ss += r * r;
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  ss += __shfl_xor(ss, 4);
  return sqrtf(ss);
}

// Workgroup max of per-thread values, then one atomic max into *gmax
// (non-negative floats order like their bit patterns, so the result does not
// depend on arrival order).  Every thread of the workgroup must call it.
__device__ __forceinline__ void wg_atomic_max(float v, unsigned* smax, float* gmax) {
  if (threadIdx.x == 0) *smax = 0u;
  __syncthreads();
  if (v > 0.f) atomicMax(smax, __float_as_uint(v));
  __syncthreads();
  if (threadIdx.x == 0 && *smax) atomicMax(reinterpret_cast<unsigned*>(gmax), *smax);
}

// Gather-sum of one CSR segment [m0, m1) of member rows, 8 channels per lane,
// in member order with separately rounded fp32 adds.  Member ids are fetched
// C at a time and all C rows are requested before the first add, so a lane
// keeps up to C row loads (times the number of tensors) in flight instead of
// one dependent chain per member.  Rows past m1 re-read the segment's first
// row (already in flight) and are not added.
template <typename T, int C, int NT>
__device__ __forceinline__ void gather_sum(const T* const (&X)[NT], const int32_t* __restrict__ mem, int m0,
                                           int m1, int part, float (&acc)[NT][8]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
  for (int mb = m0; mb < m1; mb += C) {
    int tok[C];
#pragma unroll
    for (int j = 0; j < C; ++j) tok[j] = mem[mb + j < m1 ? mb + j : mb];
    float x[C][NT][8];
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
      for (int t = 0; t < NT; ++t) load8(X[t] + (size_t)tok[j] * kD + part * 8, x[j][t]);
#pragma unroll
    for (int j = 0; j < C; ++j) {
      if (mb + j < m1) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[t][e] = __fadd_rn(acc[t][e], x[j][t][e]);
      }
    }
  }
}

// Merged K and V.  One workgroup (512 threads) = 64 consecutive key slots of
// one head.  The members of those slots are contiguous in the CSR list; they
// are staged through LDS in chunks of kStage rows, loaded evenly by all
// lanes (8 lanes per row, 8 channels each) regardless of group sizes, and
// then each slot's 8 lanes add their members from LDS in member order
// (separately rounded fp32 adds, like the oracle's means).  K~ rows are
// multiplied by kscale (the softmax scale times log2 e, rounded once with
// the mean); V~ means go through LDS and are written transposed
// (vt[h][c][slot]) so that the attention kernel reads V~ along keys with plain
// row loads.
template <typename T>
struct KvStage {
  static constexpr int kRows = sizeof(T) == 2 ? 128 : 96;
  static constexpr int kChunks = (int)sizeof(T) / 2;  // 16-byte chunks per 8-channel lane part
};

template <typename T>
__device__ __forceinline__ void lds_row8_load(const u32x4* p, float* x) {
  if constexpr (sizeof(T) == 2) {
    Row8<uint16_t>::load(reinterpret_cast<const uint16_t*>(p), x);
  } else {
    Row8<float>::load(reinterpret_cast<const float*>(p), x);
  }
}

template <typename T>
__global__ __launch_bounds__(512) void merge_kv(int N, int lk, int lk_pad, float kscale, const T* __restrict__ k,
                                                const T* __restrict__ v,
                                                const int32_t* __restrict__ members,
                                                const int32_t* __restrict__ off, T* __restrict__ kt,
                                                T* __restrict__ vt, float* __restrict__ kmax,
                                                const int32_t* __restrict__ lenk) {
  constexpr int R = KvStage<T>::kRows, NC = KvStage<T>::kChunks;  // NC 16-byte chunks per lane part
  __shared__ u32x4 sRow[2][R][8 * NC];  // [tensor][row][lane part * NC + chunk]
  __shared__ int sOf[65];
  __shared__ unsigned sMax;
  const int tiles = lk_pad / 64;
  const int head = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int tid = threadIdx.x;
  const int ls = tid >> 3, part = tid & 7;
  const int slot = tile * 64 + ls;
  const T* K = k + (size_t)head * N * kD;
  const T* V = v + (size_t)head * N * kD;
  const int32_t* mem = members + (size_t)head * N;
  const int32_t* of = off + (size_t)head * (lk + 1);
  // keys of this head: lk, or fewer when the partition is data dependent (lenk)
  const int lkh = lenk ? lenk[head] : lk;
  const int nsl = min(64, lkh - tile * 64);  // real slots of this tile (<= 0: padding tile)
  if (nsl > 0 && tid <= nsl) sOf[tid] = of[tile * 64 + tid];
  __syncthreads();
  const int mb = nsl > 0 ? sOf[0] : 0, me = nsl > 0 ? sOf[nsl] : 0;
  const int m0 = slot < lkh ? sOf[ls] : 0, m1 = slot < lkh ? sOf[ls + 1] : 0;
  float acc[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[t][e] = 0.f;
  for (int c0 = mb; c0 < me; c0 += R) {
    const int cnt = min(R, me - c0);
    // stage rows c0 .. c0 + cnt: row i by the 8 lanes of group ls (i = ls, ls + 64, ...)
    int tok[(R + 63) / 64];
#pragma unroll
    for (int q = 0; q < (R + 63) / 64; ++q) {
      const int i = ls + 64 * q;
      tok[q] = i < cnt ? mem[c0 + i] : -1;
    }
#pragma unroll
    for (int q = 0; q < (R + 63) / 64; ++q) {
      const int i = ls + 64 * q;
      if (tok[q] >= 0) {
        const u32x4* kr = reinterpret_cast<const u32x4*>(K + (size_t)tok[q] * kD) + part * NC;
        const u32x4* vr = reinterpret_cast<const u32x4*>(V + (size_t)tok[q] * kD) + part * NC;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          sRow[0][i][part * NC + cc] = kr[cc];
          sRow[1][i][part * NC + cc] = vr[cc];
        }
      }
    }
    __syncthreads();
    const int a0 = max(m0, c0), a1 = min(m1, c0 + cnt);
    for (int m = a0; m < a1; ++m) {
      float xk[8], xv[8];
      lds_row8_load<T>(&sRow[0][m - c0][part * NC], xk);
      lds_row8_load<T>(&sRow[1][m - c0][part * NC], xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[0][e] = __fadd_rn(acc[0][e], xk[e]);
        acc[1][e] = __fadd_rn(acc[1][e], xv[e]);
      }
    }
    __syncthreads();  // before the next chunk overwrites the rows
  }
  float nmax = 0.f;
  if (slot < lkh) {
    const float c = (float)(m1 - m0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[0][e] = rn_div(acc[0][e], c) * kscale;
      acc[1][e] = rn_div(acc[1][e], c);
    }
  }
  store8(kt + ((size_t)head * lk_pad + slot) * kD + part * 8, acc[0]);
  const float nrm = row_norm8<T>(acc[0]);
  if (slot < lkh) nmax = nrm;
  // transpose V~ through the (now free) staging buffer: float [64 channels][65]
  float(*sV)[65] = reinterpret_cast<float(*)[65]>(&sRow[0][0][0]);
  static_assert(sizeof(sRow) >= sizeof(float) * 64 * 65, "staging buffer holds the transpose");
#pragma unroll
  for (int e = 0; e < 8; ++e) sV[part * 8 + e][ls] = acc[1][e];
  wg_atomic_max(nmax, &sMax, kmax + head);  // also orders the sV writes before the reads below
  {
    const int c = tid >> 3, j = tid & 7;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sV[c][j * 8 + e];
    store8(vt + ((size_t)head * kD + c) * lk_pad + tile * 64 + j * 8, x);
  }
}

// Query group sums and deviations.  One workgroup = G consecutive query
// groups of one head (G = 32 measured a third faster than 64 at 100 frames
// and equal at 30).  Every deviation also enters the first histogram of the
// outlier radix select (bits 31..21 of its non-negative float pattern).
// Phase 1: 8 lanes per group sum the members (fp32, member order) and keep
// the mean in LDS.  Phase 2: one lane per member computes
// sqrt(sum_c (q_c - mean_c)^2), the sum over channels in ascending order;
// members of the G groups are contiguous in the CSR, a binary search over the
// G + 1 offsets finds each member's group.
template <typename T, int G>
__global__ __launch_bounds__(8 * G) void merge_q(int N, int gq, const T* __restrict__ q,
                                               const int32_t* __restrict__ members,
                                               const int32_t* __restrict__ off,
                                               float* __restrict__ qsum,
                                               float* __restrict__ delta,
                                               uint32_t* __restrict__ hist0) {
  constexpr int NT = 8 * G;
  __shared__ float sMean[G][kD + 1];
  __shared__ int sOff[G + 1];
  __shared__ uint32_t sHist[kHist0Bins];
  for (int i = threadIdx.x; i < kHist0Bins; i += NT) sHist[i] = 0;
  const int tiles = ceil_div(gq, G);
  const int head = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int g0 = tile * G;
  const int ng = min(G, gq - g0);
  const int tid = threadIdx.x;
  const int ls = tid >> 3, part = tid & 7;
  const T* const X[1] = {q + (size_t)head * N * kD};
  const int32_t* mem = members + (size_t)head * N;
  const int32_t* of = off + (size_t)head * (gq + 1);
  if (tid <= ng) sOff[tid] = of[g0 + tid];
  if (ls < ng) {
    const int grp = g0 + ls;
    const int m0 = of[grp], m1 = of[grp + 1];
    float sm[1][8];
    gather_sum<T, 8, 1>(X, mem, m0, m1, part, sm);
    Row8<float>::store(qsum + ((size_t)head * gq + grp) * kD + part * 8, sm[0]);
    const float cnt = (float)(m1 - m0);
#pragma unroll
    for (int e = 0; e < 8; ++e) sMean[ls][part * 8 + e] = rn_div(sm[0][e], cnt);
  }
  __syncthreads();
  const int mb = sOff[0], me = sOff[ng];
  for (int m = mb + tid; m < me; m += NT) {
    int lo = 0, hi = ng - 1;  // largest j with sOff[j] <= m
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sOff[mid] <= m) lo = mid; else hi = mid - 1;
    }
    const int tok = mem[m];
    const T* row = X[0] + (size_t)tok * kD;
    float acc = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < 8; ++c8) {
      float x[8];
      load8(row + c8 * 8, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = __fsub_rn(x[e], sMean[lo][c8 * 8 + e]);
        acc = __fadd_rn(acc, __fmul_rn(t, t));
      }
    }
    const float d = sqrtf(acc);
    delta[(size_t)head * N + tok] = d;
    atomicAdd(&sHist[__float_as_uint(d) >> 21], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kHist0Bins; i += NT)
    if (sHist[i]) atomicAdd(&hist0[i], sHist[i]);
}

// Restore, part 1: 8 lanes per initial query group, 32 groups per
// workgroup (the tiles of restore_rows).  A group with c members of which
// o are outliers yields (c > o) + o final slots; o counts the mask over the
// group's contiguous member list (no atomics).  Writes o per group and the
// slot total of each tile.
constexpr int kTileGroups = 32;
__global__ __launch_bounds__(256) void restore_count(int N, int gq, const int32_t* __restrict__ members,
                                                     const int32_t* __restrict__ off,
                                                     const uint8_t* __restrict__ mask,
                                                     int32_t* __restrict__ ocnt, int32_t* __restrict__ tsum) {
  __shared__ int sV[kTileGroups];
  const int tiles = ceil_div(gq, kTileGroups);
  const int head = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int ls = threadIdx.x >> 3, part = threadIdx.x & 7;
  const int g = tile * kTileGroups + ls;
  int v = 0;
  if (g < gq) {
    const int32_t* mem = members + (size_t)head * N;
    const uint8_t* mk = mask + (size_t)head * N;
    const int32_t* of = off + (size_t)head * (gq + 1);
    const int m0 = of[g], m1 = of[g + 1];
    int o = 0;
    for (int m = m0 + part; m < m1; m += 8) o += mk[mem[m]] ? 1 : 0;
    o += __shfl_xor(o, 1);
    o += __shfl_xor(o, 2);
    o += __shfl_xor(o, 4);
    if (part == 0) ocnt[(size_t)head * gq + g] = o;
    v = (m1 - m0 > o ? 1 : 0) + o;
  }
  if (part == 0) sV[ls] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int i = 0; i < kTileGroups; ++i) t += sV[i];
    tsum[(size_t)head * tiles + tile] = t;
  }
}

// Restore, part 2 (one workgroup per head): exclusive scan of the tile
// totals into tile bases; the head's final length goes to lenq and closes
// the final offsets with N.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void restore_scan(int N, int tiles, int32_t* __restrict__ tsum,
                                                             int32_t* __restrict__ lenq,
                                                             int32_t* __restrict__ foff) {
  __shared__ int wsum[kScanThreads / 64];
  const int head = blockIdx.x;
  int32_t* T = tsum + (size_t)head * tiles;
  const int per = ceil_div(tiles, kScanThreads);
  const int b0 = threadIdx.x * per, b1 = min(tiles, b0 + per);
  int local = 0;
  for (int i = b0; i < b1; ++i) local += T[i];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int acc = inc - local;
  for (int w = 0; w < wave; ++w) acc += wsum[w];
  for (int i = b0; i < b1; ++i) {
    const int c = T[i];
    T[i] = acc;
    acc += c;
  }
  if (threadIdx.x == kScanThreads - 1) {
    lenq[head] = acc;
    foff[(size_t)head * (N + 1) + acc] = N;
  }
}


// Restore, part 3: 8 lanes per initial query group.  A group's first final
// slot is its tile's base plus the slots of the tile's earlier groups.  The
// 8 lanes look at 8 members at a time: ballots over the group's lanes rank
// survivors and outliers in member order, so every member's final position
// is known without a serial walk.  Outlier rows are then subtracted from
// the group sum (in member order) and copied to their own packed rows; the
// remaining members' mean becomes the group's row (if any remain).  Writes
// the packed Q~ rows, the final partition (members reordered: remaining
// first, then outliers) and every token's packed row for unmerge.
template <typename T>
__global__ __launch_bounds__(256) void restore_rows(int heads, int N, int gq, const T* __restrict__ q,
                                                    const int32_t* __restrict__ members,
                                                    const int32_t* __restrict__ off,
                                                    const float* __restrict__ qsum,
                                                    const uint8_t* __restrict__ mask,
                                                    const int32_t* __restrict__ ocnt,
                                                    const int32_t* __restrict__ tbase,
                                                    const int32_t* __restrict__ lenq,
                                                    int32_t* __restrict__ cu_q, T* __restrict__ qt,
                                                    int32_t* __restrict__ fmembers,
                                                    int32_t* __restrict__ foff,
                                                    int32_t* __restrict__ slot) {
  __shared__ int sV[kTileGroups];
  const int tiles = ceil_div(gq, kTileGroups);
  const int head = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int tid = threadIdx.x;
  const HeadPrefix hp = head_prefix(lenq, 0, heads, 0);  // every wave, before any exit
  if (blockIdx.x == 0 && tid < 64) {
    if (tid < heads) cu_q[tid] = hp.rows_before;
    if (tid == 0) cu_q[heads] = hp.rows_total;
  }
  const int cu = __shfl(hp.rows_before, head);
  const int ls = tid >> 3, part = tid & 7;
  const int g = tile * kTileGroups + ls;
  const int sub = (tid & 63) >> 3;
  const int32_t* of = off + (size_t)head * (gq + 1);
  int m0 = 0, m1 = 0, o = 0;
  if (g < gq) {
    m0 = of[g];
    m1 = of[g + 1];
    o = ocnt[(size_t)head * gq + g];
  }
  const int nsurv = (m1 - m0) - o;
  const int surv = nsurv > 0 ? 1 : 0;
  if (part == 0) sV[ls] = g < gq ? surv + o : 0;
  __syncthreads();
  if (g >= gq) return;  // whole 8-lane groups leave together
  int before = 0;
  for (int i = 0; i < ls; ++i) before += sV[i];
  const T* Q = q + (size_t)head * N * kD;
  const int32_t* mem = members + (size_t)head * N;
  const uint8_t* mk = mask + (size_t)head * N;
  int32_t* fm = fmembers + (size_t)head * N;
  int32_t* fo = foff + (size_t)head * (N + 1);
  int32_t* sl = slot + (size_t)head * N;
  const int b = cu + tbase[(size_t)head * tiles + tile] + before;
  float sm[8];
  if (surv) Row8<float>::load(qsum + ((size_t)head * gq + g) * kD + part * 8, sm);
  const uint32_t below = (1u << part) - 1u;
  int rs = 0, ro = 0;  // survivors / outliers seen so far
  for (int mb = m0; mb < m1; mb += 8) {
    const int m = mb + part;
    const bool valid = m < m1;
    const int tok = valid ? mem[m] : 0;
    const bool isout = valid && mk[tok] != 0;
    const uint32_t bo = (uint32_t)(__ballot(isout) >> (sub * 8)) & 0xFFu;
    const uint32_t bv = (uint32_t)(__ballot(valid) >> (sub * 8)) & 0xFFu;
    const uint32_t bs = bv & ~bo;
    if (isout) {
      const int j = ro + __popc(bo & below);
      const int row = b + surv + j;
      fm[m0 + nsurv + j] = tok;
      fo[row - cu] = m0 + nsurv + j;
      sl[tok] = row;
    } else if (valid) {
      fm[m0 + rs + __popc(bs & below)] = tok;
      sl[tok] = b;
    }
    // outlier rows of this batch, in member order (all 8 lanes of the group)
    uint32_t bits = bo;
    int j = ro;
    while (bits) {
      const int src = __ffs(bits) - 1;
      bits &= bits - 1u;
      const int t = __shfl(tok, (tid & 63 & ~7) + src);
      float x[8];
      load8(Q + (size_t)t * kD + part * 8, x);
      if (surv) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm[e] = __fsub_rn(sm[e], x[e]);
      }
      store8(qt + (size_t)(b + surv + j) * kD + part * 8, x);
      ++j;
    }
    ro += __popc(bo);
    rs += __popc(bs);
  }
  if (surv) {
    const float cnt = (float)nsurv;
#pragma unroll
    for (int e = 0; e < 8; ++e) sm[e] = rn_div(sm[e], cnt);
    store8(qt + (size_t)b * kD + part * 8, sm);
    if (part == 0) fo[b - cu] = m0;
  }
}

// Cached layers: Q~ row R (packed over heads) = mean of the q rows of its
// final members (in member order).  8 lanes per row, up to 8 member rows in
// flight per lane.
template <typename T>
__global__ __launch_bounds__(256) void merge_q_cached(int heads, int N, const T* __restrict__ q,
                                                      const int32_t* __restrict__ fmembers,
                                                      const int32_t* __restrict__ foff,
                                                      const int32_t* __restrict__ lenq,
                                                      T* __restrict__ qt) {
  __shared__ int sCu[kMaxHeads + 1];
  if (threadIdx.x < 64) {
    const HeadPrefix hp = head_prefix(lenq, 0, heads, 0);
    if ((int)threadIdx.x < heads) sCu[threadIdx.x] = hp.rows_before;
    if (threadIdx.x == 0) sCu[heads] = hp.rows_total;
  }
  __syncthreads();
  const int R = blockIdx.x * 32 + (threadIdx.x >> 3), part = threadIdx.x & 7;
  if (R >= sCu[heads]) return;
  int head = 0;
  while (sCu[head + 1] <= R) ++head;
  const int sidx = R - sCu[head];
  const int32_t* fo = foff + (size_t)head * (N + 1);
  const int32_t* fm = fmembers + (size_t)head * N;
  const T* const Q[1] = {q + (size_t)head * N * kD};
  const int m0 = fo[sidx], m1 = fo[sidx + 1];
  float sm[1][8];
  gather_sum<T, 8, 1>(Q, fm, m0, m1, part, sm);
  const float cnt = (float)(m1 - m0);
#pragma unroll
  for (int e = 0; e < 8; ++e) sm[0][e] = rn_div(sm[0][e], cnt);
  store8(qt + (size_t)R * kD + part * 8, sm[0]);
}

// out[h][n][:] = o[slot[h][n]][:], 8 channels per thread (16 B for bf16).
template <typename T>
__global__ __launch_bounds__(256) void unmerge(int64_t rows, const int32_t* __restrict__ slot,
                                               const T* __restrict__ o, T* __restrict__ out) {
  // 8 lanes per 128-byte row (bf16), 8 rows per lane group: all slot and row
  // loads are in flight before the first store; the output is written once
  // and not read here again, so its stores do not allocate in the caches
  constexpr int kR = 8;
  const int64_t g8 = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 3;
  const int part = (int)(threadIdx.x & 7);
  const int64_t row0 = g8 * kR;
  int32_t sl[kR];
#pragma unroll
  for (int k = 0; k < kR; ++k) sl[k] = row0 + k < rows ? slot[row0 + k] : 0;
  if (sizeof(T) == 2) {
    u32x4 v[kR];
#pragma unroll
    for (int k = 0; k < kR; ++k) v[k] = *reinterpret_cast<const u32x4*>(o + (size_t)sl[k] * kD + part * 8);
#pragma unroll
    for (int k = 0; k < kR; ++k)
      if (row0 + k < rows)
        __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(out + (size_t)(row0 + k) * kD + part * 8));
  } else {
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      if (row0 + k >= rows) break;
      const f32x4* src = reinterpret_cast<const f32x4*>(o + (size_t)sl[k] * kD + part * 8);
      f32x4* dst = reinterpret_cast<f32x4*>(out + (size_t)(row0 + k) * kD + part * 8);
      dst[0] = src[0];
      dst[1] = src[1];
    }
  }
}

// Unmerged baseline inputs: kc[h][n] = k[h][n] * kscale, vt[h][c][n] =
// v[h][n][c] for n < N, both 0 for N <= n < pitch (whole 64-key tiles).
template <typename T>
__global__ __launch_bounds__(256) void prep_dense(int N, int pitch, float kscale, const T* __restrict__ k,
                                                  const T* __restrict__ v, T* __restrict__ kc,
                                                  T* __restrict__ vt, float* __restrict__ kmax) {
  __shared__ float sT[kD][65];
  __shared__ unsigned sMax;
  const int tiles = pitch / 64;
  const int head = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const T* K = k + (size_t)head * N * kD;
  const T* V = v + (size_t)head * N * kD;
  float nmax = 0.f;
  for (int idx = threadIdx.x; idx < 64 * 8; idx += 256) {
    const int r = idx >> 3, j = idx & 7;
    const int n = tile * 64 + r;
    float x[8];
    float kx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kx[e] = 0.f;
    if (n < N) {
      load8(K + (size_t)n * kD + j * 8, kx);
#pragma unroll
      for (int e = 0; e < 8; ++e) kx[e] *= kscale;
    }
    store8(kc + ((size_t)head * pitch + n) * kD + j * 8, kx);  // rows past N stay zero
    const float nrm = row_norm8<T>(kx);
    if (n < N) nmax = fmaxf(nmax, nrm);
    if (n < N) {
      load8(V + (size_t)n * kD + j * 8, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sT[j * 8 + e][r] = x[e];
  }
  wg_atomic_max(nmax, &sMax, kmax + head);  // also orders the sT writes before the reads below
  for (int idx = threadIdx.x; idx < 64 * 8; idx += 256) {
    const int c = idx >> 3, j = idx & 7;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sT[c][j * 8 + e];
    store8(vt + ((size_t)head * kD + c) * pitch + tile * 64 + j * 8, x);
  }
}

}  // namespace

hipError_t launch_merge_kv(int dtype, int heads, int N, int lk, int lk_pad, float kscale, const void* k,
                           const void* v, const int32_t* members, const int32_t* off, void* kt,
                           void* vt, float* kmax, hipStream_t stream, const int32_t* lenk) {
  const int grid = heads * (lk_pad / 64);
  HTTM_DISPATCH(dtype, hipLaunchKernelGGL(merge_kv<T>, dim3(grid), dim3(512), 0, stream, N, lk,
                                          lk_pad, kscale, (const T*)k, (const T*)v, members, off, (T*)kt,
                                          (T*)vt, kmax, lenk));
  return hipGetLastError();
}

hipError_t launch_merge_q(int dtype, int heads, int N, int gq, const void* q,
                          const int32_t* members, const int32_t* off, float* qsum, float* delta,
                          uint32_t* hist0, hipStream_t stream) {
  constexpr int G = kMergeQGroups;
  const int grid = heads * ceil_div(gq, G);
  HTTM_DISPATCH(dtype, hipLaunchKernelGGL((merge_q<T, G>), dim3(grid), dim3(8 * G), 0, stream, N, gq,
                                          (const T*)q, members, off, qsum, delta, hist0));
  return hipGetLastError();
}

hipError_t launch_restore(int dtype, int heads, int N, int gq, const void* q,
                          const int32_t* members, const int32_t* off, const float* qsum,
                          const uint8_t* mask, RestoreOut o, hipStream_t stream) {
  const int tiles = ceil_div(gq, kTileGroups);
  const int grid = heads * tiles;
  hipLaunchKernelGGL(restore_count, dim3(grid), dim3(256), 0, stream, N, gq, members, off, mask, o.ocnt, o.tbase);
  hipLaunchKernelGGL(restore_scan, dim3(heads), dim3(kScanThreads), 0, stream, N, tiles, o.tbase, o.lenq, o.foff);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  HTTM_DISPATCH(dtype, hipLaunchKernelGGL(restore_rows<T>, dim3(grid), dim3(256), 0, stream,
                                          heads, N, gq, (const T*)q, members, off, qsum, mask, o.ocnt,
                                          o.tbase, o.lenq, o.cu_q, (T*)o.qt, o.fmembers, o.foff,
                                          o.slot));
  return hipGetLastError();
}

hipError_t launch_merge_q_cached(int dtype, int heads, int N, int64_t q_capacity, const void* q,
                                 const int32_t* fmembers, const int32_t* foff,
                                 const int32_t* lenq, void* qt, hipStream_t stream) {
  const int grid = (int)((q_capacity + 31) / 32);
  HTTM_DISPATCH(dtype, hipLaunchKernelGGL(merge_q_cached<T>, dim3(grid), dim3(256), 0, stream,
                                          heads, N, (const T*)q, fmembers, foff, lenq, (T*)qt));
  return hipGetLastError();
}

hipError_t launch_unmerge(int dtype, int heads, int N, const int32_t* slot, const void* o,
                          void* out, hipStream_t stream) {
  const int64_t rows = (int64_t)heads * N;
  const int grid = (int)(((rows + 7) / 8 * 8 + 255) / 256);
  HTTM_DISPATCH(dtype, hipLaunchKernelGGL(unmerge<T>, dim3(grid), dim3(256), 0, stream, rows,
                                          slot, (const T*)o, (T*)out));
  return hipGetLastError();
}

hipError_t launch_prep_dense(int dtype, int heads, int N, int pitch, float kscale, const void* k,
                             const void* v, void* kc, void* vt, float* kmax, hipStream_t stream) {
  const int grid = heads * (pitch / 64);
  HTTM_DISPATCH(dtype, hipLaunchKernelGGL(prep_dense<T>, dim3(grid), dim3(256), 0, stream, N, pitch, kscale,
                                          (const T*)k, (const T*)v, (T*)kc, (T*)vt, kmax));
  return hipGetLastError();
}

}  // namespace httm
