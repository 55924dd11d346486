// Cross-head adaptive outlier selection.
//
// "HTTM: Head-wise Temporal Token Merging for Faster VGGT", key design 3: over
// all heads and tokens, the top-d % largest query deviations are outliers
// (mask M_o in {0,1}^{h x N}).  Ties go to the smaller flat index h*N + n.
//
// Deviations are non-negative floats, so their bit patterns order like their
// values.  A radix select finds the threshold pattern T = the k_o-th largest
// in three histogram passes (11, 11, 10 bits; the first is accumulated by the
// deviation producer as it writes them); every workgroup recomputes the
// prefix it needs from the previous histogram in LDS, so no serial "find the
// bin" kernel sits between the passes.  A marking pass sets values above T and
// counts values equal to T per chunk; a last pass gives the equal values
// their rank in flat-index order and keeps the first ones the budget allows.
// Counts are integer atomics only, so the mask is deterministic.
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kThreads = 256;
// Elements per thread: 16 (small layers: enough workgroups to fill the
// GPU) or 64 (large layers: a quarter of the workgroups, so each one's
// threshold prologue covers more data).  One select uses one value.
constexpr int kPerSmall = 16, kPerLarge = 64;
constexpr int64_t kLargeFrom = int64_t(1) << 22;
constexpr int kChunk = kThreads * kPerSmall;  // smallest chunk: sizes the per-chunk tie counts
constexpr int kBins = 2048;

struct Scratch {
  uint32_t* h0;   // [2048] bits 31..21
  uint32_t* h1;   // [2048] bits 20..10 under prefix B0
  uint32_t* h2;   // [2048] bits 9..0 under prefix (B0, B1)
  uint32_t* sel;  // [4] threshold, count above, ties taken, k_o
  uint32_t* ties; // [nchunks]
};

__device__ __forceinline__ Scratch scratch_of(uint32_t* s) {
  Scratch r;
  r.h0 = s;
  r.h1 = s + kBins;
  r.h2 = s + 2 * kBins;
  r.sel = s + 3 * kBins;
  r.ties = s + 3 * kBins + 4;
  return r;
}

// Zero the layer's atomic targets before its producers run (one launch);
// also writes the merge index header when asked.
__global__ void zero_init(float* kmax, int heads, int* fb_count, uint32_t* radix, int radix_words,
                          int32_t* ocnt, int64_t ocnt_words, IndexHeader hdr, uint32_t* hdr_dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (hdr_dst && i < 16) hdr_dst[i] = hdr.w[i];
  if (i < heads) kmax[i] = 0.f;
  if (i == 0) *fb_count = 0;
  if (i < radix_words) radix[i] = 0;
  for (int64_t j = i; j < ocnt_words; j += (int64_t)gridDim.x * blockDim.x) ocnt[j] = 0;
}

__global__ void fill_bytes(uint8_t* p, int64_t n, uint8_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Exclusive prefix sum over the workgroup's threads (thread order), and the
// workgroup total; wsum holds one word per wave.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const uint32_t t = wsum[w];
    before += w < wave ? t : 0u;
    total += t;
  }
  __syncthreads();  // wsum may be reused
  return before + inc - x;
}

// Find bin b with above(b) < k <= above(b) + hist[b], above(b) = sum of bins > b.
// Writes b and k - above(b) to out[0], out[1].  nb = 2048 or 1024.
__device__ void find_bin(const uint32_t* hist, int nb, uint32_t k, uint32_t* wsum, uint32_t* out) {
  const int per = nb / kThreads;
  const int t = threadIdx.x;
  // thread t owns bins [nb - (t+1)*per, nb - t*per), i.e. thread 0 the top bins
  const int hi = nb - t * per, lo = hi - per;
  uint32_t s = 0;
  for (int b = lo; b < hi; ++b) s += hist[b];
  uint32_t total;
  const uint32_t above0 = block_excl_scan(s, wsum, total);  // count strictly above thread t's bins
  if (above0 < k && above0 + s >= k) {
    uint32_t above = above0;
    for (int b = hi - 1; b >= lo; --b) {
      if (above + hist[b] >= k) {
        out[0] = (uint32_t)b;
        out[1] = k - above;
        break;
      }
      above += hist[b];
    }
  }
  __syncthreads();
}

// Keys of 16 consecutive values: the bit patterns of non-negative values
// (KEY false: deviations), or the order-preserving float_key of any finite
// value (KEY true: cosine scores).  0xFFFFFFFF, which no finite value
// yields, marks positions past the end.
template <bool KEY, int PER>
__device__ __forceinline__ void load_chunk(const float* d, int64_t total, int64_t base, uint32_t* u) {
  const int64_t i0 = base + (int64_t)threadIdx.x * PER;
  if (i0 + PER <= total) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(d + i0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[4 * q + e] = KEY ? float_key(__uint_as_float(v[e]) + 0.0f) : v[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e)
      u[e] = (i0 + e < total) ? (KEY ? float_key(d[i0 + e] + 0.0f) : __float_as_uint(d[i0 + e]))
                              : 0xFFFFFFFFu;  // sentinel: no bin
  }
}

// pass 0..2: histogram of bits [shift, shift+width) among values whose higher
// bits equal the prefix found from the previous histograms.
template <int PASS, bool KEY, int PER>
__global__ __launch_bounds__(kThreads) void radix_hist(const float* __restrict__ delta, int64_t total,
                                                       uint32_t k_o, uint32_t* scratch) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t part[kThreads / 64];
  __shared__ uint32_t res[4];
  Scratch s = scratch_of(scratch);
  uint32_t prefix = 0;
  if (PASS >= 1) {
    for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = s.h0[i];
    __syncthreads();
    find_bin(hist, kBins, k_o, part, res);
    prefix = res[0];
    if (PASS == 2) {
      const uint32_t k1 = res[1];
      __syncthreads();
      for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = s.h1[i];
      __syncthreads();
      find_bin(hist, kBins, k1, part, res);
      prefix = (prefix << 11) | res[0];
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0;
  __syncthreads();
  uint32_t u[PER];
  load_chunk<KEY, PER>(delta, total, (int64_t)blockIdx.x * kThreads * PER, u);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (u[e] == 0xFFFFFFFFu) continue;
    if (PASS == 0) {
      atomicAdd(&hist[u[e] >> 21], 1u);
    } else if (PASS == 1) {
      if ((u[e] >> 21) == prefix) atomicAdd(&hist[(u[e] >> 10) & 0x7FFu], 1u);
    } else {
      if ((u[e] >> 10) == prefix) atomicAdd(&hist[u[e] & 0x3FFu], 1u);
    }
  }
  __syncthreads();
  uint32_t* g = PASS == 0 ? s.h0 : (PASS == 1 ? s.h1 : s.h2);
  for (int i = threadIdx.x; i < kBins; i += kThreads)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

__device__ void threshold(const Scratch& s, uint32_t k_o, uint32_t* hist, uint32_t* part,
                          uint32_t* res, uint32_t& T, uint32_t& need) {
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = s.h0[i];
  __syncthreads();
  find_bin(hist, kBins, k_o, part, res);
  const uint32_t b0 = res[0], k1 = res[1];
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = s.h1[i];
  __syncthreads();
  find_bin(hist, kBins, k1, part, res);
  const uint32_t b1 = res[0], k2 = res[1];
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = s.h2[i];
  __syncthreads();
  find_bin(hist, 1024, k2, part, res);
  T = (b0 << 21) | (b1 << 10) | res[0];
  need = res[1];
  __syncthreads();
}

// Marks values above T; counts values equal to T in this chunk.
template <bool KEY, int PER>
__global__ __launch_bounds__(kThreads) void radix_mark(const float* __restrict__ delta, int64_t total,
                                                       uint32_t k_o, uint32_t* scratch,
                                                       uint8_t* __restrict__ mask) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t part[kThreads / 64];
  __shared__ uint32_t res[4];
  __shared__ uint32_t cnt;
  Scratch s = scratch_of(scratch);
  uint32_t T, need;
  threshold(s, k_o, hist, part, res, T, need);
  if (threadIdx.x == 0) cnt = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    s.sel[0] = T;
    s.sel[1] = k_o - need;
    s.sel[2] = need;
    s.sel[3] = k_o;
  }
  __syncthreads();
  uint32_t u[PER];
  const int64_t i0 = (int64_t)blockIdx.x * kThreads * PER + (int64_t)threadIdx.x * PER;
  load_chunk<KEY, PER>(delta, total, (int64_t)blockIdx.x * kThreads * PER, u);
  uint32_t eq = 0;
  uint8_t m[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const bool valid = u[e] != 0xFFFFFFFFu;
    m[e] = (valid && u[e] > T) ? 1 : 0;
    eq += (valid && u[e] == T) ? 1u : 0u;
  }
  if (i0 + PER <= total) {
#pragma unroll
    for (int b16 = 0; b16 < PER / 16; ++b16) {
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 16 * b16 + 4 * q;
        w[q] = (uint32_t)m[e] | ((uint32_t)m[e + 1] << 8) | ((uint32_t)m[e + 2] << 16) | ((uint32_t)m[e + 3] << 24);
      }
      *reinterpret_cast<u32x4*>(mask + i0 + 16 * b16) = w;
    }
  } else {
    for (int e = 0; e < PER; ++e)
      if (i0 + e < total) mask[i0 + e] = m[e];
  }
  if (eq) atomicAdd(&cnt, eq);
  __syncthreads();
  if (threadIdx.x == 0) s.ties[blockIdx.x] = cnt;
}

// Values equal to T, in flat-index order, take the remaining budget.
template <bool KEY, int PER>
__global__ __launch_bounds__(kThreads) void radix_ties(const float* __restrict__ delta, int64_t total,
                                                       uint32_t* scratch, uint8_t* __restrict__ mask) {
  __shared__ uint32_t part[kThreads / 64];
  Scratch s = scratch_of(scratch);
  if (s.ties[blockIdx.x] == 0) return;
  const uint32_t T = s.sel[0], need = s.sel[2];
  // ties in earlier chunks
  uint32_t acc = 0;
  for (int c = threadIdx.x; c < (int)blockIdx.x; c += kThreads) acc += s.ties[c];
  uint32_t before;
  (void)block_excl_scan(acc, part, before);
  if (before >= need) return;
  uint32_t u[PER];
  const int64_t i0 = (int64_t)blockIdx.x * kThreads * PER + (int64_t)threadIdx.x * PER;
  load_chunk<KEY, PER>(delta, total, (int64_t)blockIdx.x * kThreads * PER, u);
  uint32_t eq = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) eq += (u[e] == T && u[e] != 0xFFFFFFFFu) ? 1u : 0u;
  uint32_t chunk_total;
  uint32_t rank = before + block_excl_scan(eq, part, chunk_total);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (u[e] == T && u[e] != 0xFFFFFFFFu) {
      if (rank < need) mask[i0 + e] = 1;
      ++rank;
    }
  }
}

}  // namespace

namespace {
// The passes of one select with PER elements per thread; pass 0 only when
// no producer accumulated it.
template <bool KEY, int PER>
void radix_select(const float* vals, int64_t total, uint32_t k, uint32_t* scratch, uint8_t* mask, bool pass0,
                  hipStream_t stream) {
  const int nchunks = (int)((total + (int64_t)kThreads * PER - 1) / ((int64_t)kThreads * PER));
  if (pass0)
    hipLaunchKernelGGL((radix_hist<0, KEY, PER>), dim3(nchunks), dim3(kThreads), 0, stream, vals, total, k, scratch);
  hipLaunchKernelGGL((radix_hist<1, KEY, PER>), dim3(nchunks), dim3(kThreads), 0, stream, vals, total, k, scratch);
  hipLaunchKernelGGL((radix_hist<2, KEY, PER>), dim3(nchunks), dim3(kThreads), 0, stream, vals, total, k, scratch);
  hipLaunchKernelGGL((radix_mark<KEY, PER>), dim3(nchunks), dim3(kThreads), 0, stream, vals, total, k, scratch, mask);
  hipLaunchKernelGGL((radix_ties<KEY, PER>), dim3(nchunks), dim3(kThreads), 0, stream, vals, total, scratch, mask);
}
}  // namespace

size_t outlier_scratch_words(int64_t total) {
  return 3 * kBins + 4 + (size_t)((total + kChunk - 1) / kChunk);
}

hipError_t launch_zero_init(float* kmax, int heads, int* fb_count, uint32_t* radix, int radix_words,
                            int32_t* ocnt, int64_t ocnt_words, hipStream_t stream, const IndexHeader* hdr,
                            uint32_t* hdr_dst) {
  int64_t n = heads > radix_words ? heads : radix_words;
  if (ocnt_words > n) n = ocnt_words;
  int64_t grid = (n + 255) / 256;
  grid = grid < 1 ? 1 : (grid > 2048 ? 2048 : grid);
  IndexHeader h{};
  if (hdr) h = *hdr;
  hipLaunchKernelGGL(zero_init, dim3((unsigned)grid), dim3(256), 0, stream, kmax, heads, fb_count, radix,
                     radix_words, ocnt, ocnt_words, h, hdr ? hdr_dst : nullptr);
  return hipGetLastError();
}

int outlier_hist0_words() { return kBins; }

namespace {
__global__ void zero_words(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}
}  // namespace

hipError_t launch_topk(const float* vals, int64_t total, int64_t k, uint8_t* mask, uint32_t* scratch,
                       hipStream_t stream) {
  const unsigned tgrid = (unsigned)((total + 255) / 256);
  if (total <= 0) return hipSuccess;
  if (k <= 0 || k >= total) {
    hipLaunchKernelGGL(fill_bytes, dim3(tgrid), dim3(256), 0, stream, mask, total, (uint8_t)(k <= 0 ? 0 : 1));
    return hipGetLastError();
  }
  const int64_t words = (int64_t)outlier_scratch_words(total);
  hipLaunchKernelGGL(zero_words, dim3((unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)), dim3(256),
                     0, stream, scratch, words);
  const uint32_t kk = (uint32_t)k;
  if (total >= kLargeFrom)
    radix_select<true, kPerLarge>(vals, total, kk, scratch, mask, true, stream);
  else
    radix_select<true, kPerSmall>(vals, total, kk, scratch, mask, true, stream);
  return hipGetLastError();
}

hipError_t launch_outliers(const float* delta, int64_t total, int64_t k_o, uint8_t* mask,
                           uint32_t* scratch, hipStream_t stream) {
  const unsigned tgrid = (unsigned)((total + 255) / 256);
  if (k_o <= 0 || k_o >= total) {
    const uint8_t v = k_o <= 0 ? 0 : 1;
    hipLaunchKernelGGL(fill_bytes, dim3(tgrid), dim3(256), 0, stream, mask, total, v);
  } else {
    const uint32_t k = (uint32_t)k_o;
    // pass 0 (bits 31..21) was accumulated by the deviation producer into the zeroed scratch
    if (total >= kLargeFrom)
      radix_select<false, kPerLarge>(delta, total, k, scratch, mask, false, stream);
    else
      radix_select<false, kPerSmall>(delta, total, k, scratch, mask, false, stream);
  }
  return hipGetLastError();
}

}  // namespace httm
