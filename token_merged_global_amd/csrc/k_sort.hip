// Device-wide building blocks for partitions whose groups are not confined
// to fixed blocks: a stable sort of token ids by their slot (the CSR member
// lists, members ascending inside a slot) and an exclusive prefix sum.
//
// Sort.  Within each segment of n elements (one per stream and head), token
// t carries key slot(t) < 2^20; the output lists the tokens by slot, equal
// slots in ascending token id.  Two stable counting-sort passes over 10-bit
// digits (least significant first): per chunk of 4096 elements a digit
// histogram, one exclusive scan per segment over (digit, chunk), then a
// scatter in which every element's place is the scanned base of its
// (digit, chunk) plus the number of earlier elements of the chunk with the
// same digit.  The work is linear in n whatever the group sizes.
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kThreads = 256;
constexpr int kPer = 16;
constexpr int kChunk = kThreads * kPer;  // elements per chunk
constexpr int kDigitBits = 10;
constexpr int kDigits = 1 << kDigitBits;
constexpr int kScanThreads = 1024;

// Lanes of this wave whose (valid) digit equals mine: one ballot per digit bit.
__device__ __forceinline__ uint64_t same_digit(uint32_t d, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < kDigitBits; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Key of element e of a segment in a pass: pass 0 reads the caller's keys
// (the element is token e), pass 1 the keys the first pass wrote.
__global__ __launch_bounds__(kThreads) void sort_hist(const int32_t* __restrict__ keys, int n, int nchunks, int shift,
                                                      uint32_t* __restrict__ counts) {
  __shared__ uint32_t hist[kDigits];
  const int seg = blockIdx.y, chunk = blockIdx.x;
  for (int i = threadIdx.x; i < kDigits; i += kThreads) hist[i] = 0;
  __syncthreads();
  const int32_t* K = keys + (size_t)seg * n;
#pragma unroll 4
  for (int r = 0; r < kPer; ++r) {
    const int e = chunk * kChunk + r * kThreads + threadIdx.x;
    if (e < n) atomicAdd(&hist[((uint32_t)K[e] >> shift) & (kDigits - 1)], 1u);
  }
  __syncthreads();
  uint32_t* C = counts + (size_t)seg * kDigits * nchunks;
  for (int d = threadIdx.x; d < kDigits; d += kThreads) C[(size_t)d * nchunks + chunk] = hist[d];
}

// Exclusive scan, in place, of one segment's counts in (digit, chunk) order.
__global__ __launch_bounds__(kScanThreads) void sort_scan(int nchunks, uint32_t* __restrict__ counts) {
  __shared__ uint32_t wsum[kScanThreads / 64];
  const int64_t total = (int64_t)kDigits * nchunks;
  uint32_t* C = counts + (size_t)blockIdx.x * total;
  const int64_t per = (total + kScanThreads - 1) / kScanThreads;
  const int64_t b0 = threadIdx.x * per, b1 = b0 + per < total ? b0 + per : total;
  uint32_t local = 0;
  for (int64_t i = b0; i < b1; ++i) local += C[i];
  // exclusive scan of the per-thread sums over the block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t acc = inc - local;
  for (int w = 0; w < wave; ++w) acc += wsum[w];
  for (int64_t i = b0; i < b1; ++i) {
    const uint32_t c = C[i];
    C[i] = acc;
    acc += c;
  }
}

// Stable scatter of one chunk.  Rounds of 256 consecutive elements; inside a
// round the waves take turns so that places follow element order.
__global__ __launch_bounds__(kThreads) void sort_scatter(const int32_t* __restrict__ keys,
                                                         const int32_t* __restrict__ vals, int n, int nchunks,
                                                         int shift, const uint32_t* __restrict__ counts,
                                                         int32_t* __restrict__ out_keys, int32_t* __restrict__ out_a,
                                                         int32_t* __restrict__ out_b, int split) {
  __shared__ uint32_t base[kDigits];
  const int seg = blockIdx.y, chunk = blockIdx.x;
  const uint32_t* C = counts + (size_t)seg * kDigits * nchunks;
  for (int d = threadIdx.x; d < kDigits; d += kThreads) base[d] = C[(size_t)d * nchunks + chunk];
  const int32_t* K = keys + (size_t)seg * n;
  const int32_t* V = vals ? vals + (size_t)seg * n : nullptr;
  int32_t* OK = out_keys ? out_keys + (size_t)seg * n : nullptr;
  int32_t* OV = seg < split ? out_a + (size_t)seg * n : out_b + (size_t)(seg - split) * n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  __syncthreads();
  for (int r = 0; r < kPer; ++r) {
    const int e = chunk * kChunk + r * kThreads + threadIdx.x;
    if (chunk * kChunk + r * kThreads >= n) break;  // uniform over the workgroup
    const bool valid = e < n;
    const int32_t key = valid ? K[e] : 0;
    const int32_t val = valid ? (V ? V[e] : e) : 0;
    const uint32_t d = ((uint32_t)key >> shift) & (kDigits - 1);
    const uint64_t eq = same_digit(d, valid);
    const int rank = __popcll(eq & lt);
    for (int w = 0; w < kThreads / 64; ++w) {
      if (wave == w && valid) {
        const uint32_t p = base[d] + (uint32_t)rank;
        if (OK) OK[p] = key;
        OV[p] = val;
      }
      __syncthreads();  // every lane of wave w read base[] before it moves
      if (wave == w && valid && (eq >> lane) == 1ull) base[d] += (uint32_t)__popcll(eq);
      __syncthreads();
    }
  }
}

// Exclusive prefix sum of n values: per-chunk totals, one workgroup scans
// the totals, then every chunk adds its base to its local scan.
__global__ __launch_bounds__(kThreads) void scan_reduce(const int32_t* __restrict__ in, int64_t n,
                                                        int32_t* __restrict__ sums) {
  __shared__ int32_t wsum[kThreads / 64];
  int32_t s = 0;
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
#pragma unroll 4
  for (int r = 0; r < kPer; ++r) {
    const int64_t e = c0 + r * kThreads + threadIdx.x;
    if (e < n) s += in[e];
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) sums[blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

__global__ __launch_bounds__(kScanThreads) void scan_sums(int nchunks, int32_t* __restrict__ sums,
                                                          int32_t* __restrict__ total) {
  __shared__ int32_t wsum[kScanThreads / 64];
  const int per = (nchunks + kScanThreads - 1) / kScanThreads;
  const int b0 = threadIdx.x * per, b1 = b0 + per < nchunks ? b0 + per : nchunks;
  int32_t local = 0;
  for (int i = b0; i < b1; ++i) local += sums[i];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t inc = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int32_t acc = inc - local;
  for (int w = 0; w < wave; ++w) acc += wsum[w];
  if (threadIdx.x == kScanThreads - 1 && total) *total = acc + local;
  for (int i = b0; i < b1; ++i) {
    const int32_t c = sums[i];
    sums[i] = acc;
    acc += c;
  }
}

__global__ __launch_bounds__(kThreads) void scan_apply(const int32_t* __restrict__ in, int64_t n,
                                                       const int32_t* __restrict__ sums, int32_t* __restrict__ out) {
  __shared__ int32_t wsum[kThreads / 64];
  const int64_t c0 = (int64_t)blockIdx.x * kChunk + (int64_t)threadIdx.x * kPer;  // 16 consecutive per thread
  int32_t v[kPer], local = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    v[j] = c0 + j < n ? in[c0 + j] : 0;
    local += v[j];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t inc = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int32_t acc = sums[blockIdx.x] + inc - local;
  for (int w = 0; w < wave; ++w) acc += wsum[w];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (c0 + j < n) out[c0 + j] = acc;
    acc += v[j];
  }
}

}  // namespace

size_t sort_count_words(int nseg, int n) { return (size_t)nseg * kDigits * (size_t)ceil_div(n, kChunk); }

hipError_t launch_sort_by_slot(const int32_t* keys, int nseg, int n, int32_t* tmp_keys, int32_t* tmp_vals,
                               uint32_t* counts, int32_t* out_a, int32_t* out_b, int split, hipStream_t stream) {
  if (n <= 0 || nseg <= 0) return hipSuccess;
  const int nchunks = ceil_div(n, kChunk);
  const dim3 grid((unsigned)nchunks, (unsigned)nseg);
  // pass 0: digit 0 of the caller's keys -> tmp (keys and token ids)
  hipLaunchKernelGGL(sort_hist, grid, dim3(kThreads), 0, stream, keys, n, nchunks, 0, counts);
  hipLaunchKernelGGL(sort_scan, dim3((unsigned)nseg), dim3(kScanThreads), 0, stream, nchunks, counts);
  hipLaunchKernelGGL(sort_scatter, grid, dim3(kThreads), 0, stream, keys, (const int32_t*)nullptr, n, nchunks, 0,
                     counts, tmp_keys, tmp_vals, tmp_vals, nseg);
  // pass 1: digit 1 of tmp -> the output token lists
  hipLaunchKernelGGL(sort_hist, grid, dim3(kThreads), 0, stream, tmp_keys, n, nchunks, kDigitBits, counts);
  hipLaunchKernelGGL(sort_scan, dim3((unsigned)nseg), dim3(kScanThreads), 0, stream, nchunks, counts);
  hipLaunchKernelGGL(sort_scatter, grid, dim3(kThreads), 0, stream, tmp_keys, tmp_vals, n, nchunks, kDigitBits,
                     counts, (int32_t*)nullptr, out_a, out_b, split);
  return hipGetLastError();
}

size_t scan_sum_words(int64_t n) { return (size_t)((n + kChunk - 1) / kChunk) + 1; }

hipError_t launch_exclusive_scan(const int32_t* in, int64_t n, int32_t* out, int32_t* sums, int32_t* total,
                                 hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int nchunks = (int)((n + kChunk - 1) / kChunk);
  hipLaunchKernelGGL(scan_reduce, dim3((unsigned)nchunks), dim3(kThreads), 0, stream, in, n, sums);
  hipLaunchKernelGGL(scan_sums, dim3(1), dim3(kScanThreads), 0, stream, nchunks, sums, total);
  hipLaunchKernelGGL(scan_apply, dim3((unsigned)nchunks), dim3(kThreads), 0, stream, in, n, sums, out);
  return hipGetLastError();
}

}  // namespace httm
