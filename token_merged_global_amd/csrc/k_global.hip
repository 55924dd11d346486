// Head-shared global matching: the merging that the HTTM page contrasts its
// design with ("HTTM: Head-wise Temporal Token Merging for Faster VGGT",
// research background and key design 1: ToMe-style merging as FastVGGT uses
// it applies one merge topology to every head and matches over the whole
// long sequence; key design 2 prices that global matching at about
// 0.19 N^2 d_head for a 25 % destination / 75 % source split).
//
// One partition of the tokens is built from the keys averaged over heads and
// handed to every head's query and key streams in the CSR form of the
// block-local matching:
//   gm_metric  m[n] = (sum over heads of k[h][n]) / h, fp32 in head order,
//              rounded to the layer's element type;
//   gm_lists   patch tokens in original order, every 4th a destination;
//   (ga_gather, ga_match: the cosine argmax of every source over all
//              destinations on MFMA, shared with the geometry-aware partition)
//   gm_scores  matched destination and cosine of every source;
//   (radix top-r of the cosines, ties to the smaller source position)
//   gm_slots   slots: destinations first (their merged sources join them),
//              then the unmerged sources, then the specials;
//   (stable sort of the token ids by slot: members ascend inside a slot)
//   gm_offsets slot offsets from the sorted members;
//   gm_spread  the partition copied to the query and key CSR of every head.
// This file is compiled with -ffp-contract=off: the metric is the written
// sequence of rounded fp32 adds and one division.
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

template <typename T>
__global__ __launch_bounds__(256) void gm_metric(const T* __restrict__ k, int heads, int N, T* __restrict__ m) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (token, 8-channel part)
  if (g >= (int64_t)N * 8) return;
  const int64_t n = g >> 3;
  const int part = (int)(g & 7);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int h = 0; h < heads; ++h) {
    float x[8];
    Row8<T>::load(k + ((size_t)h * N + n) * kD + part * 8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __fadd_rn(acc[e], x[e]);
  }
  const float hf = (float)heads;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc[e] / hf;  // correctly rounded division
  Row8<T>::store(m + n * kD + part * 8, acc);
}

// Roles from the position p of a patch token in original order: p % 4 == 0
// is destination p / 4, any other is source p - p / 4 - 1.
__global__ __launch_bounds__(256) void gm_lists(int N, int Tf, int nsp, int HW, int32_t* __restrict__ tot,
                                                int32_t* __restrict__ dst_list, int32_t* __restrict__ src_list,
                                                uint64_t* __restrict__ best, int32_t* __restrict__ dbg_match,
                                                float* __restrict__ dbg_score) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t == 0) {
    const int P = N / Tf * HW, nd = ceil_div(P, 4);
    tot[0] = 0;
    tot[1] = nd;
    tot[2] = P - nd;
  }
  if (t >= N) return;
  const int f = t / Tf, tt = t - f * Tf;
  dbg_match[t] = -1;
  dbg_score[t] = 0.f;
  if (tt < nsp) return;
  const int p = f * HW + tt - nsp;
  if ((p & 3) == 0) {
    dst_list[p >> 2] = t;
  } else {
    src_list[p - (p >> 2) - 1] = t;
    best[t] = 0;  // below every packed (key, destination)
  }
}

// Positive offset of a source's keys from its squared norm (the match
// kernel's convention: score = (key - off) / |source|).
__device__ __forceinline__ float gm_off(float ss) { return __builtin_amdgcn_sqrtf(ss) * (1.0f + 0x1p-10f); }

__global__ __launch_bounds__(256) void gm_scores(int dtype, int ns, int nd, const int32_t* __restrict__ src_list,
                                                 const int32_t* __restrict__ dst_list,
                                                 const uint64_t* __restrict__ best, const float* __restrict__ snorm,
                                                 int32_t* __restrict__ match, float* __restrict__ score,
                                                 int32_t* __restrict__ dbg_match, float* __restrict__ dbg_score) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= ns) return;
  const int tok = src_list[i];
  const uint64_t b = best[tok];
  int d = (int)(0xFFFFFFFFu - (uint32_t)b);
  if ((unsigned)d >= (unsigned)nd) d = 0;  // never: every source has a destination
  const uint32_t kb = (uint32_t)(b >> 32);
  float sc;
  if (dtype == 1) {
    const float ss = snorm[tok];
    sc = (__uint_as_float(kb) - gm_off(ss)) * __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f)) + 0.0f;
  } else {
    const uint32_t u = (kb & 0x80000000u) ? (kb & 0x7FFFFFFFu) : ~kb;  // inverse of float_key
    sc = __uint_as_float(u) * snorm[tok] + 0.0f;
  }
  match[i] = d;
  score[i] = sc;
  dbg_match[tok] = dst_list[d];
  dbg_score[tok] = sc;
}

__global__ __launch_bounds__(256) void gm_unsel(int ns, const uint8_t* __restrict__ sel, int32_t* __restrict__ u) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < ns) u[i] = sel[i] ? 0 : 1;
}

// Slot of every token: destination d -> d; a merged source -> its
// destination's slot; an unmerged source -> nd + (unmerged sources before
// it); special e (in token order) -> nd + (ns - r) + e.
__global__ __launch_bounds__(256) void gm_slots(int N, int Tf, int nsp, int HW, int nd, int ns, int r,
                                                const uint8_t* __restrict__ sel, const int32_t* __restrict__ match,
                                                const int32_t* __restrict__ urank, int32_t* __restrict__ keys) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= N) return;
  const int f = t / Tf, tt = t - f * Tf;
  int s;
  if (tt < nsp) {
    s = nd + (ns - r) + f * nsp + tt;
  } else {
    const int p = f * HW + tt - nsp;
    if ((p & 3) == 0) {
      s = p >> 2;
    } else {
      const int i = p - (p >> 2) - 1;
      s = sel[i] ? match[i] : nd + urank[i];
    }
  }
  keys[t] = s;
}

// Offsets from the members sorted by slot: every slot holds at least one
// token and slots are numbered densely, so slot s starts where its run of
// members starts.
__global__ __launch_bounds__(256) void gm_offsets(int N, int L, const int32_t* __restrict__ keys,
                                                  const int32_t* __restrict__ mem, int32_t* __restrict__ off) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= N) return;
  const int s = keys[mem[p]];
  if (p == 0 || keys[mem[p - 1]] != s) off[s] = p;
  if (p == 0) off[L] = N;
}

// The shared partition into the query and key CSR of every head.
__global__ __launch_bounds__(256) void gm_spread(int heads, int N, int L, const int32_t* __restrict__ mem,
                                                 const int32_t* __restrict__ off, const int32_t* __restrict__ grp,
                                                 int32_t* __restrict__ qm, int32_t* __restrict__ qo,
                                                 int32_t* __restrict__ qg, int32_t* __restrict__ km,
                                                 int32_t* __restrict__ ko, int32_t* __restrict__ kg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = (int64_t)2 * N + L + 1;
  if (i >= per * heads) return;
  const int h = (int)(i / per);
  const int64_t j = i - (int64_t)h * per;
  if (j < N) {
    const int32_t v = mem[j];
    qm[(size_t)h * N + j] = v;
    km[(size_t)h * N + j] = v;
  } else if (j < 2 * (int64_t)N) {
    const int64_t t = j - N;
    const int32_t v = grp[t];
    qg[(size_t)h * N + t] = v;
    kg[(size_t)h * N + t] = v;
  } else {
    const int64_t s = j - 2 * (int64_t)N;
    const int32_t v = off[s];
    qo[(size_t)h * (L + 1) + s] = v;
    ko[(size_t)h * (L + 1) + s] = v;
  }
}

}  // namespace

hipError_t launch_global_partition(int dtype, const GmShape& s, const void* k, const GmBuffers& b,
                                   hipStream_t stream, int phase) {
  const unsigned tgrid = (unsigned)ceil_div(s.N, 256);
  if (phase == 0) {
    HTTM_DISPATCH(dtype, hipLaunchKernelGGL(gm_metric<T>, dim3((unsigned)ceil_div(s.N * 8, 256)), dim3(256), 0,
                                            stream, (const T*)k, s.heads, s.N, (T*)b.metric));
    hipLaunchKernelGGL(gm_lists, dim3(tgrid), dim3(256), 0, stream, s.N, s.Tf, s.nsp, s.HW, b.tot, b.dst_list,
                       b.src_list, b.best, b.dbg_match, b.dbg_score);
    return hipGetLastError();
  }
  if (phase == 1) {
    if (s.ns > 0 && s.nd > 0)
      return launch_global_match(dtype, s.N, b.metric, b.tot, b.dst_list, b.src_list, s.ns, b.dg, b.dinv, s.dpitch,
                                 b.best, b.snorm, stream);
    return hipSuccess;
  }
  if (phase != 2) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  if (s.ns > 0 && s.nd > 0) {
    hipLaunchKernelGGL(gm_scores, dim3((unsigned)ceil_div(s.ns, 256)), dim3(256), 0, stream, dtype, s.ns, s.nd,
                       b.src_list, b.dst_list, b.best, b.snorm, b.match, b.score, b.dbg_match, b.dbg_score);
    e = launch_topk(b.score, s.ns, s.r, b.sel, b.topk, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gm_unsel, dim3((unsigned)ceil_div(s.ns, 256)), dim3(256), 0, stream, s.ns, b.sel, b.unsel);
    e = launch_exclusive_scan(b.unsel, s.ns, b.urank, b.scan_sums, nullptr, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(gm_slots, dim3(tgrid), dim3(256), 0, stream, s.N, s.Tf, s.nsp, s.HW, s.nd, s.ns, s.r, b.sel,
                     b.match, b.urank, b.keys);
  e = launch_sort_by_slot(b.keys, 1, s.N, b.sort_keys, b.sort_vals, b.sort_counts, b.members, b.members, 1, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gm_offsets, dim3(tgrid), dim3(256), 0, stream, s.N, s.L, b.keys, b.members, b.off);
  const int64_t per = (int64_t)2 * s.N + s.L + 1;
  hipLaunchKernelGGL(gm_spread, dim3((unsigned)((per * s.heads + 255) / 256)), dim3(256), 0, stream, s.heads, s.N,
                     s.L, b.members, b.off, b.keys, b.q.members, b.q.off, b.q.group, b.k.members, b.k.off, b.k.group);
  return hipGetLastError();
}

}  // namespace httm
