// Per-block top-r selection and group construction.
//
// "HTTM: Head-wise Temporal Token Merging for Faster VGGT", key design 1: the
// r matched sources with the highest similarity merge into their destination;
// a merged token stands for its destination and those sources.  Ties go to
// the smaller source position.
//
// One workgroup per (stream, head, block) works entirely in LDS:
//   1. if 0 < r < |S|: bitonic sort of 64-bit keys (descending score, then
//      ascending source index) and keep the first r;
//   2. bitonic sort of (group << 12 | position) over the block's positions,
//      group = destination index for destinations and selected sources, and
//      |D| for unselected sources (they follow as singletons);
//   3. the sorted order is the member list (CSR): members ascend inside a
//      group, which for frame-major blocks is ascending original token id.
// Everything is integer work after the float-to-key transform, so the result
// is deterministic.  Extra workgroups fill the special-token slots.
#include "common.h"
#include "kernels.h"

namespace httm {

namespace {

constexpr int kThreads = 512;

struct SelArgs {
  Geo g;
  const int32_t* match[2];
  const float* score[2];
  Csr csr[2];
};

template <typename K>
__device__ void bitonic_sort(K* key, int n_pad) {
  for (int k = 2; k <= n_pad; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n_pad; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const K a = key[i], b = key[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            key[i] = b;
            key[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

__global__ __launch_bounds__(kThreads) void block_select(SelArgs a) {
  __shared__ uint64_t s64[kMaxBlock];
  __shared__ uint8_t sel[kMaxBlock];
  const Geo& g = a.g;
  const int per_head = g.nblocks + 1;
  const int st = blockIdx.x / (g.heads * per_head);
  const int rem = blockIdx.x % (g.heads * per_head);
  const int head = rem / per_head;
  const int b = rem % per_head;
  const Csr c = a.csr[st];
  const size_t tokbase = (size_t)head * g.N;
  const size_t slotbase = (size_t)head * (g.nslots[st] + 1);

  if (b == g.nblocks) {
    // special tokens: one slot each, after the patch slots; then the end marker
    const int nspec = g.F * g.nsp;
    const int slot_sp0 = g.nslots[st] - nspec;
    for (int e = threadIdx.x; e < nspec; e += blockDim.x) {
      const int tok = (e / g.nsp) * g.T + (e % g.nsp);
      c.members[tokbase + g.P + e] = tok;
      c.off[slotbase + slot_sp0 + e] = g.P + e;
      c.group[tokbase + tok] = slot_sp0 + e;
    }
    if (threadIdx.x == 0) c.off[slotbase + g.nslots[st]] = g.N;
    return;
  }

  const BlockInfo bi = block_info(g, b, st);
  const int s = g.s[st];
  const int32_t* match = a.match[st] + (size_t)head * g.nsrc[st] + bi.src0;
  const float* score = a.score[st] + (size_t)head * g.nsrc[st] + bi.src0;

  // 1. which sources merge
  if (bi.r >= bi.ns) {
    for (int i = threadIdx.x; i < bi.ns; i += blockDim.x) sel[i] = 1;
  } else if (bi.r == 0) {
    for (int i = threadIdx.x; i < bi.ns; i += blockDim.x) sel[i] = 0;
  } else {
    const int np = pow2_at_least(bi.ns);
    for (int i = threadIdx.x; i < np; i += blockDim.x) {
      uint64_t key = ~0ull;
      if (i < bi.ns) key = ((uint64_t)(~float_key(score[i] + 0.0f)) << 32) | (uint32_t)i;
      s64[i] = key;
    }
    __syncthreads();
    bitonic_sort(s64, np);
    for (int i = threadIdx.x; i < bi.ns; i += blockDim.x) {
      const int k = (int)(uint32_t)s64[i];
      sel[k] = i < bi.r ? 1 : 0;
    }
  }
  __syncthreads();

  // 2. group keys over block positions
  uint32_t* s32 = reinterpret_cast<uint32_t*>(s64);
  const int np = pow2_at_least(bi.n);
  for (int i = threadIdx.x; i < np; i += blockDim.x) {
    uint32_t key = 0xFFFFFFFFu;
    if (i < bi.n) {
      int grp;
      if (i % s == 0) {
        grp = i / s;
      } else {
        const int k = i - i / s - 1;
        const int mk = match[k];
        grp = sel[k] ? ((unsigned)mk < (unsigned)bi.nd ? mk : 0) : bi.nd;
      }
      key = ((uint32_t)grp << 12) | (uint32_t)i;
    }
    s32[i] = key;
  }
  __syncthreads();
  bitonic_sort(s32, np);

  // 3. CSR
  const int first_single = bi.nd + bi.r;
  for (int p = threadIdx.x; p < bi.n; p += blockDim.x) {
    const uint32_t key = s32[p];
    const int grp = (int)(key >> 12);
    const int pos = (int)(key & 0xFFFu);
    const int tok = block_token(g, bi, pos);
    c.members[tokbase + bi.start + p] = tok;
    int slot;
    if (grp < bi.nd) {
      slot = bi.slot0 + grp;
      if (p == 0 || (int)(s32[p - 1] >> 12) != grp) c.off[slotbase + slot] = bi.start + p;
    } else {
      slot = bi.slot0 + bi.nd + (p - first_single);
      c.off[slotbase + slot] = bi.start + p;
    }
    c.group[tokbase + tok] = slot;
  }
}

}  // namespace

hipError_t launch_select(const Geo& g, const int32_t* match_q, const float* score_q,
                         const int32_t* match_k, const float* score_k, Csr q, Csr k,
                         hipStream_t stream) {
  SelArgs a;
  a.g = g;
  a.match[0] = match_q;
  a.match[1] = match_k;
  a.score[0] = score_q;
  a.score[1] = score_k;
  a.csr[0] = q;
  a.csr[1] = k;
  const int grid = 2 * g.heads * (g.nblocks + 1);
  hipLaunchKernelGGL(block_select, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace httm
