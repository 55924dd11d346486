// Geometry-aware three-class partition and global matching.
//
// "LiteVGGT: Boosting Vanilla VGGT via Geometry-aware Cached Token Merging",
// key design 1: a geometry score per token (here its token-variance half:
// the variance of the features in the token's 3x3 neighbourhood on its
// frame's patch grid); key design 2: per frame, the highest-score patches are
// protected, destinations are every unprotected patch of the first frame and
// the lowest-score unprotected patch of each 2x2 cell in the other frames,
// the rest are sources; key design 3: every source joins its most similar
// destination (cosine) over the whole sequence and each destination's group
// is merged by the mean.  Like HTTM's matching this runs per head and per
// stream (Q and K).
//
// The groups are handed to the rest of the layer in the same form as the
// block-local matching produces: per head a CSR of members (ascending token
// ids inside a group) over `bound` slots, slots past the head's group count
// empty, and the group (slot) of every token.
//
// Pipeline: ga_variance -> ga_roles (per frame: radix top-k, 2x2 minima) ->
// ga_scan (per-frame offsets) -> ga_slots (anchor slots, destination and
// source lists) -> ga_gather (destination rows and inverse norms, bf16) ->
// ga_match (MFMA cosine argmax of sources against all destinations, split
// over destinations, packed 64-bit atomic maxima) -> ga_decode (matches,
// scores, member counts per slot) -> ga_offsets (slot offsets) -> ga_keys
// (slot of every token) -> a stable sort of the token ids by slot (members
// ascend inside a slot; linear in N whatever the group sizes).  No memset:
// the result does not depend on the order of the atomics.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "sim_tile.h"

namespace httm {

namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x) { Row8<T>::load(p, x); }

constexpr int kRoleSrc = 0, kRoleDst = 1, kRoleProtect = 2, kRoleSpecial = 3;

// fp32 sum of the available cells (centre, and left / right when present),
// left to right, for 8 channels.
__device__ __forceinline__ void row3(const float* l, const float* c, const float* r, bool hl, bool hr, float* o) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float t = hl ? __fadd_rn(l[e], c[e]) : c[e];
    o[e] = hr ? __fadd_rn(t, r[e]) : t;
  }
}

// Variance map.  A workgroup takes a tile of R x C patches of one frame
// (R * C <= 256, one thread per patch) and stages the tile with a one-patch
// halo in LDS (coalesced 16-byte loads along each grid row).  Per channel
// octet: the three rows' sums (x and x*x) left to right, then top to
// bottom; var = s2/cnt - (s1/cnt)^2 summed over channels in ascending order,
// divided by 64.  Specials get 0.
constexpr int kVarMaxStage = 340;  // staged patches: (R + 2) * (C + 2) over the tile shapes the host picks
template <typename T>
struct VarStage {
  static constexpr int kChunks = kD * (int)sizeof(T) / 16;  // 16-byte chunks of one patch
  static constexpr int kPitch = kChunks + 1;               // padded row pitch (16-byte units)
};

template <typename T>
__device__ __forceinline__ void lds_load8(const u32x4* row, int c8, float* x) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 a = row[c8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(a[i] << 16);
      x[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  } else {
    const u32x4 a = row[2 * c8], b = row[2 * c8 + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(a[i]);
      x[4 + i] = __uint_as_float(b[i]);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void ga_variance(const T* __restrict__ q, const T* __restrict__ k, int heads,
                                                   int N, int Tf, int nsp, int H, int W, int R, int C, int tiles_x,
                                                   float* __restrict__ var) {
  constexpr int P = VarStage<T>::kPitch, NC = VarStage<T>::kChunks;
  __shared__ u32x4 sX[kVarMaxStage * P];
  const int f = blockIdx.y;
  const int sh = blockIdx.z, st = sh / heads, head = sh % heads;
  const int tid = threadIdx.x;
  float* V = var + ((size_t)st * heads + head) * N + (size_t)f * Tf;
  if (blockIdx.x == 0)
    for (int j = tid; j < nsp; j += 256) V[j] = 0.f;  // specials: no score
  const int y0 = (blockIdx.x / tiles_x) * R, x0 = (blockIdx.x % tiles_x) * C;
  const int sw = C + 2, nst = (R + 2) * sw;
  const u32x4* X = reinterpret_cast<const u32x4*>((st == 0 ? q : k) + ((size_t)head * N + (size_t)f * Tf + nsp) * kD);
  // every load of the tile is issued before the first LDS store (a loop of
  // load-then-store would wait out one memory latency per iteration);
  // halo chunks outside the frame are never read and stay unwritten
  constexpr int kPer = (kVarMaxStage * NC + 255) / 256;
  u32x4 buf[kPer];
  int dst[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + j * 256;
    const int i = e / NC, c = e - i * NC;
    const int yy = y0 - 1 + i / sw, xx = x0 - 1 + i % sw;
    dst[j] = -1;
    if (e < nst * NC && yy >= 0 && yy < H && xx >= 0 && xx < W) {
      buf[j] = X[(size_t)(yy * W + xx) * NC + c];
      dst[j] = i * P + c;
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (dst[j] >= 0) sX[dst[j]] = buf[j];
  __syncthreads();
  const int ly = tid / C, lx = tid - ly * C;
  const int y = y0 + ly, x = x0 + lx;
  if (ly >= R || y >= H || x >= W) return;
  const bool hl = x > 0, hr = x + 1 < W, hu = y > 0, hd = y + 1 < H;
  const float cnt = (float)((1 + hl + hr) * (1 + hu + hd));
  const float rc = 1.0f / cnt;
  const int centre = (ly + 1) * sw + lx + 1;
  float acc = 0.f;
  for (int c8 = 0; c8 < 8; ++c8) {
    float s1[8], s2[8];
    for (int dy = -1; dy <= 1; ++dy) {
      if ((dy < 0 && !hu) || (dy > 0 && !hd)) continue;
      const int ci = centre + dy * sw;
      float a[8], b[8], c[8], a2[8], b2[8], c2[8];
      lds_load8<T>(&sX[ci * P], c8, b);
      if (hl) lds_load8<T>(&sX[(ci - 1) * P], c8, a);
      if (hr) lds_load8<T>(&sX[(ci + 1) * P], c8, c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a2[e] = hl ? __fmul_rn(a[e], a[e]) : 0.f;
        b2[e] = __fmul_rn(b[e], b[e]);
        c2[e] = hr ? __fmul_rn(c[e], c[e]) : 0.f;
      }
      float h1[8], h2[8];
      row3(a, b, c, hl, hr, h1);
      row3(a2, b2, c2, hl, hr, h2);
      if (dy < 0 || (dy == 0 && !hu)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s1[e] = h1[e];
          s2[e] = h2[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s1[e] = __fadd_rn(s1[e], h1[e]);
          s2[e] = __fadd_rn(s2[e], h2[e]);
        }
      }
    }
    // s / cnt correctly rounded in three operations: q0 = s * RN(1/cnt), then
    // one residual correction.  Checked against IEEE division for every
    // finite float and cnt in {1, 2, 3, 4, 6, 9}: equal except that -0 gives
    // +0 (harmless: only m * m and s2 >= +0 are used) and, for cnt = 6,
    // nonzero |s| < 2^-125, which take the plain division below.
    float var8[8];
    bool slow = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q1 = s1[e] * rc, q2 = s2[e] * rc;
      const float m = fmaf(fmaf(-q1, cnt, s1[e]), rc, q1);
      const float v2 = fmaf(fmaf(-q2, cnt, s2[e]), rc, q2);
      var8[e] = __fsub_rn(v2, __fmul_rn(m, m));
      slow |= cnt == 6.0f && ((s1[e] != 0.f && fabsf(s1[e]) < 0x1p-125f) || (s2[e] != 0.f && s2[e] < 0x1p-125f));
    }
    if (slow) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float m = s1[e] / cnt;
        var8[e] = __fsub_rn(s2[e] / cnt, __fmul_rn(m, m));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __fadd_rn(acc, var8[e]);
  }
  V[nsp + y * W + x] = acc / 64.0f;
}

constexpr int kRoleThreads = 256;

// Exclusive prefix over the workgroup's threads (thread order) and the total.
__device__ __forceinline__ int wg_excl_scan(int x, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kRoleThreads / 64; ++w) {
    const int t = wsum[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + inc - x;
}

// Roles of one frame: the k_protect largest scores are protected (ties to
// the smaller patch), then destinations (first frame: every other patch;
// other frames: the lowest-score unprotected patch of each 2x2 cell, ties to
// the smaller patch), sources for the rest.  Counts anchors (non-sources,
// specials included), destinations and sources per frame.
__global__ __launch_bounds__(kRoleThreads) void ga_roles(const float* __restrict__ var, int heads, int N, int Tf,
                                                          int nsp, int H, int W, int F, int k_protect,
                                                          uint8_t* __restrict__ role, int32_t* __restrict__ fcnt) {
  __shared__ uint32_t sKey[kMaxFrameHW];
  __shared__ uint8_t sRole[kMaxFrameHW];
  __shared__ uint32_t sHist[256];
  __shared__ uint32_t sSel[2];
  __shared__ int wsum[kRoleThreads / 64];
  __shared__ int sCnt[2];
  const int HW = H * W;
  const int f = blockIdx.x, sh = blockIdx.y, st = sh / heads, head = sh % heads;
  const int tid = threadIdx.x;
  const size_t tok0 = (size_t)f * Tf + nsp;
  const float* V = var + ((size_t)st * heads + head) * N + tok0;
  for (int j = tid; j < HW; j += kRoleThreads) sKey[j] = float_key(V[j] + 0.0f);
  if (tid < 2) sCnt[tid] = 0;
  __syncthreads();
  // radix select of the k-th largest key, 8 bits at a time
  uint32_t prefix = 0, kk = (uint32_t)k_protect;
  const bool any = k_protect > 0 && k_protect < HW;
  for (int pass = 0; pass < 4 && any; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kRoleThreads) sHist[i] = 0;
    __syncthreads();
    const uint32_t hmask = pass == 0 ? 0u : (0xFFFFFFFFu << (32 - 8 * pass));
    for (int j = tid; j < HW; j += kRoleThreads) {
      const uint32_t key = sKey[j];
      if ((key & hmask) == prefix) atomicAdd(&sHist[(key >> shift) & 0xFF], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // the bin of the kk-th largest key: the largest b >= 1 whose suffix
      // count S(b) = sum of bins >= b reaches kk, else 0; lane l holds bins
      // 4l .. 4l + 3 and the suffix sums come from one wave scan
      const int l = tid;
      const uint32_t h0 = sHist[4 * l], h1 = sHist[4 * l + 1], h2 = sHist[4 * l + 2], h3 = sHist[4 * l + 3];
      const uint32_t t = h0 + h1 + h2 + h3;
      uint32_t x = t;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = (uint32_t)__shfl_down((int)x, d);
        if (l + d < 64) x += y;
      }
      const uint32_t s3 = x - t + h3, s2 = s3 + h2, s1 = s2 + h1, s0 = s1 + h0;
      int cand = -1;
      if (s3 >= kk) cand = 4 * l + 3;
      else if (s2 >= kk) cand = 4 * l + 2;
      else if (s1 >= kk) cand = 4 * l + 1;
      else if (s0 >= kk && l > 0) cand = 4 * l;
      int bsel = cand;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) bsel = max(bsel, __shfl_xor(bsel, d));
      bsel = bsel < 0 ? 0 : bsel;
      if (l == (bsel >> 2)) {
        const int r = bsel & 3;
        const uint32_t sb = r == 3 ? s3 : r == 2 ? s2 : r == 1 ? s1 : s0;
        const uint32_t hb = r == 3 ? h3 : r == 2 ? h2 : r == 1 ? h1 : h0;
        sSel[0] = prefix | ((uint32_t)bsel << shift);
        sSel[1] = kk - (sb - hb);  // minus the keys in bins above bsel
      }
    }
    __syncthreads();
    prefix = sSel[0];
    kk = sSel[1];
    __syncthreads();
  }
  // protected: key above the threshold, or equal and among the first kk equal keys by patch
  const int per = ceil_div(HW, kRoleThreads);
  const int j0 = tid * per, j1 = min(HW, j0 + per);
  int eq = 0;
  if (any)
    for (int j = j0; j < j1; ++j) eq += sKey[j] == prefix;
  int total;
  int rank = wg_excl_scan(eq, wsum, total);
  for (int j = j0; j < j1; ++j) {
    bool prot;
    if (k_protect <= 0) prot = false;
    else if (k_protect >= HW) prot = true;
    else if (sKey[j] > prefix) prot = true;
    else if (sKey[j] == prefix) prot = (uint32_t)(rank++) < kk;
    else prot = false;
    sRole[j] = prot ? kRoleProtect : (f == 0 ? kRoleDst : kRoleSrc);
  }
  __syncthreads();
  if (f > 0) {
    const int cw = (W + 1) / 2, ncell = cw * ((H + 1) / 2);
    for (int c = tid; c < ncell; c += kRoleThreads) {
      const int cy = (c / cw) * 2, cx = (c % cw) * 2;
      int best = -1;
      uint32_t bk = 0;
      for (int dy = 0; dy < 2; ++dy)
        for (int dx = 0; dx < 2; ++dx) {
          const int y = cy + dy, x = cx + dx;
          if (y >= H || x >= W) continue;
          const int j = y * W + x;
          if (sRole[j] == kRoleProtect) continue;
          if (best < 0 || sKey[j] < bk || (sKey[j] == bk && j < best)) {
            best = j;
            bk = sKey[j];
          }
        }
      if (best >= 0) sRole[best] = kRoleDst;
    }
  }
  __syncthreads();
  uint8_t* R = role + ((size_t)st * heads + head) * N + (size_t)f * Tf;
  int nd = 0, ns = 0;
  for (int j = tid; j < HW; j += kRoleThreads) {
    const uint8_t r = sRole[j];
    R[nsp + j] = r;
    nd += r == kRoleDst;
    ns += r == kRoleSrc;
  }
  for (int j = tid; j < nsp; j += kRoleThreads) R[j] = kRoleSpecial;
  if (nd) atomicAdd(&sCnt[0], nd);
  if (ns) atomicAdd(&sCnt[1], ns);
  __syncthreads();
  if (tid == 0) {
    int32_t* c = fcnt + (((size_t)st * heads + head) * F + f) * 3;
    c[0] = Tf - sCnt[1];  // anchors: every token that is not a source
    c[1] = sCnt[0];
    c[2] = sCnt[1];
  }
}

// Per (stream, head): exclusive prefixes of the per-frame counts, and totals.
__global__ __launch_bounds__(256) void ga_scan(const int32_t* __restrict__ fcnt, int F, int heads,
                                               int32_t* __restrict__ foff, int32_t* __restrict__ tot,
                                               int32_t* __restrict__ lenk) {
  __shared__ int wsum[4];
  const int sh = blockIdx.x;
  const int32_t* c = fcnt + (size_t)sh * F * 3;
  int32_t* o = foff + (size_t)sh * F * 3;
  const int per = ceil_div(F, 256);
  const int f0 = threadIdx.x * per, f1 = min(F, f0 + per);
  for (int t = 0; t < 3; ++t) {
    int loc = 0;
    for (int f = f0; f < f1; ++f) loc += c[f * 3 + t];
    int total;
    int acc = wg_excl_scan(loc, wsum, total);
    for (int f = f0; f < f1; ++f) {
      o[f * 3 + t] = acc;
      acc += c[f * 3 + t];
    }
    if (threadIdx.x == 0) {
      tot[sh * 3 + t] = total;
      if (t == 0 && sh >= heads) lenk[sh - heads] = total;  // keys per head: the key stream's groups
    }
  }
}

// Per (stream, head, frame): slots of the anchors in token order, the
// destination list (with each destination's slot) and the source list.
__global__ __launch_bounds__(kRoleThreads) void ga_slots(const uint8_t* __restrict__ role, int heads, int N, int Tf,
                                                          int F, int bound, const int32_t* __restrict__ foff,
                                                          int32_t* __restrict__ slot, int32_t* __restrict__ dst_list,
                                                          int32_t* __restrict__ dst_slot,
                                                          int32_t* __restrict__ src_list, int32_t* __restrict__ gdst,
                                                          float* __restrict__ gscore, int32_t* __restrict__ cnt,
                                                          uint64_t* __restrict__ best) {
  __shared__ int wsum[kRoleThreads / 64];
  const int f = blockIdx.x, sh = blockIdx.y;
  const size_t hb = (size_t)sh * N;
  const uint8_t* R = role + hb + (size_t)f * Tf;
  const int32_t* o = foff + ((size_t)sh * F + f) * 3;
  const int per = ceil_div(Tf, kRoleThreads);
  const int t0 = threadIdx.x * per, t1 = min(Tf, t0 + per);
  int na = 0, nd = 0, ns = 0;
  for (int t = t0; t < t1; ++t) {
    const uint8_t r = R[t];
    na += r != kRoleSrc;
    nd += r == kRoleDst;
    ns += r == kRoleSrc;
  }
  int tot_a, tot_d, tot_s;
  int ra = o[0] + wg_excl_scan(na, wsum, tot_a);
  int rd = o[1] + wg_excl_scan(nd, wsum, tot_d);
  int rs = o[2] + wg_excl_scan(ns, wsum, tot_s);
  for (int t = t0; t < t1; ++t) {
    const uint8_t r = R[t];
    const int tok = f * Tf + t;
    if (r != kRoleSrc) {
      slot[hb + tok] = ra;
      gdst[hb + tok] = -1;
      gscore[hb + tok] = 0.f;
      cnt[(size_t)sh * bound + ra] = 1;  // the anchor; ga_match adds the sources
      if (r == kRoleDst) {
        dst_list[hb + rd] = tok;
        dst_slot[hb + rd] = ra;
        ++rd;
      }
      ++ra;
    } else {
      slot[hb + tok] = -1;
      best[hb + tok] = 0;  // below every packed (key, destination)
      src_list[hb + rs++] = tok;
    }
  }
}

// Global match, bf16: per (stream, head, 256 sources, destination split)
// like the block-local similarity kernel, with source and destination rows
// taken from the lists.  Each split's best (key, destination) of a source
// goes to one 64-bit atomic max: larger key, then smaller destination index,
// whatever the order of the splits.
constexpr int kSrcPerWg = 256, kDstTile = 64;
// Destination splits per source chunk: four times the workgroups of one
// split each, so the last round of workgroups is a small part of the launch.
constexpr int kDstSplits = 4;
struct GaMatchArgs {
  const void* x[2];
  int heads, N, chunks;
  const int32_t* tot;       // [2][h][3]: anchors, destinations, sources
  const int32_t* dst_list;  // [2][h][N]
  const int32_t* dst_slot;
  const int32_t* src_list;
  uint64_t* best;           // [2][h][N] per source: packed (key, ~destination index), atomic max
  float* snorm;             // [2][h][N] per source: squared norm (bf16) / inverse norm (fp32)
  int dsplit;               // destination splits per source chunk
  const uint16_t* dg;       // bf16: [2][h][dpitch][64] gathered destination rows
  const float* dinv;        // bf16: [2][h][dpitch] their inverse norms
  int dpitch;               // rows per (stream, head), a multiple of 64
};

// Positive offset of a source's keys (above |score| * |source|) from its
// squared norm; the score is (key - off) / |source|.
__device__ __forceinline__ float ga_off(float ss) { return __builtin_amdgcn_sqrtf(ss) * (1.0f + 0x1p-10f); }

// Destination rows of every (stream, head) gathered into one contiguous
// matrix (rows past the head's destinations up to the next 64 are zero), with
// the inverse norm of each row: the match then streams whole tiles with
// direct-to-LDS copies and no index indirection.  Four lanes per row; the
// squared norm adds each lane's 16 values, then lanes 0+1 and 2+3, then both.
__global__ __launch_bounds__(256) void ga_gather(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                 int heads, int N, int dpitch, const int32_t* __restrict__ tot,
                                                 const int32_t* __restrict__ dst_list, uint16_t* __restrict__ dg,
                                                 float* __restrict__ dinv) {
  const int sh = blockIdx.y, st = sh / heads, head = sh % heads;
  const int nd = tot[sh * 3 + 1];
  const int d = blockIdx.x * 64 + (threadIdx.x >> 2), part = threadIdx.x & 3;
  if (blockIdx.x * 64 >= nd) return;  // whole workgroups past the last tile
  u32x4 v0 = u32x4{0u, 0u, 0u, 0u}, v1 = v0;
  if (d < nd) {
    const u32x4* row = reinterpret_cast<const u32x4*>((st == 0 ? q : k) +
                                                      ((size_t)head * N + dst_list[(size_t)sh * N + d]) * kD);
    v0 = row[part * 2];
    v1 = row[part * 2 + 1];
  }
  float ss = sumsq8(__builtin_bit_cast(bf16x8, v1), sumsq8(__builtin_bit_cast(bf16x8, v0), 0.f));
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  u32x4* out = reinterpret_cast<u32x4*>(dg + ((size_t)sh * dpitch + d) * kD);
  out[part * 2] = v0;
  out[part * 2 + 1] = v1;
  if (part == 0) dinv[(size_t)sh * dpitch + d] = d < nd ? __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f)) : 0.f;
}

// 16 bytes per lane straight into LDS (lane i -> lds_wave_base + 16 i) from a
// buffer resource of `bytes` bytes at p: fixed per-lane offset voff,
// wave-uniform offset soff (no vector instruction per tile).
__device__ __forceinline__ void ga_lds_copy16_buf(const void* p, uint32_t bytes, uint32_t voff, uint32_t soff,
                                                  u32x4* lds_wave_base) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                                                     0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff,
                                           soff, 0, 0);
}
__device__ __forceinline__ void ga_wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__global__ __launch_bounds__(256) void ga_match_bf16(GaMatchArgs a) {
  // two tile buffers as separate LDS objects: reads of one need not wait
  // for the direct-to-LDS copies into the other
  __shared__ u32x4 sD0[kDstTile * 8], sD1[kDstTile * 8];
  __shared__ __attribute__((aligned(16))) float sI0[kDstTile], sI1[kDstTile];
  // chunk fastest: concurrent workgroups stream the same destination tiles
  const int chunk = blockIdx.x % a.chunks, rest = blockIdx.x / a.chunks;
  const int split = rest % a.dsplit, sh = rest / a.dsplit;
  const int st = sh / a.heads, head = sh % a.heads;
  const int nd = a.tot[sh * 3 + 1], ns = a.tot[sh * 3 + 2];
  const int ntiles = ceil_div(nd, kDstTile);
  const int t0 = (int)((int64_t)split * ntiles / a.dsplit), t1 = (int)((int64_t)(split + 1) * ntiles / a.dsplit);
  if (chunk * kSrcPerWg >= ns || t0 >= t1) return;
  const size_t hb = (size_t)sh * a.N;
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.x[st]) + (size_t)head * a.N * kD;
  const int32_t* SL = a.src_list + hb;
  const char* Dg = reinterpret_cast<const char*>(a.dg + (size_t)sh * a.dpitch * kD);
  const char* Di = reinterpret_cast<const char*>(a.dinv + (size_t)sh * a.dpitch);
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lg = lane >> 4, l16 = lane & 15;
  // direct-to-LDS tile copies: the lane at LDS chunk slot p (row p / 8,
  // stored chunk p % 8) fetches logical chunk (p % 8) ^ swz(row) of that row
  uint32_t goff[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int p = rd * 256 + wave * 64 + lane, row = p >> 3;
    goff[rd] = (uint32_t)(row * kD * 2 + (((p & 7) ^ swz(row)) * 16));
  }
  const uint32_t dbytes = (uint32_t)a.dpitch * kD * 2, ibytes = (uint32_t)a.dpitch * 4;
  auto load_tile = [&](int t, u32x4* sDb, float* sIb) {
    const uint32_t ts = (uint32_t)t * kDstTile * kD * 2;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) ga_lds_copy16_buf(Dg, dbytes, goff[rd], ts, sDb + rd * 256 + wave * 64);
    if (wave == 0 && lane < kDstTile / 4)
      ga_lds_copy16_buf(Di, ibytes, (uint32_t)lane * 16, (uint32_t)t * kDstTile * 4, reinterpret_cast<u32x4*>(sIb));
  };
  load_tile(t0, sD0, sI0);
  bf16x8 bs[4][2];
  float off[4];
  int ksrc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int kidx = chunk * kSrcPerWg + wave * 64 + c * 16 + l16;
    ksrc[c] = kidx;
    const int tok = SL[kidx < ns ? kidx : 0];
    const uint16_t* row = X + (size_t)tok * kD;
    float ss = 0.f;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(row + kc * 32 + lg * 8);
      bs[c][kc] = __builtin_bit_cast(bf16x8, u);
      ss = sumsq8(bs[c][kc], ss);
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    off[c] = ga_off(ss);
    // the last split is never empty
    if (split == a.dsplit - 1 && lg == 0 && kidx < ns) a.snorm[hb + tok] = ss;
  }
  uint32_t best[4] = {0u, 0u, 0u, 0u}, bestT[4] = {0u, 0u, 0u, 0u};
  int bt[4] = {0, 0, 0, 0};
  auto update = [&](const uint32_t (&tm)[4], int t) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t tT = tm[c] & ~15u;
      if (t == t0 || tT > bestT[c]) {
        best[c] = tm[c];
        bestT[c] = tT;
        bt[c] = t;
      }
    }
  };
  // only the head's last tile can be partial: it runs after the loop.  The
  // loop is unrolled by two so that every read names its buffer statically.
  const int tfull = (t1 == ntiles && nd % kDstTile) ? t1 - 1 : t1;
  auto step = [&](int t, const u32x4* sDc, const float* sIc, u32x4* sDn, float* sIn) {
    __builtin_amdgcn_sched_barrier(0);  // the previous tile's work stays before the wait
    ga_wait_vm();
    __syncthreads();
    if (t + 1 < t1) load_tile(t + 1, sDn, sIn);
    uint32_t tm[4];
    tile_argmax<false>(sDc, sIc, bs, off, lg, l16, kDstTile, tm);
    update(tm, t);
  };
  int t = t0;
  for (; t + 1 < tfull; t += 2) {
    step(t, sD0, sI0, sD1, sI1);
    step(t + 1, sD1, sI1, sD0, sI0);
  }
  if (t < tfull) {
    step(t, sD0, sI0, sD1, sI1);
    ++t;
  }
  if (t < t1) {
    // the partial tile sits in buffer (t - t0) & 1
    ga_wait_vm();
    __syncthreads();
    uint32_t tm[4];
    if ((t - t0) & 1)
      tile_argmax<true>(sD1, sI1, bs, off, lg, l16, nd - t * kDstTile, tm);
    else
      tile_argmax<true>(sD0, sI0, bs, off, lg, l16, nd - t * kDstTile, tm);
    update(tm, t);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int i = 15 - (int)(best[c] & 15u);
    int d = bt[c] * kDstTile + (i >> 2) * 16 + 4 * lg + (i & 3);
    uint32_t kb = bestT[c];
    {
      const uint32_t ko = (uint32_t)__shfl_xor((int)kb, 16);
      const int dob = __shfl_xor(d, 16);
      take_better(kb, d, ko, dob);
    }
    {
      const uint32_t ko = (uint32_t)__shfl_xor((int)kb, 32);
      const int dob = __shfl_xor(d, 32);
      take_better(kb, d, ko, dob);
    }
    if (lg == 0 && ksrc[c] < ns) {
      const uint32_t dd = (uint32_t)(d < nd ? d : 0);
      atomicMax(reinterpret_cast<unsigned long long*>(&a.best[hb + SL[ksrc[c]]]),
                ((unsigned long long)kb << 32) | (unsigned long long)(0xFFFFFFFFu - dd));
    }
  }
}

// fp32 inputs: one thread per source, destinations through LDS, fp32 dots.
__global__ __launch_bounds__(256) void ga_match_f32(GaMatchArgs a) {
  __shared__ float sD[kDstTile][kD + 1];
  __shared__ float sInv[kDstTile];
  const int chunk = blockIdx.x % a.chunks, rest = blockIdx.x / a.chunks;
  const int split = rest % a.dsplit, sh = rest / a.dsplit;
  const int st = sh / a.heads, head = sh % a.heads;
  const int nd = a.tot[sh * 3 + 1], ns = a.tot[sh * 3 + 2];
  const int ntiles = ceil_div(nd, kDstTile);
  const int tt0 = (int)((int64_t)split * ntiles / a.dsplit), tt1 = (int)((int64_t)(split + 1) * ntiles / a.dsplit);
  if (chunk * kSrcPerWg >= ns || tt0 >= tt1) return;
  const size_t hb = (size_t)sh * a.N;
  const float* X = reinterpret_cast<const float*>(a.x[st]) + (size_t)head * a.N * kD;
  const int32_t* DL = a.dst_list + hb;
  const int tid = threadIdx.x;
  const int kidx = chunk * kSrcPerWg + tid;
  const int stok = a.src_list[hb + (kidx < ns ? kidx : 0)];
  float xs[kD];
  float ss = 0.f;
  for (int c = 0; c < kD; ++c) {
    xs[c] = X[(size_t)stok * kD + c];
    ss = fmaf(xs[c], xs[c], ss);
  }
  const float inv_src = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
  float bestv = -INFINITY;
  int bidx = tt0 * kDstTile;
  for (int t0 = tt0 * kDstTile; t0 < min(nd, tt1 * kDstTile); t0 += kDstTile) {
    __syncthreads();
    for (int e = tid; e < kDstTile * kD; e += blockDim.x) {
      const int r = e / kD, c = e % kD;
      const int d = t0 + r < nd ? t0 + r : 0;
      sD[r][c] = X[(size_t)DL[d] * kD + c];
    }
    __syncthreads();
    if (tid < kDstTile) {
      float qn = 0.f;
      for (int c = 0; c < kD; ++c) qn = fmaf(sD[tid][c], sD[tid][c], qn);
      sInv[tid] = 1.0f / fmaxf(sqrtf(qn), 1e-12f);
    }
    __syncthreads();
    const int nt = min(kDstTile, nd - t0);
    for (int r = 0; r < nt; ++r) {
      float dot = 0.f;
      for (int c = 0; c < kD; ++c) dot = fmaf(xs[c], sD[r][c], dot);
      const float v = dot * sInv[r];
      if (v > bestv) {
        bestv = v;
        bidx = t0 + r;
      }
    }
  }
  if (kidx < ns) {
    if (split == a.dsplit - 1) a.snorm[hb + stok] = inv_src;  // the last split is never empty
    atomicMax(reinterpret_cast<unsigned long long*>(&a.best[hb + stok]),
              ((unsigned long long)float_key(bestv + 0.0f) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)bidx));
  }
}

// Matches from the packed atomic maxima: destination token, its slot, the
// cosine, and one more member for that slot.
__global__ __launch_bounds__(256) void ga_decode(int dtype, int heads, int N, int bound,
                                                 const int32_t* __restrict__ tot, const int32_t* __restrict__ dst_list,
                                                 const int32_t* __restrict__ dst_slot,
                                                 const int32_t* __restrict__ src_list,
                                                 const uint64_t* __restrict__ best, const float* __restrict__ snorm,
                                                 int32_t* __restrict__ gdst, int32_t* __restrict__ gslot,
                                                 float* __restrict__ gscore, int32_t* __restrict__ cnt) {
  const int sh = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= tot[sh * 3 + 2]) return;
  const size_t hb = (size_t)sh * N;
  const int tok = src_list[hb + i];
  const uint64_t b = best[hb + tok];
  int d = (int)(0xFFFFFFFFu - (uint32_t)b);
  if ((unsigned)d >= (unsigned)tot[sh * 3 + 1]) d = 0;  // never: every source has a destination
  const uint32_t kb = (uint32_t)(b >> 32);
  const int ds = dst_slot[hb + d];
  gdst[hb + tok] = dst_list[hb + d];
  gslot[hb + tok] = ds;
  float sc;
  if (dtype == 1) {
    const float ss = snorm[hb + tok];
    sc = (__uint_as_float(kb) - ga_off(ss)) * __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f)) + 0.0f;
  } else {
    const uint32_t u = (kb & 0x80000000u) ? (kb & 0x7FFFFFFFu) : ~kb;  // inverse of float_key
    sc = __uint_as_float(u) * snorm[hb + tok] + 0.0f;
  }
  gscore[hb + tok] = sc;
  atomicAdd(&cnt[(size_t)sh * bound + ds], 1);
}

// Slot offsets of one (stream, head): exclusive prefix of the member counts
// over the anchors' slots, N for the empty slots past them and at `bound`.
// 256 threads x 16 slots per chunk.
constexpr int kOffPer = 16;
__global__ __launch_bounds__(kRoleThreads) void ga_offsets(const int32_t* __restrict__ cnt,
                                                            const int32_t* __restrict__ tot, int heads, int N,
                                                            int bound, int32_t* __restrict__ off_q,
                                                            int32_t* __restrict__ off_k) {
  __shared__ int wsum[kRoleThreads / 64];
  const int sh = blockIdx.x, st = sh / heads, head = sh % heads;
  const int ng = tot[sh * 3 + 0];
  const int32_t* c = cnt + (size_t)sh * bound;
  int32_t* o = (st == 0 ? off_q : off_k) + (size_t)head * (bound + 1);
  int carry = 0;
  for (int c0 = 0; c0 < bound; c0 += kRoleThreads * kOffPer) {
    const int s0 = c0 + threadIdx.x * kOffPer;
    int v[kOffPer], local = 0;
#pragma unroll
    for (int j = 0; j < kOffPer; ++j) {
      v[j] = s0 + j < ng ? c[s0 + j] : 0;
      local += v[j];
    }
    int total;
    int acc = carry + wg_excl_scan(local, wsum, total);
#pragma unroll
    for (int j = 0; j < kOffPer; ++j) {
      if (s0 + j < bound) o[s0 + j] = s0 + j < ng ? acc : N;
      acc += v[j];
    }
    carry += total;
  }
  if (threadIdx.x == 0) o[bound] = N;
}

// The token -> slot maps, and the slot of every token as the sort key of its
// (stream, head) segment: the member lists then come from a stable sort of
// the token ids by slot (linear in N whatever the group sizes; members
// ascend by token id inside a slot).
__global__ __launch_bounds__(256) void ga_keys(const uint8_t* __restrict__ role, const int32_t* __restrict__ slot,
                                               const int32_t* __restrict__ gslot, int heads, int N,
                                               int32_t* __restrict__ keys, int32_t* __restrict__ grp_q,
                                               int32_t* __restrict__ grp_k) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)2 * heads * N) return;
  const int sh = (int)(i / N), tok = (int)(i - (int64_t)sh * N);
  const int st = sh / heads, head = sh % heads;
  const int s = role[i] == kRoleSrc ? gslot[i] : slot[i];
  keys[i] = s;
  (st == 0 ? grp_q : grp_k)[(size_t)head * N + tok] = s;
}

}  // namespace

hipError_t launch_global_match(int dtype, int N, const void* x, const int32_t* tot, const int32_t* dst_list,
                               const int32_t* src_list, int ns, uint16_t* dg, float* dinv, int dpitch, uint64_t* best,
                               float* snorm, hipStream_t stream) {
  if (ns <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(ga_gather, dim3((unsigned)(dpitch / 64), 1u), dim3(256), 0, stream, (const uint16_t*)x,
                       (const uint16_t*)x, 1, N, dpitch, tot, dst_list, dg, dinv);
  GaMatchArgs a;
  a.x[0] = x;
  a.x[1] = x;
  a.heads = 1;
  a.N = N;
  a.chunks = ceil_div(ns, kSrcPerWg);
  a.tot = tot;
  a.dst_list = dst_list;
  a.dst_slot = nullptr;
  a.src_list = src_list;
  a.best = best;
  a.snorm = snorm;
  a.dsplit = kDstSplits;
  a.dg = dg;
  a.dinv = dinv;
  a.dpitch = dpitch;
  const unsigned mgrid = (unsigned)(kDstSplits * a.chunks);
  if (dtype == 1)
    hipLaunchKernelGGL(ga_match_bf16, dim3(mgrid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(ga_match_f32, dim3(mgrid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_ga_partition(int dtype, const GaShape& s, const void* q, const void* k, const GaBuffers& b,
                               hipStream_t stream, int phase) {
  const int SH = 2 * s.heads;
  if (phase == 0) {
    // near-equal tiles of at most 32 columns and 16 rows (<= 256 patches)
    const int tx = ceil_div(s.W, 32), C = ceil_div(s.W, tx);
    const int r0 = std::min(16, 256 / C), ty = ceil_div(s.H, r0), R = ceil_div(s.H, ty);
    if ((R + 2) * (C + 2) > kVarMaxStage) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(tx * ty), (unsigned)s.F, (unsigned)SH);
    HTTM_DISPATCH(dtype, hipLaunchKernelGGL(ga_variance<T>, grid, dim3(256), 0, stream, (const T*)q, (const T*)k,
                                            s.heads, s.N, s.Tf, s.nsp, s.H, s.W, R, C, tx, b.var));
    hipLaunchKernelGGL(ga_roles, dim3((unsigned)s.F, (unsigned)SH), dim3(kRoleThreads), 0, stream, b.var, s.heads,
                       s.N, s.Tf, s.nsp, s.H, s.W, s.F, s.k_protect, b.role, b.fcnt);
    hipLaunchKernelGGL(ga_scan, dim3((unsigned)SH), dim3(256), 0, stream, b.fcnt, s.F, s.heads, b.foff, b.tot,
                       b.lenk);
    hipLaunchKernelGGL(ga_slots, dim3((unsigned)s.F, (unsigned)SH), dim3(kRoleThreads), 0, stream, b.role, s.heads,
                       s.N, s.Tf, s.F, s.bound, b.foff, b.slot, b.dst_list, b.dst_slot, b.src_list, b.gdst, b.gscore,
                       b.cnt, b.best);
    return hipGetLastError();
  }
  if (s.max_src == 0 && phase < 3) return hipSuccess;  // a single frame: no sources, every token is its own group
  if (phase == 1) {
    if (dtype == 1)
      hipLaunchKernelGGL(ga_gather, dim3((unsigned)(s.dpitch / 64), (unsigned)SH), dim3(256), 0, stream,
                         (const uint16_t*)q, (const uint16_t*)k, s.heads, s.N, s.dpitch, b.tot, b.dst_list, b.dg,
                         b.dinv);
    return hipGetLastError();
  }
  if (phase == 2) {
    GaMatchArgs a;
    a.x[0] = q;
    a.x[1] = k;
    a.heads = s.heads;
    a.N = s.N;
    a.chunks = ceil_div(s.max_src, kSrcPerWg);
    a.tot = b.tot;
    a.dst_list = b.dst_list;
    a.dst_slot = b.dst_slot;
    a.src_list = b.src_list;
    a.best = b.best;
    a.snorm = b.snorm;
    a.dsplit = kDstSplits;
    a.dg = b.dg;
    a.dinv = b.dinv;
    a.dpitch = s.dpitch;
    const unsigned mgrid = (unsigned)(SH * kDstSplits * a.chunks);
    if (dtype == 1)
      hipLaunchKernelGGL(ga_match_bf16, dim3(mgrid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(ga_match_f32, dim3(mgrid), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (phase != 3) return hipErrorInvalidValue;
  if (s.max_src > 0)
    hipLaunchKernelGGL(ga_decode, dim3((unsigned)ceil_div(s.max_src, 256), (unsigned)SH), dim3(256), 0, stream,
                       dtype, s.heads, s.N, s.bound, b.tot, b.dst_list, b.dst_slot, b.src_list, b.best, b.snorm,
                       b.gdst, b.gslot, b.gscore, b.cnt);
  hipLaunchKernelGGL(ga_offsets, dim3((unsigned)SH), dim3(kRoleThreads), 0, stream, b.cnt, b.tot, s.heads, s.N,
                     s.bound, b.off_q, b.off_k);
  const unsigned grid = (unsigned)(((int64_t)SH * s.N + 255) / 256);
  hipLaunchKernelGGL(ga_keys, dim3(grid), dim3(256), 0, stream, b.role, b.slot, b.gslot, s.heads, s.N, b.tmp,
                     b.grp_q, b.grp_k);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sort_by_slot(b.tmp, SH, s.N, b.sort_keys, b.sort_vals, b.sort_counts, b.mem_q, b.mem_k, s.heads,
                             stream);
}

}  // namespace httm
