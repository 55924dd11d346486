// Ragged flash attention over the merged sequences.
//
// "HTTM: Head-wise Temporal Token Merging for Faster VGGT", overall framework
// and settings: attention runs on the shortened Q~ / K~ / V~ (bf16,
// FlashAttention on the page's A100).  Q~ is ragged per head because the
// outlier budget is shared across heads (key design 3); K~ / V~ have the same
// length in every head.
//
// Work unit = (head, tile of 256 query rows, key split).  One workgroup = 4
// waves x 64 query rows (four 16-row tiles per wave) on
// v_mfma_f32_16x16x32_bf16, the full-rate bf16 MFMA of gfx950; 64 rows per
// wave halve the LDS operand bytes per FLOP against 32, and 4 waves share
// each key tile copy.  Key tiles of 64 rows of K~ and the matching 64 columns
// of V~^T (stored transposed by the merge kernel) go global -> LDS directly
// (global_load_lds_dwordx4), double buffered.  K~ arrives multiplied by
// scale * log2(e), so scores are in exp2 units.
//
// Softmax reference.  Cauchy-Schwarz bounds every score of a row by
// m = |q| * max_k |k~| (max over the head's keys, computed by the K~
// producer), so with acc = k~.q - m the probabilities exp2(acc) never exceed
// 1: no running max, no cross-lane max and no rescaling in the key loop.  The
// bound enters the MFMA as its initial accumulator.  If a row's sum ends
// below 2^-60 (scores far below the bound: large norms) the unit is queued
// and recomputed by the exact kernel below, which tracks the running max.
//
// Layouts.  S^T tile (16 keys x 16 queries): lane l holds query l%16 and
// tile rows 4g..4g+3 (g = l/16).  The K~ rows of the two S tiles of a 32-key
// chunk are permuted so that lane group g holds keys 8g..8g+7 of the chunk:
// exactly the B operand of the P V MFMA, whose V~^T operand is then one
// 16-byte LDS read.  The row sum adds the bf16-rounded probabilities that the
// P V product uses, on the MFMA pipe (a constant all-ones operand row).
//
// Key split.  The keys of every query tile are split in S contiguous ranges;
// each range writes its fp32 partial O, row sum and reference, and a
// finalize kernel combines them in split order (deterministic).  With S = 1
// the unit writes normalized rows.
//
// Schedule.  Query tiles are dealt to the 8 XCDs in contiguous ranges (the
// hardware hands workgroup ids to the XCDs round-robin); each XCD runs its
// tiles split-major, so the workgroups resident at one time sweep the same
// key range.  An XCD whose S-split workgroups would end in a partly filled
// round gives its last (tiles mod tiles-per-round) tiles 2S shorter splits:
// the final round then holds half-length workgroups.
#include "attn_common.h"

namespace httm {

namespace {

// Unit u -> (head, first packed row of the head, head length, query tile,
// key split); units of one head are ordered split-major so that concurrent
// units share key tiles.
__device__ __forceinline__ bool locate(const AttnArgs& a, int u, int rows, Unit& o) {
  int acc = 0;
  o.cu = 0;
  for (int h = 0; h < a.heads; ++h) {
    const int len = a.lenq ? a.lenq[h] : a.lq_uniform;
    const int nt = ceil_div(len, rows);
    const int nu = nt * a.split;
    if (u < acc + nu) {
      const int j = u - acc;
      o.head = h;
      o.L = len;
      o.split = j / nt;
      o.tile = j % nt;
      return true;
    }
    acc += nu;
    o.cu += len;
  }
  return false;
}

// Shared state of one unit: operands, loaders, output.
struct UnitCtx {
  const uint16_t* Kp;
  const uint16_t* Vp;
  uint32_t kbytes, vbytes;  // sizes of the head's K~ rows and V~^T rows (buffer bounds)
  int t0, t1, ntiles_all, lk;  // key tiles of this unit, of the head; keys of the head
  uint32_t koff[8 / kNW], voff[8 / kNW];  // per-lane byte offsets of the tile copies
  bf16x8 bq[kQT][2];
  int qrow0, L;  // this lane's row of query tile 0 inside the head; head length
  __device__ __forceinline__ bool valid(int qt) const { return qrow0 + qt * 16 < L; }
};

__device__ __forceinline__ void unit_setup(const AttnArgs& a, const Unit& u, int wave, int g, int l16, UnitCtx& c,
                                           float* qnorm2) {
  const uint16_t* Qp = reinterpret_cast<const uint16_t*>(a.q);
  c.Kp = uniform_ptr(reinterpret_cast<const uint16_t*>(a.k) + (size_t)u.head * a.k_rows * kD);
  c.Vp = uniform_ptr(reinterpret_cast<const uint16_t*>(a.vt) + (size_t)u.head * kD * a.vt_pitch);
  c.kbytes = (uint32_t)a.k_rows * (kD * 2);
  c.vbytes = (uint32_t)kD * a.vt_pitch * 2;
  c.lk = __builtin_amdgcn_readfirstlane(a.lenk ? a.lenk[u.head] : a.lk);
  c.ntiles_all = ceil_div(c.lk, kKeyTile);
  // the copy of key tile t reads tile offset(t) + these lane offsets: every
  // key buffer holds whole 64-key tiles (zero past lk), so no clamp is needed
#pragma unroll
  for (int rd = 0; rd < 8 / kNW; ++rd) {
    const int p = (rd * kNW + wave) * 64 + (threadIdx.x & 63);
    const int row = p >> 3, pc = p & 7;
    c.koff[rd] = (uint32_t)(row * kD + (pc ^ swzK(row)) * 8) * 2u;
    c.voff[rd] = (uint32_t)(row * a.vt_pitch + (pc ^ swzV(row)) * 8) * 2u;
  }
  c.t0 = __builtin_amdgcn_readfirstlane((int)((int64_t)u.split * c.ntiles_all / u.nsplit));
  c.t1 = __builtin_amdgcn_readfirstlane((int)((int64_t)(u.split + 1) * c.ntiles_all / u.nsplit));
  c.qrow0 = u.tile * kRows + wave * kQT * 16 + l16;
  c.L = u.L;
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qr = c.qrow0 + qt * 16;
    const size_t r = (size_t)u.cu + (qr < u.L ? qr : u.L - 1);
    float ss = 0.f;
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(Qp + r * kD + dc * 32 + g * 8);
      c.bq[qt][dc] = __builtin_bit_cast(bf16x8, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(v[e] << 16), hi = __uint_as_float(v[e] & 0xFFFF0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
    qnorm2[qt] = sum_xor16(sum_xor32(ss));
  }
}

// Copy key tile t (64 keys of K~ and V~^T) into LDS buffer buf.  Each wave
// issues 8/kNW + 8/kNW copies of 64 x 16 bytes; lane i fetches the global
// chunk that belongs at its swizzled LDS slot (offsets fixed per lane).
__device__ __forceinline__ void load_tile(const UnitCtx& c, u32x4* sKb, u32x4* sVb, int t, int wave) {
  const uint32_t ks = (uint32_t)t * (kKeyTile * kD * 2), vs = (uint32_t)t * (kKeyTile * 2);
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(c.Kp, c.kbytes), rv = buffer_rsrc(c.Vp, c.vbytes);
#pragma unroll
  for (int rd = 0; rd < 8 / kNW; ++rd) {
    const int slot = (rd * kNW + wave) * 64;
    lds_copy16_buf(rk, c.koff[rd], ks, sKb + slot);
    lds_copy16_buf(rv, c.voff[rd], vs, sVb + slot);
  }
}

// S^T - m for one 64-key tile: sacc[qt][kt], kt = 2*kc + p holds keys
// 32kc + 8g + 4p + r in register r of lane group g.
__device__ __forceinline__ void scores(const u32x4* sKb, const UnitCtx& c, const f32x4* negm, int g, int l16,
                                       f32x4 (*sacc)[4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int row = 32 * (kt >> 1) + 8 * (l16 >> 2) + 4 * (kt & 1) + (l16 & 3);
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, sKb[row * 8 + ((4 * dc + g) ^ swzK(row))]);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt)
        sacc[qt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, c.bq[qt][dc], dc == 0 ? negm[qt] : sacc[qt][kt],
                                                                 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void mask_tail(int lk, int t, int g, f32x4 (*sacc)[4]) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (t * kKeyTile + 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + r >= lk) {
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) sacc[qt][kt][r] = -INFINITY;
      }
}

// p = exp2(acc) as bf16 B operands, and the running row sum of those values.
__device__ __forceinline__ void probs(f32x4 (*sacc)[4], bf16x8 (*bp)[2], float* lrun) {
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    float ls0 = lrun[qt], ls1 = 0.f;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8 pb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pb[r] = (__bf16)__builtin_amdgcn_exp2f(sacc[qt][2 * kc][r]);
        pb[4 + r] = (__bf16)__builtin_amdgcn_exp2f(sacc[qt][2 * kc + 1][r]);
      }
      bp[qt][kc] = pb;
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        const bf16x2 p0 = {pb[e], pb[e + 1]}, p1 = {pb[e + 2], pb[e + 3]};
        ls0 = __builtin_amdgcn_fdot2_f32_bf16(p0, one2, ls0, false);
        ls1 = __builtin_amdgcn_fdot2_f32_bf16(p1, one2, ls1, false);
      }
    }
    lrun[qt] = ls0 + ls1;
  }
}

// O^T += V~^T P^T for one 64-key tile.
__device__ __forceinline__ void pv(const u32x4* sVb, bf16x8 (*bp)[2], int g, int l16, f32x4 (*oacc)[4]) {
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int vrow = dt * 16 + l16;
      const bf16x8 vb = __builtin_bit_cast(bf16x8, sVb[vrow * 8 + ((4 * kc + g) ^ swzV(vrow))]);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt)
        oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, bp[qt][kc], oacc[qt][dt], 0, 0, 0);
    }
  }
}

// Key half h of a tile (keys 32h .. 32h + 31: kt = 2h, 2h + 1).
__device__ __forceinline__ void scores_half(const u32x4* sKb, const UnitCtx& c, const f32x4* negm, int g, int l16,
                                            int h, f32x4 (*sacc)[4]) {
#pragma unroll
  for (int kt = 2 * h; kt < 2 * h + 2; ++kt) {
    const int row = 32 * (kt >> 1) + 8 * (l16 >> 2) + 4 * (kt & 1) + (l16 & 3);
#pragma unroll
    for (int dc = 0; dc < 2; ++dc) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, sKb[row * 8 + ((4 * dc + g) ^ swzK(row))]);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt)
        sacc[qt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, c.bq[qt][dc], dc == 0 ? negm[qt] : sacc[qt][kt],
                                                                 0, 0, 0);
    }
  }
}
__device__ __forceinline__ void mask_half(int lk, int t, int g, int h, f32x4 (*sacc)[4]) {
#pragma unroll
  for (int kt = 2 * h; kt < 2 * h + 2; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (t * kKeyTile + 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + r >= lk) {
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) sacc[qt][kt][r] = -INFINITY;
      }
}
__device__ __forceinline__ void probs_half(f32x4 (*sacc)[4], bf16x8 (*bp)[2], int kc) {
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    bf16x8 pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pb[r] = (__bf16)__builtin_amdgcn_exp2f(sacc[qt][2 * kc][r]);
      pb[4 + r] = (__bf16)__builtin_amdgcn_exp2f(sacc[qt][2 * kc + 1][r]);
    }
    bp[qt][kc] = pb;
  }
}
__device__ __forceinline__ void pv_half(const u32x4* sVb, bf16x8 (*bp)[2], int g, int l16, int kc,
                                        f32x4 (*oacc)[4]) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int vrow = dt * 16 + l16;
    const bf16x8 vb = __builtin_bit_cast(bf16x8, sVb[vrow * 8 + ((4 * kc + g) ^ swzV(vrow))]);
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt)
      oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, bp[qt][kc], oacc[qt][dt], 0, 0, 0);
  }
}
__device__ __forceinline__ void psum_half(const bf16x8 ones, bf16x8 (*bp)[2], int kc, f32x4* osum) {
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt)
    osum[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bp[qt][kc], osum[qt], 0, 0, 0);
}

// One 64-key tile in key halves, so that the exp2 of one half runs between
// the MFMAs of the other: S(0) | S(1) + P(0) | PV(0) + P(1) | PV(1).  The
// scheduling groups ask for one MFMA (mask 0x008) then 3 or 2 VALU
// instructions (mask 0x002) in turn; left alone, the compiler clusters the
// exp2s and the MFMAs (measured 1.3 % slower at 30 and 100 frames).
template <bool MASK>
__device__ __forceinline__ void tile_step(const AttnArgs& a, const u32x4* sKb, const u32x4* sVb, const UnitCtx& c,
                                          const f32x4* negm, int g, int l16, int t, const bf16x8 ones,
                                          f32x4* osum, f32x4 (*oacc)[4]) {
  f32x4 sacc[kQT][4];
  bf16x8 bp[kQT][2];
  scores_half(sKb, c, negm, g, l16, 0, sacc);
  __builtin_amdgcn_sched_barrier(0);
  scores_half(sKb, c, negm, g, l16, 1, sacc);
  if (MASK) mask_half(c.lk, t, g, 0, sacc);
  probs_half(sacc, bp, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (MASK) mask_half(c.lk, t, g, 1, sacc);
  pv_half(sVb, bp, g, l16, 0, oacc);
  psum_half(ones, bp, 0, osum);
  probs_half(sacc, bp, 1);
#pragma unroll
  for (int i = 0; i < 20; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 1);
  }
  __builtin_amdgcn_sched_barrier(0);
  pv_half(sVb, bp, g, l16, 1, oacc);
  psum_half(ones, bp, 1, osum);
}

// Write one unit's rows (reference -negm per query tile).
__device__ __forceinline__ void store_unit(const AttnArgs& a, const Unit& u, const UnitCtx& c, int g,
                                           f32x4 (*oacc)[4], const float* lsum, const f32x4* negm) {
  float mref[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) mref[qt] = -negm[qt][0];
  store_rows(a, u, c.qrow0, c.L, g, oacc, lsum, mref);
}

// Fast path: the Cauchy-Schwarz reference, no running max.
__global__ __launch_bounds__(kNW * 64, 2) void attn_fast(AttnArgs a) {
  // the two tile buffers are separate LDS objects, so the compiler can see
  // that reads of one do not wait for the direct-to-LDS copies into the other
  __shared__ u32x4 sK0[kKeyTile * 8], sK1[kKeyTile * 8];
  __shared__ u32x4 sV0[kD * 8], sV1[kD * 8];
  const int w = blockIdx.x;
  Unit u;
  if (!schedule(a, w, u)) return;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  UnitCtx c;
  float qn2[kQT];
  unit_setup(a, u, wave, g, l16, c, qn2);
  const float km = a.kmax[u.head];
  f32x4 negm[kQT], osum[kQT];
  f32x4 oacc[kQT][4];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const float m = sqrtf(qn2[qt]) * km;
    osum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) negm[qt][r] = -m;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (c.t0 == c.t1) {
    // a head with fewer key tiles than splits: this split adds nothing (l = 0,
    // skipped by the combine); no tile load is left in flight
    float lz[kQT];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) lz[qt] = 0.f;
    store_unit(a, u, c, g, oacc, lz, negm);
    return;
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)(l16 == 0 ? 1.0f : 0.0f);
  load_tile(c, sK0, sV0, c.t0, wave);
  // only the head's last key tile can be partial: it runs outside the main
  // loop, so the loop body is one basic block and the exp2 of one key group
  // can overlap the score MFMAs of the next.  Unrolled by two so that every
  // tile names its buffer statically.
  const int tfull = (c.t1 == c.ntiles_all && c.lk % kKeyTile) ? c.t1 - 1 : c.t1;
  auto step = [&](int t, const u32x4* sKc, const u32x4* sVc, u32x4* sKn, u32x4* sVn) {
    __builtin_amdgcn_sched_barrier(0);  // the previous tile's work stays before the wait
    wait_vm();
    __syncthreads();
    if (t + 1 < c.t1) load_tile(c, sKn, sVn, t + 1, wave);
    tile_step<false>(a, sKc, sVc, c, negm, g, l16, t, ones, osum, oacc);
  };
  int t = c.t0;
  for (; t + 1 < tfull; t += 2) {
    step(t, sK0, sV0, sK1, sV1);
    step(t + 1, sK1, sV1, sK0, sV0);
  }
  if (t < tfull) {
    step(t, sK0, sV0, sK1, sV1);
    ++t;
  }
  if (t < c.t1) {
    // the partial tile sits in buffer (t - t0) & 1
    __builtin_amdgcn_sched_barrier(0);
    wait_vm();
    __syncthreads();
    if ((t - c.t0) & 1)
      tile_step<true>(a, sK1, sV1, c, negm, g, l16, t, ones, osum, oacc);
    else
      tile_step<true>(a, sK0, sV0, c, negm, g, l16, t, ones, osum, oacc);
  }
  float lsum[kQT];
  bool tiny = false;
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    lsum[qt] = __shfl(osum[qt][0], l16);  // from lane group 0
    tiny |= c.valid(qt) && !(lsum[qt] >= kTinySum);
  }
  if (__syncthreads_or(tiny)) {
    if (tid == 0) {
      const int slot = atomicAdd(a.fb_count, 1);
      a.fb_list[slot] = w;
    }
    return;
  }
  store_unit(a, u, c, g, oacc, lsum, negm);
}

// Exact path for queued units: online max (raised only when a score exceeds
// it by more than 8 in log2 units; the final division makes it exact).
// A small grid strides over the queue (usually empty).
constexpr int kExactGrid = 512;
__device__ __forceinline__ void exact_unit(const AttnArgs& a, int w, u32x4 (*sK)[kKeyTile * 8],
                                           u32x4 (*sV)[kD * 8]) {
  Unit u;
  if (!schedule(a, w, u)) return;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  UnitCtx c;
  float qn2[kQT];
  unit_setup(a, u, wave, g, l16, c, qn2);
  f32x4 negm[kQT];
  float mref[kQT], lrun[kQT];
  f32x4 oacc[kQT][4];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    mref[qt] = 0.f;
    lrun[qt] = 0.f;
    negm[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  load_tile(c, sK[0], sV[0], c.t0, wave);
  for (int t = c.t0; t < c.t1; ++t) {
    const int buf = (t - c.t0) & 1;
    wait_vm();
    __syncthreads();
    if (t + 1 < c.t1) load_tile(c, sK[buf ^ 1], sV[buf ^ 1], t + 1, wave);
    f32x4 sacc[kQT][4];
    scores(sK[buf], c, negm, g, l16, sacc);
    if ((t + 1) * kKeyTile > c.lk) mask_tail(c.lk, t, g, sacc);
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      const f32x4* sa = sacc[qt];
      const float m0 = max3(sa[0][0], sa[0][1], sa[0][2]), m1 = max3(sa[0][3], sa[1][0], sa[1][1]);
      const float m2 = max3(sa[1][2], sa[1][3], sa[2][0]), m3 = max3(sa[2][1], sa[2][2], sa[2][3]);
      const float m4 = max3(sa[3][0], sa[3][1], sa[3][2]);
      float mx = fmaxf(max3(m0, m1, m2), max3(m3, m4, sa[3][3]));
      mx = max_xor16(max_xor32(mx));
      const bool first = (t == c.t0);
      const bool grow = first || mx > 8.0f;
      if (__any(grow)) {
        float shift = 0.f;
        if (grow) {
          shift = mx;
          mref[qt] += mx;
#pragma unroll
          for (int r = 0; r < 4; ++r) negm[qt][r] = -mref[qt];
        }
        if (!first) {
          const float alpha = __builtin_amdgcn_exp2f(-shift);
          lrun[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[qt][dt][r] *= alpha;
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sacc[qt][kt][r] -= shift;
      }
    }
    bf16x8 bp[kQT][2];
    probs(sacc, bp, lrun);
    pv(sV[buf], bp, g, l16, oacc);
  }
  float lsum[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) lsum[qt] = sum_xor16(sum_xor32(lrun[qt]));
  store_unit(a, u, c, g, oacc, lsum, negm);
}

__global__ __launch_bounds__(kNW * 64) void attn_exact(AttnArgs a) {
  __shared__ u32x4 sK[2][kKeyTile * 8];
  __shared__ u32x4 sV[2][kD * 8];
  const int n = *a.fb_count;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    __syncthreads();  // the previous unit's waves are done with the key buffers
    exact_unit(a, a.fb_list[i], sK, sV);
  }
}

// Combine the key-split partials of every packed row (split order fixed):
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M = max_s m_s over the
// splits with l_s > 0 (an empty key range carries no weight).  A row's split
// count and partial slots follow from the schedule of its query tile.  Every
// load of a row (row sums, references and partial rows of all its splits) is
// issued before the first use.
constexpr int kMaxSplit = 8;
__global__ __launch_bounds__(256) void attn_finalize(AttnArgs a) {
  __shared__ int sCu[kMaxHeads + 1], sUt[kMaxHeads + 1];
  __shared__ int sU0[8], sNr[8];
  if (threadIdx.x < 64) {
    const HeadPrefix hp = head_prefix(a.lenq, a.lq_uniform, a.heads, kRows);
    if ((int)threadIdx.x < a.heads) {
      sCu[threadIdx.x] = hp.rows_before;
      sUt[threadIdx.x] = hp.tiles_before;
    }
    if (threadIdx.x == 0) {
      sCu[a.heads] = hp.rows_total;
      sUt[a.heads] = hp.tiles_total;
    }
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const XcdShare sh = xcd_share(a, sUt[a.heads], threadIdx.x);
    sU0[threadIdx.x] = sh.u0;
    sNr[threadIdx.x] = sh.nr;
  }
  __syncthreads();
  const int64_t R = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  if (R >= sCu[a.heads]) return;
  int h = 0;
  while (sCu[h + 1] <= R) ++h;
  const int rin = (int)(R - sCu[h]), tile = rin / kRows;
  const int ug = sUt[h] + tile;
  int x = 7;
  while (sU0[x] > ug) --x;  // the XCD whose tile range holds ug
  int ns = a.split, tord = -1;
  if (ug >= sU0[x] + sNr[x]) {
    ns = a.tail_split;
    tord = x * kMaxTailTiles + (ug - sU0[x] - sNr[x]);
  }
  float l[kMaxSplit], m[kMaxSplit];
  f32x4 x0[kMaxSplit], x1[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    if (s < ns) {
      const size_t pr = part_row(a, s, (size_t)R, tord, rin - tile * kRows);
      l[s] = a.lpart[pr];
      m[s] = a.mpart[pr];
      const f32x4* src = reinterpret_cast<const f32x4*>(a.opart + pr * kD + part * 8);
      x0[s] = src[0];
      x1[s] = src[1];
    } else {
      l[s] = 0.f;
      m[s] = 0.f;
      x0[s] = x1[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (l[s] > 0.f) M = fmaxf(M, m[s]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, lt = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    if (!(l[s] > 0.f)) continue;
    const float f = __builtin_amdgcn_exp2f(m[s] - M);
    lt = fmaf(f, l[s], lt);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = fmaf(f, x0[s][e], acc[e]);
      acc[4 + e] = fmaf(f, x1[s][e], acc[4 + e]);
    }
  }
  const float inv = 1.0f / lt;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  Row8<uint16_t>::store(reinterpret_cast<uint16_t*>(a.o) + R * kD + part * 8, acc);
}


// fp32 inputs: one thread per query row, key tiles staged in LDS, fp32
// online softmax.  For fp32 layers (small correctness workloads).
__global__ __launch_bounds__(kRowsF32) void attn_f32(AttnArgs a) {
  __shared__ float sK[kKeyTile][kD + 1];
  __shared__ float sV[kD][kKeyTile + 1];
  Unit u;
  if (!locate(a, blockIdx.x, kRowsF32, u)) return;
  const int head = u.head, cu = u.cu, L = u.L, tile = u.tile;
  const int lk = a.lenk ? a.lenk[head] : a.lk;
  const float* Qp = reinterpret_cast<const float*>(a.q);
  const float* Kp = reinterpret_cast<const float*>(a.k) + (size_t)head * a.k_rows * kD;
  const float* Vp = reinterpret_cast<const float*>(a.vt) + (size_t)head * kD * a.vt_pitch;
  const int qr = tile * kRowsF32 + threadIdx.x;
  const bool valid = qr < L;
  const size_t qrow = (size_t)cu + (valid ? qr : L - 1);
  float qv[kD], acc[kD];
  for (int c = 0; c < kD; ++c) {
    qv[c] = Qp[qrow * kD + c];
    acc[c] = 0.f;
  }
  float mrun = -INFINITY, lrun = 0.f;
  for (int t0 = 0; t0 < lk; t0 += kKeyTile) {
    __syncthreads();
    for (int e = threadIdx.x; e < kKeyTile * kD; e += blockDim.x) {
      const int r = e / kD, c = e % kD;
      const int key = t0 + r < lk ? t0 + r : lk - 1;
      sK[r][c] = Kp[(size_t)key * kD + c];
      sV[e / kKeyTile][e % kKeyTile] = Vp[(size_t)(e / kKeyTile) * a.vt_pitch + t0 + e % kKeyTile];
    }
    __syncthreads();
    const int nt = min(kKeyTile, lk - t0);
    for (int r = 0; r < nt; ++r) {
      float s = 0.f;
      for (int c = 0; c < kD; ++c) s = fmaf(qv[c], sK[r][c], s);  // K~ carries scale*log2 e
      const float mnew = fmaxf(mrun, s);
      const float alpha = exp2f(mrun - mnew);
      const float p = exp2f(s - mnew);
      lrun = lrun * alpha + p;
      for (int c = 0; c < kD; ++c) acc[c] = fmaf(acc[c], alpha, p * sV[c][r]);
      mrun = mnew;
    }
  }
  if (valid) {
    float* Op = reinterpret_cast<float*>(a.o) + ((size_t)cu + qr) * kD;
    for (int c = 0; c < kD; ++c) Op[c] = acc[c] / lrun;
  }
}

}  // namespace

int attention_rows_per_unit() { return kRows; }

static_assert(kMaxSplit >= 8, "attention_split and its tail splits stay within kMaxSplit");
int attention_split(int64_t q_capacity, int heads) {
  // Four key splits: at 30 frames they fill the GPU (540 units of 256 rows
  // for 512 resident workgroups), and at 100-500 frames four shorter key
  // sweeps per unit keep concurrent workgroups on nearby keys (better L2
  // reuse of K~ / V~^T); measured best or within 1 % of best at every size.
  (void)q_capacity;
  (void)heads;
  return 4;
}

AttnTail attention_tail(int split) {
  // host-only: capacities use the bound of kMaxTailTiles tail tiles per XCD;
  // the device's tiles per round is read at launch (per_round_for)
  AttnTail t{split, 0, 0};
  if (split <= 1 || 2 * split > kMaxSplit) return t;
  t.tail_split = 2 * split;
  t.tail_rows = (int64_t)8 * kMaxTailTiles * kRows;
  return t;
}


int64_t attention_workgroups(int dtype, const AttnShape& s) {
  if (dtype != 1) return (s.q_capacity + kRowsF32 - 1) / kRowsF32 + s.heads;
  const int64_t units = (s.q_capacity + kRows - 1) / kRows + s.heads;
  const int64_t nmax = (units + 7) / 8;
  int64_t per_xcd = s.split * nmax;
  if (s.tail_split > s.split) {
    // tail tiles per XCD: fewer than a round's worth, at most kMaxTailTiles
    const int64_t cap = s.per_round > 0 ? s.per_round - 1 : kMaxTailTiles;
    const int64_t t = nmax < cap ? nmax : cap;
    per_xcd += (int64_t)(s.tail_split - s.split) * t;
  }
  return 8 * per_xcd;
}

int64_t attention_partial_rows(const AttnShape& s) {
  return (int64_t)s.split * s.q_capacity + (int64_t)(s.tail_split > s.split ? s.tail_split - s.split : 0) * s.tail_rows;
}


hipError_t launch_attention(int dtype, const AttnShape& s, const void* q, const void* k,
                            const void* vt, const int32_t* lenq, void* o, hipStream_t stream) {
  if (dtype == 1 && s.k8) return launch_attention_fp8(s, q, vt, lenq, o, stream);
  const AttnArgs a = make_attn_args(dtype, s, q, k, vt, lenq, o, per_round_for<attn_fast>);
  if (dtype == 1) {
    hipLaunchKernelGGL(attn_fast, dim3(a.total_wg), dim3(kNW * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL(attn_f32, dim3(a.total_wg), dim3(kRowsF32), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_attention_tail(int dtype, const AttnShape& s, const void* q, const void* k,
                                 const void* vt, const int32_t* lenq, void* o, hipStream_t stream) {
  if (dtype != 1) return hipSuccess;
  hipError_t e;
  AttnArgs a{};
  if (s.k8) {
    e = launch_attention_fp8_exact(s, q, vt, lenq, o, stream);
    a = make_attn_args(dtype, s, q, k, vt, lenq, o, attention_fp8_per_round);
  } else {
    a = make_attn_args(dtype, s, q, k, vt, lenq, o, per_round_for<attn_fast>);
    hipLaunchKernelGGL(attn_exact, dim3(a.total_wg < kExactGrid ? a.total_wg : kExactGrid), dim3(kNW * 64), 0,
                       stream, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess || a.split == 1) return e;
  const int fgrid = (int)((s.q_capacity + 31) / 32);
  hipLaunchKernelGGL(attn_finalize, dim3(fgrid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace httm
