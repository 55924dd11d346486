// Ragged attention with FP8 (OCP e4m3) scores.
//
// "LiteVGGT: Boosting Vanilla VGGT via Geometry-aware Cached Token Merging",
// training strategy and ablations: the page runs inference with FP8
// quantisation (through NVIDIA's Transformer Engine).  This is our own
// gfx950 variant for the score product of the HTTM layer's attention: the
// merged queries and keys are e4m3, the probabilities and merged values stay
// bf16, every sum is fp32.
//
// Scales.  Every merged query row and every head's key matrix carries a
// power-of-two scale that puts its largest magnitude in [128, 256); values
// are rounded to nearest-even e4m3 (v_cvt_pk_fp8_f32).  The scales enter the
// score MFMA as its per-lane E8M0 operands, so the product comes out
// unscaled: no VALU work per score.
//
// Score tile.  S^T (32 keys x 32 queries) = K8 Q8^T on
// v_mfma_scale_f32_32x32x64_f8f6f4: one instruction covers d = 64 at twice
// the bf16 rate.  A-operand row m holds key sigma(m) of the 32-key block, so
// that output lane l (query l % 32, half h = l / 32) holds keys 16h .. 16h+15
// in accumulator order.  The bf16 probabilities of 8 consecutive keys form
// one dword quad; one v_permlane16_swap per dword moves them into the B
// operand of v_mfma_f32_16x16x32_bf16 (query l % 16, keys 8g .. 8g+7 of the
// block, g = l / 16), whose V~^T operand is one 16-byte LDS read.  The row sum
// uses those operands against a constant all-ones row (as in the bf16
// kernel), and the output O^T tiles, key splits, combine and unmerge are the
// bf16 kernel's.
//
// Reference: the Cauchy-Schwarz bound m = |q| max|k~| of the bf16 operands
// (an FP8 score can exceed it by a few percent of m: exp2 stays finite).  A
// unit whose row sum underflows (2^-60) is queued for the exact kernel below
// (online max), like the bf16 path.
#include "attn_common.h"

namespace httm {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// fp8 key tile in LDS: 64 rows of 64 bytes (four 16-byte chunks); chunk c of
// row r sits at chunk c ^ swz8(r).  A score operand read touches rows
// sigma(0..15) (or sigma(16..31)) of a block at one chunk: swz8 gives rows of
// equal (r mod 4) distinct chunks, so the 16 lanes of a read hit 16 distinct
// bank quads.
__device__ __forceinline__ int swz8(int r) { return ((r >> 2) & 1) | ((r >> 3) & 2); }
__device__ __forceinline__ int sigma(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// Power-of-two scale exponent of a block with largest magnitude amax: amax *
// 2^e in [128, 256), clamped to [-127, 127]; 0 for an all-zero block.
__device__ __forceinline__ int fp8_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const int e = 8 - __builtin_amdgcn_frexp_expf(amax);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four values (already scaled) -> four e4m3 bytes, nearest-even.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

struct Ctx8 {
  const uint8_t* K8;
  const uint16_t* Vp;
  uint32_t kbytes, vbytes;  // sizes of the head's e4m3 key rows and V~^T rows (buffer bounds)
  int t0, t1, ntiles_all, lk;
  uint32_t koff, voff[2];  // per-lane byte offsets of the tile copies
  i32x8 bq[2];             // fp8 query operands of the wave's two 32-query blocks
  int qs[2];               // E8M0 scale of this lane's query in each block
  float negm[2];           // -reference of this lane's query in each block (score layout)
  int ks;                  // E8M0 scale of the head's keys
  int qrow0, L;            // output layout: this lane's row of query tile 0; head length
};

// Unit setup: tile copy offsets, and the wave's 64 query rows quantised in
// the score layout (lane l: query 32 qb + l % 32, channels 16h..16h+15 and
// 32+16h..32+16h+15, h = l / 32).  Split 0 of a unit also writes the codes
// and exponents (a.q8 / a.qexp) for inspection.
__device__ __forceinline__ void setup8(const AttnArgs& a, const Unit& u, int wave, int lane, Ctx8& c) {
  const uint16_t* Qp = reinterpret_cast<const uint16_t*>(a.q);
  c.K8 = uniform_ptr(a.k8 + (size_t)u.head * a.k_rows * kD);
  c.Vp = uniform_ptr(reinterpret_cast<const uint16_t*>(a.vt) + (size_t)u.head * kD * a.vt_pitch);
  c.kbytes = (uint32_t)a.k_rows * kD;
  c.vbytes = (uint32_t)kD * a.vt_pitch * 2;
  c.lk = __builtin_amdgcn_readfirstlane(a.lenk ? a.lenk[u.head] : a.lk);
  c.ntiles_all = ceil_div(c.lk, kKeyTile);
  {
    // key tile: 256 slots of 16 bytes, one per lane of the workgroup
    const int p = wave * 64 + lane;
    const int row = p >> 2, pc = p & 3;
    c.koff = (uint32_t)(row * kD + (pc ^ swz8(row)) * 16);
  }
#pragma unroll
  for (int rd = 0; rd < 8 / kNW; ++rd) {
    const int p = (rd * kNW + wave) * 64 + lane;
    const int row = p >> 3, pc = p & 7;
    c.voff[rd] = (uint32_t)(row * a.vt_pitch + (pc ^ swzV(row)) * 8) * 2u;
  }
  c.t0 = __builtin_amdgcn_readfirstlane((int)((int64_t)u.split * c.ntiles_all / u.nsplit));
  c.t1 = __builtin_amdgcn_readfirstlane((int)((int64_t)(u.split + 1) * c.ntiles_all / u.nsplit));
  c.qrow0 = u.tile * kRows + wave * kQT * 16 + (lane & 15);
  c.L = u.L;
  c.ks = 127 - a.kexp[u.head];
  const float km = a.kmax[u.head];
  const int h = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = u.tile * kRows + wave * kQT * 16 + 32 * qb + (lane & 31);
    const size_t r = (size_t)u.cu + (qr < u.L ? qr : u.L - 1);
    float x[32];
#pragma unroll
    for (int part = 0; part < 2; ++part) {
#pragma unroll
      for (int hv = 0; hv < 2; ++hv) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(Qp + r * kD + 32 * part + 16 * h + 8 * hv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[16 * part + 8 * hv + 2 * e] = __uint_as_float(v[e] << 16);
          x[16 * part + 8 * hv + 2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
        }
      }
    }
    float amax = 0.f, ss = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      amax = fmaxf(amax, fabsf(x[i]));
      ss = fmaf(x[i], x[i], ss);
    }
    amax = max_xor32(amax);
    ss = sum_xor32(ss);
    const int e = fp8_exponent(amax);
    c.qs[qb] = 127 - e;
    c.negm[qb] = -(sqrtf(ss) * km);
#pragma unroll
    for (int w = 0; w < 8; ++w)
      c.bq[qb][w] = (int)pack_fp8x4(ldexpf(x[4 * w], e), ldexpf(x[4 * w + 1], e), ldexpf(x[4 * w + 2], e),
                                    ldexpf(x[4 * w + 3], e));
    if (a.q8 && u.split == 0 && qr < u.L) {
      uint8_t* dst = a.q8 + ((size_t)u.cu + qr) * kD;
      *reinterpret_cast<u32x4*>(dst + 16 * h) = u32x4{(uint32_t)c.bq[qb][0], (uint32_t)c.bq[qb][1],
                                                      (uint32_t)c.bq[qb][2], (uint32_t)c.bq[qb][3]};
      *reinterpret_cast<u32x4*>(dst + 32 + 16 * h) = u32x4{(uint32_t)c.bq[qb][4], (uint32_t)c.bq[qb][5],
                                                           (uint32_t)c.bq[qb][6], (uint32_t)c.bq[qb][7]};
      if (h == 0) a.qexp[(size_t)u.cu + qr] = e;
    }
  }
}

__device__ __forceinline__ void load_tile8(const Ctx8& c, u32x4* sKb, u32x4* sVb, int t, int wave) {
  const uint32_t ks = (uint32_t)t * (kKeyTile * kD), vs = (uint32_t)t * (kKeyTile * 2);
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(c.K8, c.kbytes), rv = buffer_rsrc(c.Vp, c.vbytes);
  lds_copy16_buf(rk, c.koff, ks, sKb + wave * 64);
#pragma unroll
  for (int rd = 0; rd < 8 / kNW; ++rd) lds_copy16_buf(rv, c.voff[rd], vs, sVb + (rd * kNW + wave) * 64);
}

// Scores of key block kb for both query blocks: s[qb] = S^T - m (lane l:
// query 32 qb + l % 32; accumulator r: key 32 kb + 16 h + r).
__device__ __forceinline__ void scores8(const u32x4* sKb, const Ctx8& c, int kb, int l32, int h, f32x16* s,
                                        const float* negm) {
  const int row = 32 * kb + sigma(l32);
  const u32x4 lo = sKb[row * 4 + (h ^ swz8(row))];
  const u32x4 hi = sKb[row * 4 + ((2 + h) ^ swz8(row))];
  const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    f32x16 init;
#pragma unroll
    for (int r = 0; r < 16; ++r) init[r] = negm[qb];
    s[qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, c.bq[qb], init, 0, 0, 0, c.ks, 0, c.qs[qb]);
  }
}

__device__ __forceinline__ void mask8(int lk, int t, int kb, int h, f32x16* s) {
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (t * kKeyTile + 32 * kb + 16 * h + r >= lk) {
      s[0][r] = -INFINITY;
      s[1][r] = -INFINITY;
    }
}

// exp2 of a score block pair -> the B operands of query tiles 2 qb and
// 2 qb + 1 for this key block.
__device__ __forceinline__ void probs8(const f32x16* s, bf16x8 (*bp)[2], int kb) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    u32x4 x, y;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      x[d] = pack_bf16_trunc(__builtin_amdgcn_exp2f(s[qb][2 * d]), __builtin_amdgcn_exp2f(s[qb][2 * d + 1]));
      y[d] = pack_bf16_trunc(__builtin_amdgcn_exp2f(s[qb][8 + 2 * d]), __builtin_amdgcn_exp2f(s[qb][9 + 2 * d]));
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto r = __builtin_amdgcn_permlane16_swap(x[d], y[d], false, false);
      x[d] = r[0];
      y[d] = r[1];
    }
    bp[2 * qb][kb] = __builtin_bit_cast(bf16x8, x);
    bp[2 * qb + 1][kb] = __builtin_bit_cast(bf16x8, y);
  }
}

__device__ __forceinline__ void pv8(const u32x4* sVb, bf16x8 (*bp)[2], const bf16x8 ones, int g, int l16, int kb,
                                    f32x4 (*oacc)[4], f32x4* osum) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int vrow = dt * 16 + l16;
    const bf16x8 vb = __builtin_bit_cast(bf16x8, sVb[vrow * 8 + ((4 * kb + g) ^ swzV(vrow))]);
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt)
      oacc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, bp[qt][kb], oacc[qt][dt], 0, 0, 0);
  }
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt)
    osum[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bp[qt][kb], osum[qt], 0, 0, 0);
}

// One 64-key tile: S(0) S(1) | P(0) | PV(0) + P(1) | PV(1).
template <bool MASK>
__device__ __forceinline__ void tile8(const u32x4* sKb, const u32x4* sVb, const Ctx8& c, int t, int lane,
                                      const bf16x8 ones, f32x4* osum, f32x4 (*oacc)[4]) {
  const int l32 = lane & 31, h = lane >> 5, g = lane >> 4, l16 = lane & 15;
  f32x16 s0[2], s1[2];
  bf16x8 bp[kQT][2];
  scores8(sKb, c, 0, l32, h, s0, c.negm);
  scores8(sKb, c, 1, l32, h, s1, c.negm);
  if (MASK) {
    mask8(c.lk, t, 0, h, s0);
    mask8(c.lk, t, 1, h, s1);
  }
  probs8(s0, bp, 0);
  __builtin_amdgcn_sched_barrier(0);
  pv8(sVb, bp, ones, g, l16, 0, oacc, osum);
  probs8(s1, bp, 1);
#pragma unroll
  for (int i = 0; i < 20; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  pv8(sVb, bp, ones, g, l16, 1, oacc, osum);
}

// Reference of each output-layout query tile (lane: query 16 qt + l16) from
// the score layout (lane 16 w + l16 of block qb holds query 32 qb + 16 w + l16).
__device__ __forceinline__ void out_refs(const float* v, int l16, float* o) {
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) o[qt] = __shfl(v[qt >> 1], 16 * (qt & 1) + l16);
}

__global__ __launch_bounds__(kNW * 64, 2) void attn_fast8(AttnArgs a) {
  __shared__ u32x4 sK0[kKeyTile * 4], sK1[kKeyTile * 4];
  __shared__ u32x4 sV0[kD * 8], sV1[kD * 8];
  const int w = blockIdx.x;
  Unit u;
  if (!schedule(a, w, u)) return;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, l16 = lane & 15;
  Ctx8 c;
  setup8(a, u, wave, lane, c);
  f32x4 osum[kQT];
  f32x4 oacc[kQT][4];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    osum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float mref[kQT];
  {
    const float m[2] = {-c.negm[0], -c.negm[1]};
    out_refs(m, l16, mref);
  }
  if (c.t0 == c.t1) {
    float lz[kQT];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) lz[qt] = 0.f;
    store_rows(a, u, c.qrow0, c.L, g, oacc, lz, mref);
    return;
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)(l16 == 0 ? 1.0f : 0.0f);
  load_tile8(c, sK0, sV0, c.t0, wave);
  const int tfull = (c.t1 == c.ntiles_all && c.lk % kKeyTile) ? c.t1 - 1 : c.t1;
  auto step = [&](int t, const u32x4* sKc, const u32x4* sVc, u32x4* sKn, u32x4* sVn) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm();
    __syncthreads();
    if (t + 1 < c.t1) load_tile8(c, sKn, sVn, t + 1, wave);
    tile8<false>(sKc, sVc, c, t, lane, ones, osum, oacc);
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
    __builtin_amdgcn_sched_barrier(0);
    wait_vm();
    __syncthreads();
    if ((t - c.t0) & 1)
      tile8<true>(sK1, sV1, c, t, lane, ones, osum, oacc);
    else
      tile8<true>(sK0, sV0, c, t, lane, ones, osum, oacc);
  }
  float lsum[kQT];
  bool tiny = false;
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    lsum[qt] = __shfl(osum[qt][0], l16);
    tiny |= (c.qrow0 + qt * 16 < c.L) && !(lsum[qt] >= kTinySum);
  }
  if (__syncthreads_or(tiny)) {
    if (tid == 0) {
      const int slot = atomicAdd(a.fb_count, 1);
      a.fb_list[slot] = w;
    }
    return;
  }
  store_rows(a, u, c.qrow0, c.L, g, oacc, lsum, mref);
}

// Exact path for queued units: per-query running reference, raised only when
// a tile's maximum exceeds it by more than 8 (log2 units); the final division
// makes the result exact.
constexpr int kExactGrid8 = 512;
__device__ __forceinline__ void exact_unit8(const AttnArgs& a, int w, u32x4 (*sK)[kKeyTile * 4],
                                            u32x4 (*sV)[kD * 8]) {
  Unit u;
  if (!schedule(a, w, u)) return;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5, g = lane >> 4, l16 = lane & 15;
  Ctx8 c;
  setup8(a, u, wave, lane, c);
  float ref[2] = {0.f, 0.f};  // score layout: reference of this lane's query per block
  f32x4 osum[kQT];
  f32x4 oacc[kQT][4];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    osum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[qt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)(l16 == 0 ? 1.0f : 0.0f);
  load_tile8(c, sK[0], sV[0], c.t0, wave);
  for (int t = c.t0; t < c.t1; ++t) {
    const int buf = (t - c.t0) & 1;
    wait_vm();
    __syncthreads();
    if (t + 1 < c.t1) load_tile8(c, sK[buf ^ 1], sV[buf ^ 1], t + 1, wave);
    f32x16 s0[2], s1[2];
    const float negr[2] = {-ref[0], -ref[1]};
    scores8(sK[buf], c, 0, l32, h, s0, negr);
    scores8(sK[buf], c, 1, l32, h, s1, negr);
    if ((t + 1) * kKeyTile > c.lk) {
      mask8(c.lk, t, 0, h, s0);
      mask8(c.lk, t, 1, h, s1);
    }
    float shift[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[qb][r], s1[qb][r]));
      mx = max_xor32(mx);
      const bool grow = (t == c.t0) || mx > 8.0f;
      shift[qb] = grow ? mx : 0.f;
      ref[qb] += shift[qb];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[qb][r] -= shift[qb];
        s1[qb][r] -= shift[qb];
      }
    }
    if (t != c.t0) {
      float sh[kQT];
      out_refs(shift, l16, sh);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) {
        const float alpha = __builtin_amdgcn_exp2f(-sh[qt]);
#pragma unroll
        for (int r = 0; r < 4; ++r) osum[qt][r] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[qt][dt][r] *= alpha;
      }
    }
    bf16x8 bp[kQT][2];
    probs8(s0, bp, 0);
    probs8(s1, bp, 1);
    pv8(sV[buf], bp, ones, g, l16, 0, oacc, osum);
    pv8(sV[buf], bp, ones, g, l16, 1, oacc, osum);
  }
  float lsum[kQT], mref[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) lsum[qt] = __shfl(osum[qt][0], l16);
  out_refs(ref, l16, mref);
  store_rows(a, u, c.qrow0, c.L, g, oacc, lsum, mref);
}

__global__ __launch_bounds__(kNW * 64) void attn_exact8(AttnArgs a) {
  __shared__ u32x4 sK[2][kKeyTile * 4];
  __shared__ u32x4 sV[2][kD * 8];
  const int n = *a.fb_count;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    __syncthreads();  // the previous unit's waves are done with the key buffers
    exact_unit8(a, a.fb_list[i], sK, sV);
  }
}

// Largest |K~| per (head, chunk of its rows): bf16 magnitudes compare as
// integers.  Grid (kKeyAmaxChunks, heads).
__global__ __launch_bounds__(256) void key_amax(const uint16_t* __restrict__ kt, int k_rows,
                                                float* __restrict__ kpart) {
  __shared__ uint32_t sM[4];
  const int h = blockIdx.y, chunk = blockIdx.x;
  const int64_t n8 = (int64_t)k_rows * kD / 8;  // 16-byte groups of the head
  const int64_t per = (n8 + kKeyAmaxChunks - 1) / kKeyAmaxChunks;
  const int64_t b = chunk * per, e = b + per < n8 ? b + per : n8;
  const u32x4* K = reinterpret_cast<const u32x4*>(kt + (size_t)h * k_rows * kD);
  uint32_t m = 0;
  for (int64_t i = b + threadIdx.x; i < e; i += 256) {
    const u32x4 v = K[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = v[j] & 0x7FFFu, hi = (v[j] >> 16) & 0x7FFFu;
      m = m > lo ? m : lo;
      m = m > hi ? m : hi;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t x = (uint32_t)__shfl_xor((int)m, o);
    m = m > x ? m : x;
  }
  if ((threadIdx.x & 63) == 0) sM[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = sM[0];
    for (int i = 1; i < 4; ++i) r = r > sM[i] ? r : sM[i];
    kpart[h * kKeyAmaxChunks + chunk] = __uint_as_float(r << 16);
  }
}

// K~ -> e4m3 with the head's exponent.  Grid (blocks over the head's 16-byte
// groups, heads); 8 bf16 in, 8 bytes out per thread and step.
__global__ __launch_bounds__(256) void key_quant(const uint16_t* __restrict__ kt, int k_rows,
                                                 const float* __restrict__ kpart, uint8_t* __restrict__ k8,
                                                 int32_t* __restrict__ kexp) {
  const int h = blockIdx.y;
  float am = 0.f;
  {
    const int lane = threadIdx.x & 63;
    am = kpart[h * kKeyAmaxChunks + lane];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
  }
  const int e = fp8_exponent(am);
  if (blockIdx.x == 0 && threadIdx.x == 0) kexp[h] = e;
  const int64_t n8 = (int64_t)k_rows * kD / 8;
  const u32x4* K = reinterpret_cast<const u32x4*>(kt + (size_t)h * k_rows * kD);
  u32x2* O = reinterpret_cast<u32x2*>(k8 + (size_t)h * k_rows * kD);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const u32x4 v = K[i];
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = ldexpf(__uint_as_float(v[j] << 16), e);
      x[2 * j + 1] = ldexpf(__uint_as_float(v[j] & 0xFFFF0000u), e);
    }
    O[i] = u32x2{pack_fp8x4(x[0], x[1], x[2], x[3]), pack_fp8x4(x[4], x[5], x[6], x[7])};
  }
}

}  // namespace

static_assert(kKeyAmaxChunks == 64, "key_quant reduces the partial maxima with one wave");

int attention_fp8_per_round(int split) { return per_round_for<attn_fast8>(split); }

hipError_t launch_quantize_keys(int heads, int k_rows, const void* kt, float* kpart, uint8_t* k8, int32_t* kexp,
                                hipStream_t stream) {
  if (heads <= 0 || k_rows <= 0 || k_rows % 64) return hipErrorInvalidValue;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(kt);
  hipLaunchKernelGGL(key_amax, dim3(kKeyAmaxChunks, heads), dim3(256), 0, stream, K, k_rows, kpart);
  const int64_t n8 = (int64_t)k_rows * kD / 8;
  const int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(key_quant, dim3((unsigned)(blocks < 1024 ? blocks : 1024), heads), dim3(256), 0, stream, K,
                     k_rows, kpart, k8, kexp);
  return hipGetLastError();
}

hipError_t launch_attention_fp8(const AttnShape& s, const void* q, const void* vt, const int32_t* lenq, void* o,
                                hipStream_t stream) {
  const AttnArgs a = make_attn_args(1, s, q, nullptr, vt, lenq, o, attention_fp8_per_round);
  hipLaunchKernelGGL(attn_fast8, dim3(a.total_wg), dim3(kNW * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attention_fp8_exact(const AttnShape& s, const void* q, const void* vt, const int32_t* lenq,
                                      void* o, hipStream_t stream) {
  const AttnArgs a = make_attn_args(1, s, q, nullptr, vt, lenq, o, attention_fp8_per_round);
  hipLaunchKernelGGL(attn_exact8, dim3(a.total_wg < kExactGrid8 ? a.total_wg : kExactGrid8), dim3(kNW * 64), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace httm
