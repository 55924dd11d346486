// Host side of the HTTM layer library: parameter validation, the plan (block
// geometry and sizes), workspace / index layouts, and the launch sequence.
//
// The launch sequence follows the layer as the HTTM page describes it
// ("HTTM: Head-wise Temporal Token Merging for Faster VGGT", overall framework):
// block-local matching of Q and K (key designs 1, 2), top-r merge, mean merge
// of K and V, query deviation, cross-head outlier selection and restore (key
// design 3), attention on the shortened sequences, unmerge.  Every per-head
// ragged length stays on the device; the host only uses bounds that follow
// from the parameters, so a call never waits for the GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/httm.h"
#include "geo.h"
#include "kernels.h"

using namespace httm;

namespace {

thread_local std::string g_err;

httm_status fail(httm_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

std::atomic<uint64_t> g_plan_counter{0x48540000ull};

// The K/V merge runs on a library stream (one per device, default priority)
// concurrently with the query path on the caller's stream: forked after the
// block selection, joined before attention.  The lock makes each call's
// record/wait pairs on the shared fork/join events atomic.
constexpr int kMaxDevices = 64;
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_launch_mu;
SideStream g_side[kMaxDevices];

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr float kLog2e = 1.4426950408889634f;

struct Region {
  size_t off = 0, bytes = 0;
};

struct Layout {
  Region match[2], score[2];
  Region q_members, q_off, q_group, k_group;
  Region qsum, delta, mask, radix, base, ocnt;
  Region qt, kt, vt, o;
  Region kmax, fb, opart, lpart, mpart;  // attention: key norms, fallback queue, split partials
  Region k8, kpart, kexp, q8, qexp;       // FP8 scores: e4m3 keys, key maxima, exponents, queries
  // geometry-aware partition (partition 1 only)
  Region ga_var, ga_role, ga_fcnt, ga_foff, ga_tot, ga_slot, ga_dlist, ga_dslot, ga_slist;
  Region ga_gdst, ga_gslot, ga_gscore, ga_best, ga_snorm, ga_cnt, ga_tmp, ga_dg, ga_dinv;
  Region sort_keys, sort_vals, sort_counts;  // stable sort by slot (partitions 1 and 2)
  // head-shared partition (partition 2 only)
  Region gm_metric, gm_tot, gm_dlist, gm_slist, gm_dg, gm_dinv, gm_best, gm_snorm, gm_match, gm_score, gm_sel,
      gm_topk, gm_unsel, gm_urank, gm_sums, gm_keys, gm_members, gm_off, gm_dbg_match, gm_dbg_score;
  Region index;  // used when the caller passes no index buffer
  size_t total = 0;
};

struct IndexLayout {
  Region header, k_members, k_off, fmembers, foff, slot, lenq, cu_q, lenk;
  size_t total = 0;
};

constexpr uint32_t kIndexMagic = 0x58495448u;  // "HTIX"
constexpr uint32_t kIndexVersion = 1;

// FNV-1a, 64-bit, over little-endian words.
struct Fnv {
  uint64_t h = 0xcbf29ce484222325ull;
  void add(uint64_t x) {
    for (int i = 0; i < 8; ++i) {
      h ^= (x >> (8 * i)) & 0xffu;
      h *= 0x100000001b3ull;
    }
  }
  void addd(double x) {
    uint64_t u;
    std::memcpy(&u, &x, 8);
    add(u);
  }
};

struct Builder {
  size_t cur = 0;
  Region take(size_t bytes) {
    Region r;
    r.off = cur;
    r.bytes = bytes;
    cur = align256(cur + bytes);
    return r;
  }
};

}  // namespace

struct httm_plan {
  httm_params p;
  uint64_t id;
  Geo g;
  int64_t k_o;
  int64_t q_cap;
  int64_t attn_units;  // upper bound of attention work units (all key splits; for the exact-path queue)
  int32_t lk_pad;
  float scale;
  size_t esize;
  Layout L;
  IndexLayout I;
  size_t dense_ws;
  size_t dense_vt_bytes, dense_kc_bytes;
  int32_t attn_split;
  IndexHeader index_header;  // identity written at the start of every index this plan fills
  AttnTail attn_tail;
  int64_t attn_part_rows;  // rows of each key-split partial buffer
  int32_t ga_kp = 0, ga_bound = 0, ga_max_src = 0;  // geometry-aware partition sizes
  int32_t ga_dpitch = 0;  // gathered destination rows per (stream, head)
  int32_t gm_nd = 0, gm_ns = 0, gm_r = 0, gm_dpitch = 0;  // head-shared partition sizes
  std::vector<httm_block> blocks;
};

namespace {

int stride_of(double ratio, int32_t given) {
  if (given > 0) return given;
  const int s = (int)std::ceil(1.0 / (1.0 - ratio) - 1e-9);
  return s > 4 ? s : 4;
}

int32_t merge_count(double ratio, int32_t n, int32_t ns) {
  const int32_t r = (int32_t)std::floor(ratio * (double)n + 1e-9);
  return r < ns ? r : ns;
}

httm_status build(const httm_params& p, httm_plan* pl) {
  if (p.heads < 1 || p.frames < 1 || p.grid_h < 1 || p.grid_w < 1 || p.n_special < 0 || p.n_s < 1 ||
      p.n_t < 1)
    return fail(HTTM_ERR_INVALID_ARG, "heads, frames, grid, n_s, n_t must be >= 1 and n_special >= 0");
  if (!(p.q_ratio >= 0.0 && p.q_ratio < 1.0) || !(p.kv_ratio >= 0.0 && p.kv_ratio < 1.0))
    return fail(HTTM_ERR_INVALID_ARG, "merge ratios must lie in [0, 1)");
  if (!(p.outlier_pct >= 0.0 && p.outlier_pct <= 100.0))
    return fail(HTTM_ERR_INVALID_ARG, "outlier_pct must lie in [0, 100]");
  if (p.q_dst_stride < 0 || p.kv_dst_stride < 0 || p.q_dst_stride == 1 || p.kv_dst_stride == 1)
    return fail(HTTM_ERR_INVALID_ARG, "destination strides must be 0 (derived) or >= 2");
  if (!(p.softmax_scale >= 0.0f) || std::isinf(p.softmax_scale))
    return fail(HTTM_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (p.dtype != HTTM_F32 && p.dtype != HTTM_BF16) return fail(HTTM_ERR_INVALID_ARG, "unknown dtype");
  if (p.d_head != kD) return fail(HTTM_ERR_UNSUPPORTED, "only d_head == 64 is built");
  if (p.heads > kMaxHeads) return fail(HTTM_ERR_UNSUPPORTED, "at most 64 heads (per-head prefix tables live in LDS)");
  if (p.block_order != 0 && p.block_order != 1) return fail(HTTM_ERR_INVALID_ARG, "block_order must be 0 or 1");
  if (p.partition < 0 || p.partition > 2) return fail(HTTM_ERR_INVALID_ARG, "partition must be 0, 1 or 2");
  if (p.partition == 1 && !(p.protect_pct >= 0.0 && p.protect_pct <= 100.0))
    return fail(HTTM_ERR_INVALID_ARG, "protect_pct must lie in [0, 100]");
  if ((int64_t)p.n_s * p.n_t > kMaxBlock) return fail(HTTM_ERR_UNSUPPORTED, "n_s * n_t must be <= 4096");
  if (p.attn_split != 0 && p.attn_split != 1 && p.attn_split != 2 && p.attn_split != 4 && p.attn_split != 8)
    return fail(HTTM_ERR_INVALID_ARG, "attn_split must be 0, 1, 2, 4 or 8");
  if (p.attn_fp8 != 0 && p.attn_fp8 != 1) return fail(HTTM_ERR_INVALID_ARG, "attn_fp8 must be 0 or 1");
  if (p.attn_fp8 && p.dtype != HTTM_BF16) return fail(HTTM_ERR_UNSUPPORTED, "FP8 scores need a bf16 layer");
  const int64_t T = (int64_t)p.n_special + (int64_t)p.grid_h * p.grid_w;
  const int64_t N = (int64_t)p.frames * T;
  if ((int64_t)p.heads * N >= (1ll << 31) || (int64_t)p.heads * N * kD >= (1ll << 40))
    return fail(HTTM_ERR_INVALID_ARG, "heads * N must be < 2^31");
  if (N >= (1ll << 24))
    return fail(HTTM_ERR_UNSUPPORTED, "N must be < 2^24 (a head's merged keys are addressed with 32-bit offsets)");

  pl->p = p;
  Geo& g = pl->g;
  std::memset(&g, 0, sizeof(g));
  g.heads = p.heads;
  g.F = p.frames;
  g.HW = p.grid_h * p.grid_w;
  g.nsp = p.n_special;
  g.T = (int32_t)T;
  g.N = (int32_t)N;
  g.P = p.frames * g.HW;
  g.n_s = p.n_s < g.HW ? p.n_s : g.HW;
  g.n_t = p.n_t < p.frames ? p.n_t : p.frames;
  g.A = ceil_div(g.HW, g.n_s);
  g.G = ceil_div(g.F, g.n_t);
  g.nf_last = g.F - (g.G - 1) * g.n_t;
  g.run_last = g.HW - (g.A - 1) * g.n_s;
  g.nblocks = g.A * g.G;
  g.order = p.block_order;
  const double ratio[2] = {p.q_ratio, p.kv_ratio};
  g.s[0] = stride_of(p.q_ratio, p.q_dst_stride);
  g.s[1] = stride_of(p.kv_ratio, p.kv_dst_stride);
  for (int st = 0; st < 2; ++st) {
    for (int lg = 0; lg < 2; ++lg)
      for (int lr = 0; lr < 2; ++lr) {
        const int32_t nf = lg ? g.nf_last : g.n_t;
        const int32_t run = lr ? g.run_last : g.n_s;
        const int32_t n = nf * run;
        const int32_t nd = ceil_div(n, g.s[st]);
        g.r[st][lg][lr] = merge_count(ratio[st], n, n - nd);
      }
    // one full temporal group: (A-1) full runs and the last run, nf = n_t
    const int32_t nfull = g.n_t * g.n_s, nlast = g.n_t * g.run_last;
    const int32_t ndf = ceil_div(nfull, g.s[st]), ndl = ceil_div(nlast, g.s[st]);
    if (g.A > 1) {
      g.grp_slots[st] = (g.A - 1) * (nfull - g.r[st][0][0]) + (nlast - g.r[st][0][1]);
      g.grp_src[st] = (g.A - 1) * (nfull - ndf) + (nlast - ndl);
    } else {
      g.grp_slots[st] = nlast - g.r[st][0][1];
      g.grp_src[st] = nlast - ndl;
    }
  }
  // Per-block table (host copy, for callers and for totals); the kernels
  // recompute the same rows from Geo.
  pl->blocks.resize(g.nblocks);
  int64_t slots[2] = {0, 0}, srcs[2] = {0, 0};
  for (int b = 0; b < g.nblocks; ++b) {
    const BlockInfo q = block_info(g, b, kQ), k = block_info(g, b, kK);
    if (q.slot0 != slots[0] || k.slot0 != slots[1] || q.src0 != srcs[0] || k.src0 != srcs[1])
      return fail(HTTM_ERR_INVALID_ARG, "internal: block prefix mismatch");
    httm_block& r = pl->blocks[b];
    r.start = q.start;
    r.n = q.n;
    r.f0 = q.f0;
    r.nf = q.nf;
    r.j0 = q.j0;
    r.run = q.run;
    r.q_dst = q.nd;
    r.q_src = q.ns;
    r.q_r = q.r;
    r.kv_dst = k.nd;
    r.kv_src = k.ns;
    r.kv_r = k.r;
    r.q_slot0 = q.slot0;
    r.kv_slot0 = k.slot0;
    r.q_src0 = q.src0;
    r.kv_src0 = k.src0;
    slots[0] += q.n - q.r;
    slots[1] += k.n - k.r;
    srcs[0] += q.ns;
    srcs[1] += k.ns;
  }
  for (int st = 0; st < 2; ++st) {
    g.nslots[st] = (int32_t)(slots[st] + (int64_t)g.F * g.nsp);
    g.nsrc[st] = (int32_t)srcs[st];
  }
  if (p.partition == 1) {
    // groups per head: every anchor (special, protected or destination) is
    // one; the first frame's patches are all anchors, another frame has its
    // protected patches and at most one destination per 2x2 cell
    if (g.HW > kMaxFrameHW) return fail(HTTM_ERR_UNSUPPORTED, "geometry-aware partition: at most 4096 patches per frame");
    if (N >= (1 << 20)) return fail(HTTM_ERR_UNSUPPORTED, "geometry-aware partition: at most 2^20 - 1 tokens");
    const int64_t kp = (int64_t)std::floor(p.protect_pct / 100.0 * (double)g.HW + 1e-9);
    const int64_t cells = (int64_t)((p.grid_h + 1) / 2) * ((p.grid_w + 1) / 2);
    const int64_t bound = (int64_t)g.F * g.nsp + g.HW + (int64_t)(g.F - 1) * (kp + cells);
    const int64_t bound_c = bound < N ? bound : N;
    pl->ga_kp = (int32_t)kp;
    pl->ga_bound = (int32_t)bound_c;
    pl->ga_max_src = (int32_t)((int64_t)(g.F - 1) * g.HW);
    // destinations: the first frame's unprotected patches, one per 2x2 cell elsewhere
    const int64_t max_dst = (g.HW - kp) + (int64_t)(g.F - 1) * cells;
    pl->ga_dpitch = (int32_t)(((max_dst < 1 ? 1 : max_dst) + 63) / 64 * 64);
    g.nslots[kQ] = g.nslots[kK] = (int32_t)bound_c;
    g.nsrc[kQ] = g.nsrc[kK] = pl->ga_max_src;
  }
  if (p.partition == 2) {
    // one block of every patch token in original order, every 4th a
    // destination; r of the sources merge; N - r groups per head
    if (N >= (1 << 20)) return fail(HTTM_ERR_UNSUPPORTED, "head-shared partition: at most 2^20 - 1 tokens");
    const int32_t P = g.P;
    pl->gm_nd = ceil_div(P, 4);
    pl->gm_ns = P - pl->gm_nd;
    pl->gm_r = merge_count(p.kv_ratio, P, pl->gm_ns);
    pl->gm_dpitch = ceil_div(pl->gm_nd > 0 ? pl->gm_nd : 1, 64) * 64;
    g.nslots[kQ] = g.nslots[kK] = g.N - pl->gm_r;
    g.nsrc[kQ] = g.nsrc[kK] = pl->gm_ns;
  }
  pl->k_o = (int64_t)std::floor(p.outlier_pct * (double)p.heads * (double)N / 100.0 + 1e-9);
  pl->q_cap = (int64_t)p.heads * g.nslots[kQ] + pl->k_o;
  pl->lk_pad = ceil_div(g.nslots[kK], 64) * 64;
  pl->scale = p.softmax_scale > 0.0f ? p.softmax_scale : 1.0f / std::sqrt((float)kD);
  pl->esize = p.dtype == HTTM_BF16 ? 2 : 4;
  pl->attn_split = p.dtype != HTTM_BF16 ? 1 : (p.attn_split > 0 ? p.attn_split : attention_split(pl->q_cap, p.heads));
  pl->attn_tail = attention_tail(pl->attn_split);
  {
    // exact-path queue capacity: workgroups of the layer's or the unmerged
    // baseline's attention launch, whichever is larger
    AttnShape s{};
    s.heads = p.heads;
    s.q_capacity = pl->q_cap;
    s.split = pl->attn_split;
    s.tail_split = pl->attn_tail.tail_split;
    s.per_round = pl->attn_tail.per_round;
    s.tail_rows = pl->attn_tail.tail_rows;
    const int64_t layer_wgs = attention_workgroups(p.dtype, s);
    pl->attn_part_rows = pl->attn_split > 1 ? attention_partial_rows(s) : 0;
    AttnShape d{};
    d.heads = p.heads;
    d.q_capacity = (int64_t)p.heads * N;
    d.split = 1;
    const int64_t dense_wgs = attention_workgroups(p.dtype, d);
    pl->attn_units = layer_wgs > dense_wgs ? layer_wgs : dense_wgs;
  }

  const size_t h = (size_t)p.heads, n = (size_t)N, E = pl->esize;
  // index layout
  {
    Builder b;
    IndexLayout& I = pl->I;
    I.header = b.take(sizeof(IndexHeader));
    I.k_members = b.take(4 * h * n);
    I.k_off = b.take(4 * h * ((size_t)g.nslots[kK] + 1));
    I.fmembers = b.take(4 * h * n);
    I.foff = b.take(4 * h * (n + 1));
    I.slot = b.take(4 * h * n);
    I.lenq = b.take(4 * h);
    I.cu_q = b.take(4 * (h + 1));
    I.lenk = b.take(4 * h);  // keys per head (geometry-aware partition)
    I.total = b.cur;
  }
  {
    Builder b;
    Layout& Lw = pl->L;
    const bool ga = p.partition == 1;
    for (int st = 0; st < 2; ++st) {  // block-local matches (partition 0)
      Lw.match[st] = b.take(ga ? 0 : 4 * h * (size_t)g.nsrc[st]);
      Lw.score[st] = b.take(ga ? 0 : 4 * h * (size_t)g.nsrc[st]);
    }
    if (ga) {
      const size_t sh = 2 * h, F = (size_t)g.F;
      Lw.ga_var = b.take(4 * sh * n);
      Lw.ga_role = b.take(sh * n);
      Lw.ga_fcnt = b.take(4 * sh * F * 3);
      Lw.ga_foff = b.take(4 * sh * F * 3);
      Lw.ga_tot = b.take(4 * sh * 3);
      Lw.ga_slot = b.take(4 * sh * n);
      Lw.ga_dlist = b.take(4 * sh * n);
      Lw.ga_dslot = b.take(4 * sh * n);
      Lw.ga_slist = b.take(4 * sh * n);
      Lw.ga_gdst = b.take(4 * sh * n);
      Lw.ga_gslot = b.take(4 * sh * n);
      Lw.ga_gscore = b.take(4 * sh * n);
      Lw.ga_best = b.take(8 * sh * n);
      Lw.ga_snorm = b.take(4 * sh * n);
      Lw.ga_cnt = b.take(4 * sh * (size_t)pl->ga_bound);
      Lw.ga_tmp = b.take(4 * sh * n);
      Lw.sort_keys = b.take(4 * sh * n);
      Lw.sort_vals = b.take(4 * sh * n);
      Lw.sort_counts = b.take(4 * sort_count_words((int)sh, (int)n));
      const bool bf = p.dtype == HTTM_BF16;
      Lw.ga_dg = b.take(bf ? 2 * sh * (size_t)pl->ga_dpitch * kD : 0);
      Lw.ga_dinv = b.take(bf ? 4 * sh * (size_t)pl->ga_dpitch : 0);
    }
    if (p.partition == 2) {
      const size_t ns = (size_t)pl->gm_ns, dp = (size_t)pl->gm_dpitch;
      Lw.gm_metric = b.take(E * n * kD);
      Lw.gm_tot = b.take(4 * 3);
      Lw.gm_dlist = b.take(4 * dp);
      Lw.gm_slist = b.take(4 * (ns + 1));
      Lw.gm_dg = b.take(E == 2 ? 2 * dp * kD : 0);
      Lw.gm_dinv = b.take(E == 2 ? 4 * dp : 0);
      Lw.gm_best = b.take(8 * n);
      Lw.gm_snorm = b.take(4 * n);
      Lw.gm_match = b.take(4 * (ns + 1));
      Lw.gm_score = b.take(4 * (ns + 1));
      Lw.gm_sel = b.take(ns + 16);
      Lw.gm_topk = b.take(4 * outlier_scratch_words((int64_t)ns));
      Lw.gm_unsel = b.take(4 * (ns + 1));
      Lw.gm_urank = b.take(4 * (ns + 1));
      Lw.gm_sums = b.take(4 * scan_sum_words((int64_t)ns));
      Lw.gm_keys = b.take(4 * n);
      Lw.sort_keys = b.take(4 * n);
      Lw.sort_vals = b.take(4 * n);
      Lw.sort_counts = b.take(4 * sort_count_words(1, (int)n));
      Lw.gm_members = b.take(4 * n);
      Lw.gm_off = b.take(4 * ((size_t)g.nslots[kQ] + 1));
      Lw.gm_dbg_match = b.take(4 * n);
      Lw.gm_dbg_score = b.take(4 * n);
    }
    Lw.q_members = b.take(4 * h * n);
    Lw.q_off = b.take(4 * h * ((size_t)g.nslots[kQ] + 1));
    Lw.q_group = b.take(4 * h * n);
    Lw.k_group = b.take(4 * h * n);
    Lw.qsum = b.take(4 * h * (size_t)g.nslots[kQ] * kD);
    Lw.delta = b.take(4 * h * n);
    Lw.mask = b.take(h * n);
    Lw.radix = b.take(4 * outlier_scratch_words((int64_t)h * n));
    Lw.base = b.take(4 * h * (size_t)g.nslots[kQ]);
    Lw.ocnt = b.take(4 * h * (size_t)g.nslots[kQ]);
    Lw.qt = b.take(E * (size_t)pl->q_cap * kD);
    Lw.kt = b.take(E * h * (size_t)pl->lk_pad * kD);
    Lw.vt = b.take(E * h * (size_t)pl->lk_pad * kD);
    Lw.o = b.take(E * (size_t)pl->q_cap * kD);
    Lw.kmax = b.take(4 * h);
    Lw.fb = b.take(4 * (1 + (size_t)pl->attn_units));  // exact-path queue: count, then unit ids
    if (pl->attn_split > 1) {
      Lw.opart = b.take(4 * (size_t)pl->attn_part_rows * kD);
      Lw.lpart = b.take(4 * (size_t)pl->attn_part_rows);
      Lw.mpart = b.take(4 * (size_t)pl->attn_part_rows);
    }
    if (p.attn_fp8) {
      Lw.k8 = b.take(h * (size_t)pl->lk_pad * kD);
      Lw.kpart = b.take(4 * h * (size_t)kKeyAmaxChunks);
      Lw.kexp = b.take(4 * h);
      Lw.q8 = b.take((size_t)pl->q_cap * kD);
      Lw.qexp = b.take(4 * (size_t)pl->q_cap);
    }
    Lw.index = b.take(pl->I.total);
    Lw.total = b.cur;
  }
  pl->dense_vt_bytes = align256(E * h * (size_t)ceil_div(g.N, 64) * 64 * kD);
  pl->dense_kc_bytes = align256(E * h * (size_t)ceil_div(g.N, 64) * 64 * kD);
  pl->dense_ws = pl->dense_vt_bytes + pl->dense_kc_bytes + pl->L.kmax.bytes + 256 + pl->L.fb.bytes;
  pl->id = ++g_plan_counter;
  {
    // what an index depends on: every parameter and the index geometry
    Fnv f;
    f.add((uint64_t)p.heads);
    f.add((uint64_t)p.d_head);
    f.add((uint64_t)p.frames);
    f.add((uint64_t)p.grid_h);
    f.add((uint64_t)p.grid_w);
    f.add((uint64_t)p.n_special);
    f.add((uint64_t)p.n_s);
    f.add((uint64_t)p.n_t);
    f.addd(p.q_ratio);
    f.addd(p.kv_ratio);
    f.addd(p.outlier_pct);
    f.add((uint64_t)g.s[kQ]);
    f.add((uint64_t)g.s[kK]);
    f.add((uint64_t)p.block_order);
    f.add((uint64_t)p.dtype);
    f.add((uint64_t)g.N);
    f.add((uint64_t)g.nslots[kQ]);
    f.add((uint64_t)g.nslots[kK]);
    f.add((uint64_t)pl->I.total);
    f.add((uint64_t)p.partition);
    f.addd(p.partition == 1 ? p.protect_pct : 0.0);
    IndexHeader& H = pl->index_header;
    std::memset(&H, 0, sizeof(H));
    H.w[0] = kIndexMagic;
    H.w[1] = kIndexVersion;
    H.w[2] = (uint32_t)f.h;
    H.w[3] = (uint32_t)(f.h >> 32);
    H.w[4] = (uint32_t)pl->I.total;
    H.w[5] = (uint32_t)((uint64_t)pl->I.total >> 32);
    H.w[6] = (uint32_t)p.heads;
    H.w[7] = (uint32_t)g.N;
  }
  return HTTM_OK;
}

template <typename P>
P* at(void* base, const Region& r) {
  return reinterpret_cast<P*>(reinterpret_cast<char*>(base) + r.off);
}

// ---------------------------------------------------------------- timing
// HIP events around selected stages, for up to kSlots consecutive calls.
constexpr int kSlots = 32;
struct Timing {
  int32_t mask = 0;
  bool serial = false;
  bool created = false;
  int calls = 0;
  hipEvent_t ev[kSlots][2 * HTTM_T_COUNT] = {};
  bool used[kSlots][HTTM_T_COUNT] = {};
};
Timing g_timing;

void stage_begin(int s, hipStream_t st) {
  if ((g_timing.mask >> s) & 1) {
    const int slot = g_timing.calls % kSlots;
    (void)hipEventRecord(g_timing.ev[slot][2 * s], st);
    g_timing.used[slot][s] = true;
  }
}
void stage_end(int s, hipStream_t st) {
  if ((g_timing.mask >> s) & 1) (void)hipEventRecord(g_timing.ev[g_timing.calls % kSlots][2 * s + 1], st);
}
void timing_begin_call() {
  if (!g_timing.mask) return;
  const int slot = g_timing.calls % kSlots;
  for (int i = 0; i < HTTM_T_COUNT; ++i) g_timing.used[slot][i] = false;
}
void timing_end_call() {
  if (g_timing.mask) ++g_timing.calls;
}
// While timing with HTTM_TIMING_SERIAL, layers enqueue every launch on the
// caller's stream, so that each stage's events bracket kernels running alone.
bool timing_serial() { return g_timing.serial; }

// Test hook (httm_debug_fail_launch): the n-th checked launch after it is
// set reports a failure instead of running, once.
std::atomic<int32_t> g_fail_at{0}, g_fail_tick{0};
bool forced_failure() {
  if (g_fail_at.load(std::memory_order_relaxed) <= 0) return false;
  if (g_fail_tick.fetch_add(1) + 1 != g_fail_at.load()) return false;
  g_fail_at.store(0);
  return true;
}

#define CHECK_LAUNCH(expr)                                                        \
  do {                                                                            \
    if (forced_failure()) return fail(HTTM_ERR_DEVICE, std::string("forced launch failure before ") + #expr); \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) return fail(HTTM_ERR_DEVICE, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

// Side stream of the current device (created on first use; call with g_launch_mu held).
httm_status side_stream(SideStream** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(HTTM_ERR_DEVICE, "no usable current device");
  SideStream& s = g_side[dev];
  if (!s.st) {
    // the fork / join events order two streams of one device: device-scope
    // release and acquire suffice, without the system-scope cache fences
    const unsigned ef = hipEventDisableTiming | hipEventDisableSystemFence;
    if (hipStreamCreateWithFlags(&s.st, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&s.fork, ef) != hipSuccess || hipEventCreateWithFlags(&s.join, ef) != hipSuccess)
      return fail(HTTM_ERR_DEVICE, "creating the library stream failed");
  }
  *out = &s;
  return HTTM_OK;
}

httm_status check_common(const httm_plan* plan, void* ws, size_t ws_bytes, const void* q,
                         const void* k, const void* v, void* out, size_t need) {
  if (!plan) return fail(HTTM_ERR_INVALID_ARG, "plan is NULL");
  if (!q || !k || !v || !out) return fail(HTTM_ERR_INVALID_ARG, "q, k, v and out must not be NULL");
  if (!ws) return fail(HTTM_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < need) return fail(HTTM_ERR_WORKSPACE, "workspace smaller than httm_workspace_size()");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)ws) & 15)
    return fail(HTTM_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  return HTTM_OK;
}

// Attention + unmerge, shared by the full and cached layers.
httm_status attend_unmerge(const httm_plan* pl, void* ws, char* idx, const void* qt,
                           void* out, hipStream_t st) {
  const Geo& g = pl->g;
  const int dt = pl->p.dtype;
  AttnShape s{};
  s.heads = g.heads;
  s.lk = g.nslots[kK];
  s.k_rows = pl->lk_pad;
  s.vt_pitch = pl->lk_pad;
  s.lq_uniform = 0;
  s.q_capacity = pl->q_cap;
  s.scale = pl->scale;
  s.split = pl->attn_split;
  s.tail_split = pl->attn_tail.tail_split;
  s.per_round = pl->attn_tail.per_round;
  s.tail_rows = pl->attn_tail.tail_rows;
  s.opart = pl->attn_split > 1 ? at<float>(ws, pl->L.opart) : nullptr;
  s.lpart = pl->attn_split > 1 ? at<float>(ws, pl->L.lpart) : nullptr;
  s.mpart = pl->attn_split > 1 ? at<float>(ws, pl->L.mpart) : nullptr;
  s.kmax = at<float>(ws, pl->L.kmax);
  s.fb_count = at<int>(ws, pl->L.fb);
  s.fb_list = at<int>(ws, pl->L.fb) + 1;
  s.lenk = pl->p.partition == 1 ? reinterpret_cast<const int32_t*>(idx + pl->I.lenk.off) : nullptr;
  const int32_t* lenq = reinterpret_cast<const int32_t*>(idx + pl->I.lenq.off);
  if (pl->p.attn_fp8) {
    s.k8 = at<uint8_t>(ws, pl->L.k8);
    s.kexp = at<int32_t>(ws, pl->L.kexp);
    s.q8 = at<uint8_t>(ws, pl->L.q8);
    s.qexp = at<int32_t>(ws, pl->L.qexp);
    stage_begin(HTTM_T_KEY_FP8, st);
    CHECK_LAUNCH(launch_quantize_keys(g.heads, pl->lk_pad, at<void>(ws, pl->L.kt), at<float>(ws, pl->L.kpart),
                                      at<uint8_t>(ws, pl->L.k8), at<int32_t>(ws, pl->L.kexp), st));
    stage_end(HTTM_T_KEY_FP8, st);
  }
  stage_begin(HTTM_T_ATTN, st);
  CHECK_LAUNCH(launch_attention(dt, s, qt, at<void>(ws, pl->L.kt), at<void>(ws, pl->L.vt), lenq,
                                at<void>(ws, pl->L.o), st));
  stage_end(HTTM_T_ATTN, st);
  stage_begin(HTTM_T_ATTN_TAIL, st);
  CHECK_LAUNCH(launch_attention_tail(dt, s, qt, at<void>(ws, pl->L.kt), at<void>(ws, pl->L.vt), lenq,
                                     at<void>(ws, pl->L.o), st));
  stage_end(HTTM_T_ATTN_TAIL, st);
  stage_begin(HTTM_T_UNMERGE, st);
  CHECK_LAUNCH(launch_unmerge(dt, g.heads, g.N, reinterpret_cast<const int32_t*>(idx + pl->I.slot.off),
                              at<void>(ws, pl->L.o), out, st));
  stage_end(HTTM_T_UNMERGE, st);
  return HTTM_OK;
}

}  // namespace

// An imported index must keep every kernel that reads it in bounds: offsets
// rise from 0 to N, member ids and slots stay inside their head, and the
// per-head lengths fit the packed capacity.
namespace {
bool index_payload_ok(const httm_plan* pl, const char* buf) {
  const Geo& g = pl->g;
  const IndexLayout& I = pl->I;
  const int64_t N = g.N, H = g.heads, lk = g.nslots[kK];
  auto arr = [&](const Region& r) { return reinterpret_cast<const int32_t*>(buf + r.off); };
  const int32_t *km = arr(I.k_members), *ko = arr(I.k_off), *fm = arr(I.fmembers), *fo = arr(I.foff);
  const int32_t *sl = arr(I.slot), *lq = arr(I.lenq), *cu = arr(I.cu_q), *lkh = arr(I.lenk);
  const bool ga = pl->p.partition == 1;
  if (cu[0] != 0) return false;
  for (int64_t h = 0; h < H; ++h) {
    const int64_t len = lq[h];
    if (len < 1 || len > N || cu[h + 1] != cu[h] + len || cu[h + 1] > pl->q_cap) return false;
    // keys of this head: every slot (block-local matching) or the first lenk
    // slots, the rest empty (geometry-aware partition)
    const int64_t nk = ga ? lkh[h] : lk;
    if (nk < 1 || nk > lk) return false;
    const int32_t* o = ko + h * (lk + 1);
    if (o[0] != 0 || o[nk] != N) return false;
    for (int64_t j = 0; j < nk; ++j)
      if (o[j + 1] <= o[j]) return false;  // every merged key has a member
    for (int64_t j = nk; j < lk; ++j)
      if (o[j + 1] != N) return false;
    const int32_t* f = fo + h * (N + 1);
    if (f[0] != 0 || f[len] != N) return false;
    for (int64_t j = 0; j < len; ++j)
      if (f[j + 1] <= f[j]) return false;  // every packed query row has a member
    for (int64_t n = 0; n < N; ++n) {
      const int32_t a = km[h * N + n], b = fm[h * N + n], c = sl[h * N + n];
      if (a < 0 || a >= N || b < 0 || b >= N || c < cu[h] || c >= cu[h + 1]) return false;
    }
  }
  return true;
}
}  // namespace

namespace {

// Device scratch of httm_layer_noalloc: its workspace (and merge index) on
// every GPU the library runs on, held until the process ends.  In host code
// `scratch` only names the symbol; its device address on the current device
// comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kNoAllocBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];
void* g_scratch[kMaxDevices];

// Address of the current device's scratch (call with g_launch_mu held).
httm_status scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(HTTM_ERR_DEVICE, "no usable current device");
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(HTTM_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return HTTM_OK;
}

}  // namespace

namespace {

// One full layer enqueued on `st`.  With a library side stream the key branch
// forks onto it (joined back before the attention); with side == nullptr
// every launch goes to `st` in order.  Call with g_launch_mu held and the
// arguments validated.
httm_status enqueue_layer(const httm_plan* pl, void* ws, httm_index* index, const void* q, const void* k,
                          const void* v, void* out, hipStream_t st, SideStream* side) {
  const Geo& g = pl->g;
  const Layout& L = pl->L;
  const IndexLayout& I = pl->I;
  const int dt = pl->p.dtype;
  char* idx = index ? reinterpret_cast<char*>(index->dev) : at<char>(ws, L.index);
  hipStream_t kst = side ? side->st : st;  // stream of the key branch
  httm_status s = HTTM_OK;
  timing_begin_call();

  Csr cq{at<int32_t>(ws, L.q_members), at<int32_t>(ws, L.q_off), at<int32_t>(ws, L.q_group)};
  Csr ck{reinterpret_cast<int32_t*>(idx + I.k_members.off), reinterpret_cast<int32_t*>(idx + I.k_off.off),
         at<int32_t>(ws, L.k_group)};
  const int64_t hn = (int64_t)g.heads * g.N;
  // atomic targets of this layer: key norms, exact-path count, outlier scratch, outlier counts
  CHECK_LAUNCH(launch_zero_init(at<float>(ws, L.kmax), g.heads, at<int>(ws, L.fb), at<uint32_t>(ws, L.radix),
                                (int)outlier_scratch_words(hn), nullptr, 0, st, &pl->index_header,
                                reinterpret_cast<uint32_t*>(idx + I.header.off)));

  if (pl->p.partition == 1) {
    // geometry-aware partition of both streams in one pass on the caller's
    // stream, then the K / V means on the library stream
    int32_t* lenk = reinterpret_cast<int32_t*>(idx + I.lenk.off);
    GaShape gs{g.heads, g.N,         g.T,          g.nsp,          pl->p.grid_h,
               pl->p.grid_w, g.F, pl->ga_kp, pl->ga_bound, pl->ga_max_src, pl->ga_dpitch};
    GaBuffers gb;
    gb.var = at<float>(ws, L.ga_var);
    gb.role = at<uint8_t>(ws, L.ga_role);
    gb.fcnt = at<int32_t>(ws, L.ga_fcnt);
    gb.foff = at<int32_t>(ws, L.ga_foff);
    gb.tot = at<int32_t>(ws, L.ga_tot);
    gb.slot = at<int32_t>(ws, L.ga_slot);
    gb.dst_list = at<int32_t>(ws, L.ga_dlist);
    gb.dst_slot = at<int32_t>(ws, L.ga_dslot);
    gb.src_list = at<int32_t>(ws, L.ga_slist);
    gb.gdst = at<int32_t>(ws, L.ga_gdst);
    gb.gslot = at<int32_t>(ws, L.ga_gslot);
    gb.gscore = at<float>(ws, L.ga_gscore);
    gb.dg = at<uint16_t>(ws, L.ga_dg);
    gb.dinv = at<float>(ws, L.ga_dinv);
    gb.best = at<uint64_t>(ws, L.ga_best);
    gb.snorm = at<float>(ws, L.ga_snorm);
    gb.cnt = at<int32_t>(ws, L.ga_cnt);
    gb.tmp = at<int32_t>(ws, L.ga_tmp);
    gb.sort_keys = at<int32_t>(ws, L.sort_keys);
    gb.sort_vals = at<int32_t>(ws, L.sort_vals);
    gb.sort_counts = at<uint32_t>(ws, L.sort_counts);
    gb.grp_q = cq.group;
    gb.grp_k = ck.group;
    gb.mem_q = cq.members;
    gb.mem_k = ck.members;
    gb.off_q = cq.off;
    gb.off_k = ck.off;
    gb.lenk = lenk;
    stage_begin(HTTM_T_SIM, st);
    CHECK_LAUNCH(launch_ga_partition(dt, gs, q, k, gb, st, 0));
    CHECK_LAUNCH(launch_ga_partition(dt, gs, q, k, gb, st, 1));
    stage_begin(HTTM_T_GA_MATCH, st);
    CHECK_LAUNCH(launch_ga_partition(dt, gs, q, k, gb, st, 2));
    stage_end(HTTM_T_GA_MATCH, st);
    CHECK_LAUNCH(launch_ga_partition(dt, gs, q, k, gb, st, 3));
    stage_end(HTTM_T_SIM, st);
    if (side) {
      CHECK_LAUNCH(hipEventRecord(side->fork, st));
      CHECK_LAUNCH(hipStreamWaitEvent(kst, side->fork, 0));
    }
    stage_begin(HTTM_T_MERGE_KV, kst);
    CHECK_LAUNCH(launch_merge_kv(dt, g.heads, g.N, g.nslots[kK], pl->lk_pad, pl->scale * kLog2e, k, v,
                                 ck.members, ck.off, at<void>(ws, L.kt), at<void>(ws, L.vt), at<float>(ws, L.kmax),
                                 kst, lenk));
    stage_end(HTTM_T_MERGE_KV, kst);
    if (side) CHECK_LAUNCH(hipEventRecord(side->join, kst));
  } else if (pl->p.partition == 2) {
    // one head-shared partition (global matching on the head-mean key) on
    // the caller's stream, copied to every head's query and key CSR; then
    // the K / V means on the library stream
    GmShape gs{g.heads, g.N, g.T, g.nsp, g.HW, pl->gm_nd, pl->gm_ns, pl->gm_r, g.nslots[kQ], pl->gm_dpitch};
    GmBuffers gb;
    gb.metric = at<void>(ws, L.gm_metric);
    gb.tot = at<int32_t>(ws, L.gm_tot);
    gb.dst_list = at<int32_t>(ws, L.gm_dlist);
    gb.src_list = at<int32_t>(ws, L.gm_slist);
    gb.dg = at<uint16_t>(ws, L.gm_dg);
    gb.dinv = at<float>(ws, L.gm_dinv);
    gb.best = at<uint64_t>(ws, L.gm_best);
    gb.snorm = at<float>(ws, L.gm_snorm);
    gb.match = at<int32_t>(ws, L.gm_match);
    gb.score = at<float>(ws, L.gm_score);
    gb.sel = at<uint8_t>(ws, L.gm_sel);
    gb.topk = at<uint32_t>(ws, L.gm_topk);
    gb.unsel = at<int32_t>(ws, L.gm_unsel);
    gb.urank = at<int32_t>(ws, L.gm_urank);
    gb.scan_sums = at<int32_t>(ws, L.gm_sums);
    gb.keys = at<int32_t>(ws, L.gm_keys);
    gb.sort_keys = at<int32_t>(ws, L.sort_keys);
    gb.sort_vals = at<int32_t>(ws, L.sort_vals);
    gb.sort_counts = at<uint32_t>(ws, L.sort_counts);
    gb.members = at<int32_t>(ws, L.gm_members);
    gb.off = at<int32_t>(ws, L.gm_off);
    gb.dbg_match = at<int32_t>(ws, L.gm_dbg_match);
    gb.dbg_score = at<float>(ws, L.gm_dbg_score);
    gb.q = cq;
    gb.k = ck;
    stage_begin(HTTM_T_SIM, st);
    CHECK_LAUNCH(launch_global_partition(dt, gs, k, gb, st, 0));
    stage_begin(HTTM_T_GA_MATCH, st);
    CHECK_LAUNCH(launch_global_partition(dt, gs, k, gb, st, 1));
    stage_end(HTTM_T_GA_MATCH, st);
    CHECK_LAUNCH(launch_global_partition(dt, gs, k, gb, st, 2));
    stage_end(HTTM_T_SIM, st);
    if (side) {
      CHECK_LAUNCH(hipEventRecord(side->fork, st));
      CHECK_LAUNCH(hipStreamWaitEvent(kst, side->fork, 0));
    }
    stage_begin(HTTM_T_MERGE_KV, kst);
    CHECK_LAUNCH(launch_merge_kv(dt, g.heads, g.N, g.nslots[kK], pl->lk_pad, pl->scale * kLog2e, k, v,
                                 ck.members, ck.off, at<void>(ws, L.kt), at<void>(ws, L.vt), at<float>(ws, L.kmax),
                                 kst));
    stage_end(HTTM_T_MERGE_KV, kst);
    if (side) CHECK_LAUNCH(hipEventRecord(side->join, kst));
  } else {
    // key branch on the library stream (if any): matching, selection and merge of K / V
    if (side) {
      CHECK_LAUNCH(hipEventRecord(side->fork, st));
      CHECK_LAUNCH(hipStreamWaitEvent(kst, side->fork, 0));
    }
    stage_begin(HTTM_T_SIM_K, kst);
    CHECK_LAUNCH(launch_sim(g, dt, q, k, at<int32_t>(ws, L.match[kQ]), at<float>(ws, L.score[kQ]),
                            at<int32_t>(ws, L.match[kK]), at<float>(ws, L.score[kK]), 2, kst));
    stage_end(HTTM_T_SIM_K, kst);
    stage_begin(HTTM_T_SELECT_K, kst);
    CHECK_LAUNCH(launch_select(g, at<int32_t>(ws, L.match[kQ]), at<float>(ws, L.score[kQ]),
                               at<int32_t>(ws, L.match[kK]), at<float>(ws, L.score[kK]), cq, ck, 2, kst));
    stage_end(HTTM_T_SELECT_K, kst);
    stage_begin(HTTM_T_MERGE_KV, kst);
    CHECK_LAUNCH(launch_merge_kv(dt, g.heads, g.N, g.nslots[kK], pl->lk_pad, pl->scale * kLog2e, k, v,
                                 ck.members, ck.off,
                                 at<void>(ws, L.kt), at<void>(ws, L.vt), at<float>(ws, L.kmax), kst));
    stage_end(HTTM_T_MERGE_KV, kst);
    if (side) CHECK_LAUNCH(hipEventRecord(side->join, kst));

    // query branch on the caller's stream
    stage_begin(HTTM_T_SIM, st);
    CHECK_LAUNCH(launch_sim(g, dt, q, k, at<int32_t>(ws, L.match[kQ]), at<float>(ws, L.score[kQ]),
                            at<int32_t>(ws, L.match[kK]), at<float>(ws, L.score[kK]), 1, st));
    stage_end(HTTM_T_SIM, st);
    stage_begin(HTTM_T_SELECT, st);
    CHECK_LAUNCH(launch_select(g, at<int32_t>(ws, L.match[kQ]), at<float>(ws, L.score[kQ]),
                               at<int32_t>(ws, L.match[kK]), at<float>(ws, L.score[kK]), cq, ck, 1, st));
    stage_end(HTTM_T_SELECT, st);
  }

  stage_begin(HTTM_T_MERGE_Q, st);
  CHECK_LAUNCH(launch_merge_q(dt, g.heads, g.N, g.nslots[kQ], q, cq.members, cq.off,
                              at<float>(ws, L.qsum), at<float>(ws, L.delta), at<uint32_t>(ws, L.radix), st));
  stage_end(HTTM_T_MERGE_Q, st);

  stage_begin(HTTM_T_OUTLIER, st);
  CHECK_LAUNCH(launch_outliers(at<float>(ws, L.delta), hn, pl->k_o, at<uint8_t>(ws, L.mask),
                               at<uint32_t>(ws, L.radix), st));
  stage_end(HTTM_T_OUTLIER, st);

  RestoreOut ro;
  ro.qt = at<void>(ws, L.qt);
  ro.lenq = reinterpret_cast<int32_t*>(idx + I.lenq.off);
  ro.cu_q = reinterpret_cast<int32_t*>(idx + I.cu_q.off);
  ro.tbase = at<int32_t>(ws, L.base);
  ro.ocnt = at<int32_t>(ws, L.ocnt);
  ro.fmembers = reinterpret_cast<int32_t*>(idx + I.fmembers.off);
  ro.foff = reinterpret_cast<int32_t*>(idx + I.foff.off);
  ro.slot = reinterpret_cast<int32_t*>(idx + I.slot.off);
  stage_begin(HTTM_T_RESTORE, st);
  CHECK_LAUNCH(launch_restore(dt, g.heads, g.N, g.nslots[kQ], q, cq.members, cq.off,
                              at<float>(ws, L.qsum), at<uint8_t>(ws, L.mask), ro, st));
  stage_end(HTTM_T_RESTORE, st);

  if (side) CHECK_LAUNCH(hipStreamWaitEvent(st, side->join, 0));
  s = attend_unmerge(pl, ws, idx, at<void>(ws, L.qt), out, st);
  if (s != HTTM_OK) return s;
  if (index) {
    index->plan_id = pl->id;
    index->valid = 1;
  }
  timing_end_call();
  return HTTM_OK;
}

}  // namespace

extern "C" {

const char* httm_status_string(httm_status s) {
  switch (s) {
    case HTTM_OK: return "ok";
    case HTTM_ERR_INVALID_ARG: return "invalid argument";
    case HTTM_ERR_UNSUPPORTED: return "unsupported";
    case HTTM_ERR_WORKSPACE: return "workspace too small";
    case HTTM_ERR_INDEX_MISMATCH: return "index does not belong to this plan";
    case HTTM_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* httm_last_error(void) { return g_err.c_str(); }

httm_status httm_plan_create(const httm_params* params, httm_plan** out) {
  if (!params || !out) return fail(HTTM_ERR_INVALID_ARG, "params and out must not be NULL");
  *out = nullptr;
  httm_plan* pl = new httm_plan();
  const httm_status s = build(*params, pl);
  if (s != HTTM_OK) {
    delete pl;
    return s;
  }
  g_err.clear();
  *out = pl;
  return HTTM_OK;
}

void httm_plan_destroy(httm_plan* plan) { delete plan; }

httm_status httm_plan_get_info(const httm_plan* pl, httm_plan_info* info) {
  if (!pl || !info) return fail(HTTM_ERR_INVALID_ARG, "NULL argument");
  info->n_tokens = pl->g.N;
  info->n_patch = pl->g.P;
  info->n_blocks = pl->g.nblocks;
  info->q_stride = pl->g.s[kQ];
  info->kv_stride = pl->g.s[kK];
  info->q_groups = pl->g.nslots[kQ];
  info->kv_len = pl->g.nslots[kK];
  info->n_outliers = pl->k_o;
  info->q_capacity = pl->q_cap;
  info->q_src = pl->g.nsrc[kQ];
  info->kv_src = pl->g.nsrc[kK];
  info->softmax_scale = pl->scale;
  return HTTM_OK;
}

httm_status httm_plan_get_blocks(const httm_plan* pl, httm_block* rows, int32_t cap) {
  if (!pl || (!rows && cap > 0) || cap < 0) return fail(HTTM_ERR_INVALID_ARG, "bad arguments");
  const int32_t n = cap < pl->g.nblocks ? cap : pl->g.nblocks;
  for (int32_t i = 0; i < n; ++i) rows[i] = pl->blocks[i];
  return HTTM_OK;
}

httm_status httm_workspace_size(const httm_plan* pl, size_t* bytes) {
  if (!pl || !bytes) return fail(HTTM_ERR_INVALID_ARG, "NULL argument");
  *bytes = pl->L.total;
  return HTTM_OK;
}

httm_status httm_index_size(const httm_plan* pl, size_t* bytes) {
  if (!pl || !bytes) return fail(HTTM_ERR_INVALID_ARG, "NULL argument");
  *bytes = pl->I.total;
  return HTTM_OK;
}

httm_status httm_index_header(const httm_plan* pl, void* host, size_t bytes) {
  if (!pl || !host) return fail(HTTM_ERR_INVALID_ARG, "NULL argument");
  if (bytes < sizeof(IndexHeader)) return fail(HTTM_ERR_INVALID_ARG, "host buffer smaller than the index header");
  std::memcpy(host, &pl->index_header, sizeof(IndexHeader));
  return HTTM_OK;
}

httm_status httm_debug_fail_launch(int32_t n) {
  if (n < 0) return fail(HTTM_ERR_INVALID_ARG, "n must be >= 0");
  g_fail_at.store(0);
  g_fail_tick.store(0);
  g_fail_at.store(n);
  return HTTM_OK;
}

httm_status httm_peak_mfma(int32_t iters, int32_t grid, float a, float b, float* out, void* stream,
                           double* flop) {
  if (!out) return fail(HTTM_ERR_INVALID_ARG, "out is NULL");
  if (iters < 8 || iters > (1 << 30) || iters % 8)
    return fail(HTTM_ERR_INVALID_ARG, "iters must be a multiple of 8 in [8, 2^30]");
  if (grid < 1 || grid > (1 << 20)) return fail(HTTM_ERR_INVALID_ARG, "grid must be in [1, 2^20]");
  if (flop) *flop = peak_flop_per_iter_wg() * (double)grid * (double)iters;
  CHECK_LAUNCH(launch_mfma_peak(iters, grid, a, b, out, reinterpret_cast<hipStream_t>(stream)));
  return HTTM_OK;
}

httm_status httm_peak_mfma_fp8(int32_t iters, int32_t grid, float* out, void* stream, double* flop) {
  if (!out) return fail(HTTM_ERR_INVALID_ARG, "out is NULL");
  if (iters < 4 || iters > (1 << 30) || iters % 4)
    return fail(HTTM_ERR_INVALID_ARG, "iters must be a multiple of 4 in [4, 2^30]");
  if (grid < 1 || grid > (1 << 20)) return fail(HTTM_ERR_INVALID_ARG, "grid must be in [1, 2^20]");
  if (flop) *flop = peak_flop_per_iter_wg_fp8() * (double)grid * (double)iters;
  CHECK_LAUNCH(launch_mfma_peak_fp8(iters, grid, out, reinterpret_cast<hipStream_t>(stream)));
  return HTTM_OK;
}

httm_status httm_index_export(const httm_plan* pl, const httm_index* index, void* host, size_t bytes,
                              void* stream) {
  if (!pl || !index || !index->dev || !host) return fail(HTTM_ERR_INVALID_ARG, "NULL argument");
  if (index->plan_id != pl->id || !index->valid)
    return fail(HTTM_ERR_INDEX_MISMATCH, "index was not filled by httm_layer with this plan");
  if (index->bytes < pl->I.total) return fail(HTTM_ERR_WORKSPACE, "index buffer smaller than httm_index_size()");
  if (bytes < pl->I.total) return fail(HTTM_ERR_INVALID_ARG, "host buffer smaller than httm_index_size()");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host, index->dev, pl->I.total, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(HTTM_ERR_DEVICE, "index copy to host failed");
  return HTTM_OK;
}

httm_status httm_index_import(const httm_plan* pl, const void* host, size_t bytes, httm_index* index,
                              void* stream) {
  if (!pl || !host || !index || !index->dev) return fail(HTTM_ERR_INVALID_ARG, "NULL argument");
  if (index->bytes < pl->I.total) return fail(HTTM_ERR_WORKSPACE, "index buffer smaller than httm_index_size()");
  if (bytes != pl->I.total) return fail(HTTM_ERR_INDEX_MISMATCH, "buffer size is not this plan's httm_index_size()");
  const char* buf = reinterpret_cast<const char*>(host);
  if (std::memcmp(buf + pl->I.header.off, &pl->index_header, sizeof(IndexHeader)) != 0)
    return fail(HTTM_ERR_INDEX_MISMATCH, "index header does not match this plan");
  if (!index_payload_ok(pl, buf)) return fail(HTTM_ERR_INDEX_MISMATCH, "index contents out of range");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  index->valid = 0;
  if (hipMemcpyAsync(index->dev, host, pl->I.total, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(HTTM_ERR_DEVICE, "index copy to the device failed");
  index->plan_id = pl->id;
  index->valid = 1;
  return HTTM_OK;
}

httm_status httm_dense_workspace_size(const httm_plan* pl, size_t* bytes) {
  if (!pl || !bytes) return fail(HTTM_ERR_INVALID_ARG, "NULL argument");
  *bytes = pl->dense_ws;
  return HTTM_OK;
}

httm_status httm_layer(const httm_plan* pl, void* ws, size_t ws_bytes, const void* q, const void* k,
                       const void* v, void* out, httm_index* index, void* stream) {
  httm_status s = check_common(pl, ws, ws_bytes, q, k, v, out, pl ? pl->L.total : 0);
  if (s != HTTM_OK) return s;
  if (index && (!index->dev || index->bytes < pl->I.total))
    return fail(HTTM_ERR_WORKSPACE, "index buffer smaller than httm_index_size()");
  if (index && ((uintptr_t)index->dev & 15)) return fail(HTTM_ERR_INVALID_ARG, "index must be 16-byte aligned");
  std::lock_guard<std::mutex> lock(g_launch_mu);
  SideStream* side = nullptr;
  if (!timing_serial()) {
    s = side_stream(&side);
    if (s != HTTM_OK) return s;
  }
  return enqueue_layer(pl, ws, index, q, k, v, out, reinterpret_cast<hipStream_t>(stream), side);
}

httm_status httm_noalloc_capacity(size_t* bytes) {
  if (!bytes) return fail(HTTM_ERR_INVALID_ARG, "NULL argument");
  *bytes = kNoAllocBytes;
  return HTTM_OK;
}

httm_status httm_layer_noalloc(const httm_plan* pl, const void* q, const void* k, const void* v, void* out,
                               void* stream) {
  if (!pl) return fail(HTTM_ERR_INVALID_ARG, "plan is NULL");
  if (pl->L.total > kNoAllocBytes)
    return fail(HTTM_ERR_WORKSPACE, "the layer needs " + std::to_string(pl->L.total) +
                                        " bytes of workspace; httm_layer_noalloc holds " +
                                        std::to_string(kNoAllocBytes) + " (use httm_layer with a workspace)");
  if (!q || !k || !v || !out) return fail(HTTM_ERR_INVALID_ARG, "q, k, v and out must not be NULL");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15)
    return fail(HTTM_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  std::lock_guard<std::mutex> lock(g_launch_mu);
  void* ws = nullptr;
  const httm_status s = scratch_ptr(&ws);
  if (s != HTTM_OK) return s;
  return enqueue_layer(pl, ws, nullptr, q, k, v, out, reinterpret_cast<hipStream_t>(stream), nullptr);
}

httm_status httm_layer_cached(const httm_plan* pl, void* ws, size_t ws_bytes, const httm_index* index,
                              const void* q, const void* k, const void* v, void* out, void* stream) {
  httm_status s = check_common(pl, ws, ws_bytes, q, k, v, out, pl ? pl->L.total : 0);
  if (s != HTTM_OK) return s;
  if (!index || !index->dev) return fail(HTTM_ERR_INVALID_ARG, "index is NULL");
  if (index->plan_id != pl->id || !index->valid)
    return fail(HTTM_ERR_INDEX_MISMATCH, "index was not filled by httm_layer with this plan");
  if (index->bytes < pl->I.total) return fail(HTTM_ERR_WORKSPACE, "index buffer smaller than httm_index_size()");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Geo& g = pl->g;
  const IndexLayout& I = pl->I;
  const int dt = pl->p.dtype;
  char* idx = reinterpret_cast<char*>(index->dev);
  std::lock_guard<std::mutex> lock(g_launch_mu);
  SideStream* side = nullptr;
  if (!timing_serial()) {
    s = side_stream(&side);
    if (s != HTTM_OK) return s;
  }
  hipStream_t kst = side ? side->st : st;  // stream of the K / V merge
  timing_begin_call();
  CHECK_LAUNCH(launch_zero_init(at<float>(ws, pl->L.kmax), g.heads, at<int>(ws, pl->L.fb), nullptr, 0, nullptr, 0,
                                st));
  if (side) {
    CHECK_LAUNCH(hipEventRecord(side->fork, st));
    CHECK_LAUNCH(hipStreamWaitEvent(kst, side->fork, 0));
  }
  stage_begin(HTTM_T_MERGE_KV, kst);
  CHECK_LAUNCH(launch_merge_kv(dt, g.heads, g.N, g.nslots[kK], pl->lk_pad, pl->scale * kLog2e, k, v,
                               reinterpret_cast<const int32_t*>(idx + I.k_members.off),
                               reinterpret_cast<const int32_t*>(idx + I.k_off.off),
                               at<void>(ws, pl->L.kt), at<void>(ws, pl->L.vt), at<float>(ws, pl->L.kmax), kst,
                               pl->p.partition == 1 ? reinterpret_cast<const int32_t*>(idx + I.lenk.off) : nullptr));
  stage_end(HTTM_T_MERGE_KV, kst);
  if (side) CHECK_LAUNCH(hipEventRecord(side->join, kst));
  stage_begin(HTTM_T_MERGE_Q, st);
  CHECK_LAUNCH(launch_merge_q_cached(dt, g.heads, g.N, pl->q_cap, q,
                                     reinterpret_cast<const int32_t*>(idx + I.fmembers.off),
                                     reinterpret_cast<const int32_t*>(idx + I.foff.off),
                                     reinterpret_cast<const int32_t*>(idx + I.lenq.off),
                                     at<void>(ws, pl->L.qt), st));
  stage_end(HTTM_T_MERGE_Q, st);
  if (side) CHECK_LAUNCH(hipStreamWaitEvent(st, side->join, 0));
  s = attend_unmerge(pl, ws, idx, at<void>(ws, pl->L.qt), out, st);
  if (s == HTTM_OK) timing_end_call();
  return s;
}

httm_status httm_attention_dense(const httm_plan* pl, void* ws, size_t ws_bytes, const void* q,
                                 const void* k, const void* v, void* out, void* stream) {
  httm_status s = check_common(pl, ws, ws_bytes, q, k, v, out, pl ? pl->dense_ws : 0);
  if (s != HTTM_OK) return s;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Geo& g = pl->g;
  const int dt = pl->p.dtype;
  const int pitch = ceil_div(g.N, 64) * 64;
  char* kc = reinterpret_cast<char*>(ws) + pl->dense_vt_bytes;
  float* kmax = reinterpret_cast<float*>(kc + pl->dense_kc_bytes);
  int* fb = reinterpret_cast<int*>(reinterpret_cast<char*>(kmax) + align256(pl->L.kmax.bytes));
  timing_begin_call();
  stage_begin(HTTM_T_MERGE_KV, st);
  CHECK_LAUNCH(launch_zero_init(kmax, g.heads, fb, nullptr, 0, nullptr, 0, st));
  CHECK_LAUNCH(launch_prep_dense(dt, g.heads, g.N, pitch, pl->scale * kLog2e, k, v, kc, ws, kmax, st));
  stage_end(HTTM_T_MERGE_KV, st);
  AttnShape a{};
  a.heads = g.heads;
  a.lk = g.N;
  a.k_rows = pitch;
  a.vt_pitch = pitch;
  a.lq_uniform = g.N;
  a.q_capacity = (int64_t)g.heads * g.N;
  a.scale = pl->scale;
  a.split = 1;
  a.lenk = nullptr;
  a.tail_split = 1;
  a.per_round = 0;
  a.tail_rows = 0;
  a.opart = a.lpart = a.mpart = nullptr;
  a.kmax = kmax;
  a.fb_count = fb;
  a.fb_list = fb + 1;
  stage_begin(HTTM_T_ATTN, st);
  CHECK_LAUNCH(launch_attention(dt, a, q, kc, ws, nullptr, out, st));
  stage_end(HTTM_T_ATTN, st);
  stage_begin(HTTM_T_ATTN_TAIL, st);
  CHECK_LAUNCH(launch_attention_tail(dt, a, q, kc, ws, nullptr, out, st));
  stage_end(HTTM_T_ATTN_TAIL, st);
  timing_end_call();
  return HTTM_OK;
}

httm_status httm_debug_size(const httm_plan* pl, int32_t item, size_t* bytes) {
  if (!pl || !bytes) return fail(HTTM_ERR_INVALID_ARG, "NULL argument");
  const size_t h = pl->g.heads, n = pl->g.N;
  const bool ga = pl->p.partition == 1;
  const size_t E = pl->esize;
  const bool gm = pl->p.partition == 2;
  const bool ga_item = item == HTTM_DBG_GA_VAR || item == HTTM_DBG_GA_ROLE || item == HTTM_DBG_GA_MATCH ||
                       item == HTTM_DBG_GA_SCORE || item == HTTM_DBG_KV_LEN;
  const bool block_item = item == HTTM_DBG_Q_MATCH || item == HTTM_DBG_Q_SCORE || item == HTTM_DBG_KV_MATCH ||
                          item == HTTM_DBG_KV_SCORE;
  const bool gm_item = item == HTTM_DBG_GM_METRIC || item == HTTM_DBG_GM_MATCH || item == HTTM_DBG_GM_SCORE;
  const bool fp8_item = item == HTTM_DBG_K8 || item == HTTM_DBG_KEXP || item == HTTM_DBG_Q8 || item == HTTM_DBG_QEXP;
  if ((ga_item && !ga) || (block_item && (ga || gm)) || (gm_item && !gm))
    return fail(HTTM_ERR_UNSUPPORTED, "this debug item does not exist under the plan's partition");
  if (fp8_item && !pl->p.attn_fp8) return fail(HTTM_ERR_UNSUPPORTED, "FP8 items need attn_fp8 = 1");
  switch (item) {
    case HTTM_DBG_GA_VAR:
    case HTTM_DBG_GA_MATCH:
    case HTTM_DBG_GA_SCORE: *bytes = 4 * 2 * h * n; break;
    case HTTM_DBG_GA_ROLE: *bytes = 2 * h * n; break;
    case HTTM_DBG_KV_LEN: *bytes = 4 * h; break;
    case HTTM_DBG_Q_MATCH:
    case HTTM_DBG_Q_SCORE: *bytes = 4 * h * pl->g.nsrc[kQ]; break;
    case HTTM_DBG_KV_MATCH:
    case HTTM_DBG_KV_SCORE: *bytes = 4 * h * pl->g.nsrc[kK]; break;
    case HTTM_DBG_Q_GROUP:
    case HTTM_DBG_KV_GROUP:
    case HTTM_DBG_DELTA:
    case HTTM_DBG_Q_SLOT: *bytes = 4 * h * n; break;
    case HTTM_DBG_OUTLIER: *bytes = h * n; break;
    case HTTM_DBG_CU_Q: *bytes = 4 * (h + 1); break;
    case HTTM_DBG_SELECT: *bytes = 16; break;
    case HTTM_DBG_ATTN_FALLBACK: *bytes = 4; break;
    case HTTM_DBG_KT:
    case HTTM_DBG_VT: *bytes = E * h * (size_t)pl->lk_pad * kD; break;
    case HTTM_DBG_QT: *bytes = E * (size_t)pl->q_cap * kD; break;
    case HTTM_DBG_GM_METRIC: *bytes = E * n * kD; break;
    case HTTM_DBG_GM_MATCH:
    case HTTM_DBG_GM_SCORE: *bytes = 4 * n; break;
    case HTTM_DBG_K8: *bytes = h * (size_t)pl->lk_pad * kD; break;
    case HTTM_DBG_KEXP: *bytes = 4 * h; break;
    case HTTM_DBG_Q8: *bytes = (size_t)pl->q_cap * kD; break;
    case HTTM_DBG_QEXP: *bytes = 4 * (size_t)pl->q_cap; break;
    default: return fail(HTTM_ERR_INVALID_ARG, "unknown debug item");
  }
  return HTTM_OK;
}

httm_status httm_debug_read(const httm_plan* pl, const void* ws, const httm_index* index, int32_t item,
                            void* host, size_t bytes, void* stream) {
  size_t need = 0;
  httm_status s = httm_debug_size(pl, item, &need);
  if (s != HTTM_OK) return s;
  if (!ws || !host) return fail(HTTM_ERR_INVALID_ARG, "NULL buffer");
  if (bytes < need) return fail(HTTM_ERR_WORKSPACE, "host buffer too small");
  const Layout& L = pl->L;
  const char* base = reinterpret_cast<const char*>(ws);
  if (index && (!index->dev || index->plan_id != pl->id))
    return fail(HTTM_ERR_INDEX_MISMATCH, "index was not filled with this plan");
  const char* idx = index ? reinterpret_cast<const char*>(index->dev) : base + L.index.off;
  const char* src = nullptr;
  switch (item) {
    case HTTM_DBG_Q_MATCH: src = base + L.match[kQ].off; break;
    case HTTM_DBG_Q_SCORE: src = base + L.score[kQ].off; break;
    case HTTM_DBG_KV_MATCH: src = base + L.match[kK].off; break;
    case HTTM_DBG_KV_SCORE: src = base + L.score[kK].off; break;
    case HTTM_DBG_Q_GROUP: src = base + L.q_group.off; break;
    case HTTM_DBG_KV_GROUP: src = base + L.k_group.off; break;
    case HTTM_DBG_DELTA: src = base + L.delta.off; break;
    case HTTM_DBG_OUTLIER: src = base + L.mask.off; break;
    case HTTM_DBG_Q_SLOT: src = idx + pl->I.slot.off; break;
    case HTTM_DBG_CU_Q: src = idx + pl->I.cu_q.off; break;
    case HTTM_DBG_SELECT: src = base + L.radix.off + 4 * 3 * 2048; break;
    case HTTM_DBG_ATTN_FALLBACK: src = base + L.fb.off; break;
    case HTTM_DBG_GA_VAR: src = base + L.ga_var.off; break;
    case HTTM_DBG_GA_ROLE: src = base + L.ga_role.off; break;
    case HTTM_DBG_GA_MATCH: src = base + L.ga_gdst.off; break;
    case HTTM_DBG_GA_SCORE: src = base + L.ga_gscore.off; break;
    case HTTM_DBG_KV_LEN: src = idx + pl->I.lenk.off; break;
    case HTTM_DBG_KT: src = base + L.kt.off; break;
    case HTTM_DBG_VT: src = base + L.vt.off; break;
    case HTTM_DBG_QT: src = base + L.qt.off; break;
    case HTTM_DBG_GM_METRIC: src = base + L.gm_metric.off; break;
    case HTTM_DBG_GM_MATCH: src = base + L.gm_dbg_match.off; break;
    case HTTM_DBG_GM_SCORE: src = base + L.gm_dbg_score.off; break;
    case HTTM_DBG_K8: src = base + L.k8.off; break;
    case HTTM_DBG_KEXP: src = base + L.kexp.off; break;
    case HTTM_DBG_Q8: src = base + L.q8.off; break;
    case HTTM_DBG_QEXP: src = base + L.qexp.off; break;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  CHECK_LAUNCH(hipMemcpyAsync(host, src, need, hipMemcpyDeviceToHost, st));
  CHECK_LAUNCH(hipStreamSynchronize(st));
  return HTTM_OK;
}

httm_status httm_set_timing(int32_t stage_mask) {
  if (stage_mask && !g_timing.created) {
    for (int k = 0; k < kSlots; ++k)
      for (int i = 0; i < 2 * HTTM_T_COUNT; ++i)
        if (hipEventCreate(&g_timing.ev[k][i]) != hipSuccess) return fail(HTTM_ERR_DEVICE, "hipEventCreate failed");
    g_timing.created = true;
  }
  g_timing.mask = stage_mask & ((1 << HTTM_T_COUNT) - 1);
  g_timing.serial = g_timing.mask != 0 && (stage_mask & HTTM_TIMING_SERIAL) != 0;
  g_timing.calls = 0;
  for (int k = 0; k < kSlots; ++k)
    for (int i = 0; i < HTTM_T_COUNT; ++i) g_timing.used[k][i] = false;
  return HTTM_OK;
}

httm_status httm_get_timing(float* ms, int32_t n, int32_t* calls) {
  if (!ms || n < 0) return fail(HTTM_ERR_INVALID_ARG, "bad arguments");
  if (!g_timing.created) return fail(HTTM_ERR_INVALID_ARG, "timing was never enabled");
  const int nc = g_timing.calls < kSlots ? g_timing.calls : kSlots;
  if (calls) *calls = nc;
  for (int i = 0; i < n && i < HTTM_T_COUNT; ++i) {
    double sum = 0.0;
    int cnt = 0;
    for (int k = 0; k < nc; ++k) {
      if (!g_timing.used[k][i]) continue;
      if (hipEventSynchronize(g_timing.ev[k][2 * i + 1]) != hipSuccess) return fail(HTTM_ERR_DEVICE, "event sync failed");
      float t = 0.f;
      if (hipEventElapsedTime(&t, g_timing.ev[k][2 * i], g_timing.ev[k][2 * i + 1]) != hipSuccess)
        return fail(HTTM_ERR_DEVICE, "event timing failed");
      sum += t;
      ++cnt;
    }
    ms[i] = cnt ? (float)(sum / cnt) : 0.f;
  }
  return HTTM_OK;
}

}  // extern "C"
