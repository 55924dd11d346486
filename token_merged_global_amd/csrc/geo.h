// Block geometry of the temporal reordering, shared by host planning and the
// kernels.  ("HTTM: Head-wise Temporal Token Merging for Faster VGGT", key
// design 2: the tokens of one spatial region of n_s patches in n_t adjacent
// frames are stacked into one merge block of n_b = n_s * n_t tokens.)
//
// A block is identified by (g, a): temporal group g (frames g*n_t ...), spatial
// run a (raster patches a*n_s ...).  Blocks are numbered b = g*A + a.  Inside a
// block the stack is frame-major by default (the plainest reading of the
// page's "stacking"): position i <-> frame f0 + i / run, patch j0 + i % run;
// frame-minor order (order 1) puts patch j0 + i / nf, frame f0 + i % nf.  Every per-block quantity follows in closed form from the
// block's shape (nf, run), of which there are at most four (full or last
// temporal group x full or last spatial run), so kernels need no block table:
// the merge counts r of those four shapes are computed once on the host and
// passed by value.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define GEO_HD __host__ __device__ __forceinline__
#else
#define GEO_HD inline
#endif

namespace httm {

constexpr int kD = 64;          // d_head
constexpr int kMaxBlock = 4096; // largest supported block (fits LDS sorts)
constexpr int kMaxHeads = 64;   // per-head prefix tables in LDS hold kMaxHeads + 1 entries
constexpr int kMaxFrameHW = 4096;  // geometry-aware partition: one frame's patches rank in LDS

enum Stream { kQ = 0, kK = 1 };

struct Geo {
  int32_t heads;
  int32_t F, T, HW, nsp;  // frames, tokens per frame, patches per frame, specials per frame
  int32_t n_s, n_t;       // spatial run, temporal group
  int32_t A, G;           // spatial runs per frame, temporal groups
  int32_t nf_last, run_last;
  int32_t N, P;           // tokens and patch tokens per head
  int32_t nblocks;
  int32_t s[2];           // destination stride per stream
  int32_t r[2][2][2];     // merged sources [stream][last group?][last run?]
  int32_t grp_slots[2];   // slots of one full temporal group (sum of n - r)
  int32_t grp_src[2];     // sources of one full temporal group
  int32_t nslots[2];      // slots per head incl. specials (G_q, L_k)
  int32_t nsrc[2];        // sources per head
  int32_t order;          // stacking inside a block: 0 frame-major, 1 frame-minor
};

struct BlockInfo {
  int32_t start, n, f0, nf, j0, run;
  int32_t nd, ns, r;      // destinations, sources, merged sources
  int32_t slot0, src0;    // first slot / first source of the block in its head
};

GEO_HD int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

GEO_HD BlockInfo block_info(const Geo& g, int32_t b, int st) {
  BlockInfo o;
  const int32_t gg = b / g.A, a = b % g.A;
  const int lastg = (gg == g.G - 1), lastr = (a == g.A - 1);
  o.nf = lastg ? g.nf_last : g.n_t;
  o.run = lastr ? g.run_last : g.n_s;
  o.n = o.nf * o.run;
  o.f0 = gg * g.n_t;
  o.j0 = a * g.n_s;
  o.start = gg * g.n_t * g.HW + o.nf * o.j0;
  const int32_t s = g.s[st];
  o.nd = ceil_div(o.n, s);
  o.ns = o.n - o.nd;
  o.r = g.r[st][lastg][lastr];
  // earlier blocks of this group are full spatial runs with nf frames
  const int32_t nfull = o.nf * g.n_s;
  const int32_t rfull = g.r[st][lastg][0];
  const int32_t ndfull = ceil_div(nfull, s);
  o.slot0 = gg * g.grp_slots[st] + a * (nfull - rfull);
  o.src0 = gg * g.grp_src[st] + a * (nfull - ndfull);
  return o;
}

// Divisor that splits a block position into (frame, patch): the run for
// frame-major stacking, the frame count for frame-minor.
GEO_HD int32_t block_divisor(const Geo& g, const BlockInfo& bi) { return g.order ? bi.nf : bi.run; }

// Original token id of block position i.
GEO_HD int32_t block_token(const Geo& g, const BlockInfo& bi, int32_t i) {
  const int32_t d = block_divisor(g, bi), q = i / d, r = i % d;
  const int32_t f = bi.f0 + (g.order ? r : q);
  const int32_t j = bi.j0 + (g.order ? q : r);
  return f * g.T + g.nsp + j;
}

// Block position of the k-th source (positions with i mod s != 0).
GEO_HD int32_t src_pos(int32_t k, int32_t s) { return k + k / (s - 1) + 1; }

// Quotient n / d by one float product: with rcp = fl((1 + 2^-20) / d), the
// rounded product fl(n * rcp) lies in [n/d, n/d + (n/d) 2^-19.8), and the
// gap from n/d up to the next integer is at least 1/d, so truncation gives
// the exact quotient for 0 <= n < 2^19 (checked exhaustively for d <= 4096).
GEO_HD float div_rcp(int32_t d) { return (1.0f + 0x1p-20f) / (float)d; }
GEO_HD int32_t div_small(int32_t n, float rcp) { return (int32_t)((float)n * rcp); }

// block_token with precomputed rcp = div_rcp(block_divisor(g, bi)).
GEO_HD int32_t block_token_r(const Geo& g, const BlockInfo& bi, int32_t i, float rcp) {
  const int32_t d = block_divisor(g, bi);
  const int32_t q = div_small(i, rcp), r = i - q * d;
  return (bi.f0 + (g.order ? r : q)) * g.T + g.nsp + bi.j0 + (g.order ? q : r);
}

}  // namespace httm
