// Host-side launchers of the HIP kernels.  Each enqueues on `stream` and
// returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geo.h"

namespace httm {

// Index arrays of one stream's merge partition, per head:
//   members [h][N]      token ids grouped by slot (ascending inside a slot)
//   off     [h][L+1]    slot -> first member
//   group   [h][N]      token -> slot
struct Csr {
  int32_t* members;
  int32_t* off;
  int32_t* group;
};

// streams: bit 0 = the query stream, bit 1 = the key stream (both: 3).
hipError_t launch_sim(const Geo& g, int dtype, const void* q, const void* k, int32_t* match_q,
                      float* score_q, int32_t* match_k, float* score_k, int streams, hipStream_t stream);

hipError_t launch_select(const Geo& g, const int32_t* match_q, const float* score_q,
                         const int32_t* match_k, const float* score_k, Csr q, Csr k, int streams,
                         hipStream_t stream);

// Means of K and V over the key partition: kt [h][lk_pad][64] (times kscale),
// vt [h][64][lk_pad]; kmax[h] = max over the head's merged keys of |kt row|
// (atomic max into a zeroed buffer).
// lenk (nullable): per-head key counts when they vary (slots past them stay
// zero rows); the offsets keep lk + 1 entries per head.
hipError_t launch_merge_kv(int dtype, int heads, int N, int lk, int lk_pad, float kscale, const void* k,
                           const void* v, const int32_t* members, const int32_t* off, void* kt,
                           void* vt, float* kmax, hipStream_t stream, const int32_t* lenk = nullptr);

// Query group sums (fp32) and deviation of every query to its group mean;
// also adds every deviation to hist0 (bits 31..21 of its pattern, the first
// radix pass of the outlier select; zeroed beforehand).
hipError_t launch_merge_q(int dtype, int heads, int N, int gq, const void* q,
                          const int32_t* members, const int32_t* off, float* qsum, float* delta,
                          uint32_t* hist0, hipStream_t stream);

// Global top-k_o of delta [h*N] -> mask.  scratch: outlier_scratch_words(total)
// words, zeroed beforehand, whose first outlier_hist0_words() hold the first
// pass.
size_t outlier_scratch_words(int64_t total);
int outlier_hist0_words();
hipError_t launch_outliers(const float* delta, int64_t total, int64_t k_o, uint8_t* mask,
                           uint32_t* scratch, hipStream_t stream);

// Outlier restore: packed Q~ rows, per-head lengths, final partition.
struct RestoreOut {
  void* qt;            // [q_capacity][64]
  int32_t* lenq;       // [h]
  int32_t* cu_q;       // [h+1]
  int32_t* tbase;      // [h][ceil(gq / 32)] scratch: slots of each tile of 32 groups, then its first slot
  int32_t* ocnt;       // [h][gq] scratch: outlier members per initial group
  int32_t* fmembers;   // [h][N]
  int32_t* foff;       // [h][N+1]
  int32_t* slot;       // [h][N] packed row per token
};
hipError_t launch_restore(int dtype, int heads, int N, int gq, const void* q,
                          const int32_t* members, const int32_t* off, const float* qsum,
                          const uint8_t* mask, RestoreOut o, hipStream_t stream);

// Cached mode: Q~ rows as means over the final query partition.
hipError_t launch_merge_q_cached(int dtype, int heads, int N, int64_t q_capacity, const void* q,
                                 const int32_t* fmembers, const int32_t* foff,
                                 const int32_t* lenq, void* qt, hipStream_t stream);

// Ragged attention: o[row] = softmax(scale q[row] k_h^T) v_h for the packed
// rows of every head, with k already multiplied by scale * log2(e) (scores
// in exp2 units); lenq == nullptr means every head has `lq_uniform` rows.
struct AttnShape {
  int heads;
  int lk;          // keys per head
  int k_rows;      // rows per head in the key buffer (whole 64-key tiles, zero past lk)
  int vt_pitch;    // keys per row of vt (multiple of 64, >= lk)
  int lq_uniform;  // used when lenq == nullptr
  int64_t q_capacity;
  float scale;
  int split;               // key splits (bf16); partial buffers needed when > 1
  int tail_split;          // splits of each XCD's tail query tiles (<= split: none)
  int per_round;           // query tiles per full round of one XCD (0: the device's, read at launch)
  int64_t tail_rows;       // partial rows reserved for the tail tiles' extra splits
  float* opart;            // [attention_partial_rows][64]
  float* lpart;            // [attention_partial_rows]
  float* mpart;            // [attention_partial_rows]
  const float* kmax;       // [heads] max |k row|
  const int32_t* lenk;     // [heads] keys per head when they vary (nullable: lk for every head)
  int* fb_count;           // [1] units queued for the exact kernel (zeroed by launch_zero_init)
  int* fb_list;            // [units]
  // FP8 scores (bf16 layers): non-null k8 selects them
  const uint8_t* k8 = nullptr;    // [heads][k_rows][64] e4m3 keys (launch_quantize_keys)
  const int32_t* kexp = nullptr;  // [heads] their scale exponents
  uint8_t* q8 = nullptr;          // [q_capacity][64] e4m3 queries as the kernel quantised them (nullable)
  int32_t* qexp = nullptr;        // [q_capacity] their exponents (nullable)
};
// Geometry-aware three-class partition (variance map, roles, global match)
// of both streams, producing per head the same CSR groups as the block-local
// matching: members / offsets over `bound` slots (trailing slots empty) and
// the slot of every token.
struct GaShape {
  int heads, N, Tf, nsp, H, W, F;
  int k_protect;  // protected patches per frame
  int bound;      // slots per head (upper bound of anchors)
  int max_src;    // upper bound of sources per head
  int dpitch;     // rows of the gathered destination matrix per (stream, head): >= destinations, multiple of 64
};
struct GaBuffers {
  float* var;          // [2][h][N] variance map
  uint8_t* role;       // [2][h][N]
  int32_t* fcnt;       // [2][h][F][3] per frame: anchors, destinations, sources
  int32_t* foff;       // [2][h][F][3] exclusive prefixes
  int32_t* tot;        // [2][h][3] totals (anchors = groups)
  int32_t* slot;       // [2][h][N] slot of anchors, -1 for sources
  int32_t* dst_list;   // [2][h][N] destination tokens (ascending)
  int32_t* dst_slot;   // [2][h][N] their slots
  int32_t* src_list;   // [2][h][N] source tokens (ascending)
  int32_t* gdst;       // [2][h][N] matched destination token of each source
  int32_t* gslot;      // [2][h][N] its slot
  float* gscore;       // [2][h][N] its cosine
  uint16_t* dg;        // bf16: [2][h][dpitch][64] destination rows, gathered
  float* dinv;         // bf16: [2][h][dpitch] their inverse norms
  uint64_t* best;      // [2][h][N] per source: packed best (key, destination index)
  float* snorm;        // [2][h][N] per source: norm term of its score
  int32_t* cnt;        // [2][h][bound] members per slot
  int32_t* tmp;        // [2][h][N] slot of every token (sort keys)
  int32_t* sort_keys;  // [2][h][N] sort scratch
  int32_t* sort_vals;  // [2][h][N] sort scratch
  uint32_t* sort_counts;  // sort_count_words(2 h, N)
  int32_t* grp_q;      // [h][N] slot of every token (query stream)
  int32_t* grp_k;
  int32_t* mem_q;      // [h][N] members, grouped by slot, ascending inside a slot
  int32_t* mem_k;
  int32_t* off_q;      // [h][bound + 1]
  int32_t* off_k;
  int32_t* lenk;       // [h] groups of the key stream (keys per head)
};
// In four phases, enqueued in order: 0 classes (variance, roles, per-frame
// offsets, anchor slots and lists), 1 destination gather (bf16), 2 the match
// (one launch), 3 groups (decode, offsets, placement, rank).
hipError_t launch_ga_partition(int dtype, const GaShape& s, const void* q, const void* k, const GaBuffers& b,
                               hipStream_t stream, int phase);

// Stable sort of token ids by slot, per segment of n tokens (keys [nseg][n],
// slots < 2^20): out lists the tokens of segment g (g < split: out_a + g*n,
// else out_b + (g - split)*n) by slot, equal slots in ascending token id.
// Scratch: tmp_keys, tmp_vals [nseg][n]; counts sort_count_words(nseg, n).
size_t sort_count_words(int nseg, int n);
hipError_t launch_sort_by_slot(const int32_t* keys, int nseg, int n, int32_t* tmp_keys, int32_t* tmp_vals,
                               uint32_t* counts, int32_t* out_a, int32_t* out_b, int split, hipStream_t stream);
// out[i] = in[0] + ... + in[i-1] for i < n; *total (nullable) = the sum of all.
// sums: scan_sum_words(n) words of scratch.
size_t scan_sum_words(int64_t n);
hipError_t launch_exclusive_scan(const int32_t* in, int64_t n, int32_t* out, int32_t* sums, int32_t* total,
                                 hipStream_t stream);

// Top-k of n floats: mask[i] = 1 for the k largest values (any finite sign),
// ties to the smaller index.  scratch: outlier_scratch_words(n) words
// (cleared by the launch itself).
hipError_t launch_topk(const float* vals, int64_t n, int64_t k, uint8_t* mask, uint32_t* scratch,
                       hipStream_t stream);
// Cosine argmax of `ns` sources over all destinations of one matrix x
// ([N][64], rows listed by src_list / dst_list, tot = {0, nd, ns}): the
// geometry-aware partition's gather and match with one head and one stream.
// best[src token] (zeroed by the caller) receives the packed maximum,
// snorm[src token] the source norm term.
hipError_t launch_global_match(int dtype, int N, const void* x, const int32_t* tot, const int32_t* dst_list,
                               const int32_t* src_list, int ns, uint16_t* dg, float* dinv, int dpitch,
                               uint64_t* best, float* snorm, hipStream_t stream);

// Head-shared global matching (partition 2): one partition from the keys
// averaged over heads, copied to the query and key CSR of every head.
struct GmShape {
  int heads, N, Tf, nsp, HW;
  int nd, ns, r;  // destinations, sources, merged sources
  int L;          // slots (N - r)
  int dpitch;     // gathered destination rows (multiple of 64)
};
struct GmBuffers {
  void* metric;        // [N][64] element type
  int32_t* tot;        // [3]
  int32_t* dst_list;   // [nd]
  int32_t* src_list;   // [ns]
  uint16_t* dg;        // bf16: [dpitch][64]
  float* dinv;         // bf16: [dpitch]
  uint64_t* best;      // [N]
  float* snorm;        // [N]
  int32_t* match;      // [ns] destination index per source
  float* score;        // [ns]
  uint8_t* sel;        // [ns] merged sources
  uint32_t* topk;      // outlier_scratch_words(ns)
  int32_t* unsel;      // [ns]
  int32_t* urank;      // [ns]
  int32_t* scan_sums;  // scan_sum_words(ns)
  int32_t* keys;       // [N] slot of every token (also the token -> slot map)
  int32_t* sort_keys;  // [N]
  int32_t* sort_vals;  // [N]
  uint32_t* sort_counts;  // sort_count_words(1, N)
  int32_t* members;    // [N]
  int32_t* off;        // [L + 1]
  int32_t* dbg_match;  // [N] matched destination token of every source, -1 otherwise
  float* dbg_score;    // [N] its cosine, 0 otherwise
  Csr q, k;            // per-head CSR of both streams (written for every head)
};
// Three phases, enqueued in order: 0 metric and lists, 1 the match (one
// launch on bf16 after the destination gather), 2 scores, top-r, slots,
// sort, offsets and the per-head copies.
hipError_t launch_global_partition(int dtype, const GmShape& s, const void* k, const GmBuffers& b,
                                   hipStream_t stream, int phase);

// Key splits for a layer of q_capacity packed rows; rows per work unit.
int attention_split(int64_t q_capacity, int heads);
int attention_rows_per_unit();
// Tail splitting for `split` key splits (host only; tail_split == split
// disables it).  per_round stays 0: the launch reads the device's tiles per
// round; capacities assume the most tail tiles the schedule allows.
struct AttnTail {
  int tail_split, per_round;
  int64_t tail_rows;
};
AttnTail attention_tail(int split);
// Workgroups of the main attention launch (also the capacity the exact-path
// queue needs) and rows of each partial buffer, for a shape.
int64_t attention_workgroups(int dtype, const AttnShape& s);
int64_t attention_partial_rows(const AttnShape& s);
// Zero, before a layer's producers run: kmax[heads] (atomic max target of the
// K~ producer), the exact-path counter, and optionally the outlier radix
// scratch (radix_words) and the per-group outlier counts (ocnt_words).
// Words of the header at the start of a merge index (identity of the plan
// that filled it; written by the layer's first kernel).
struct IndexHeader {
  uint32_t w[16];
};
hipError_t launch_zero_init(float* kmax, int heads, int* fb_count, uint32_t* radix, int radix_words,
                            int32_t* ocnt, int64_t ocnt_words, hipStream_t stream,
                            const IndexHeader* hdr = nullptr, uint32_t* hdr_dst = nullptr);
// The main attention kernel, then the tail: exact recompute of the units the
// main kernel queued and (key splits > 1) the combine of the partials.
hipError_t launch_attention(int dtype, const AttnShape& s, const void* q, const void* k,
                            const void* vt, const int32_t* lenq, void* o, hipStream_t stream);
hipError_t launch_attention_tail(int dtype, const AttnShape& s, const void* q, const void* k,
                                 const void* vt, const int32_t* lenq, void* o, hipStream_t stream);

// FP8 (OCP e4m3) scores.  Keys: a power-of-two scale per head puts the
// head's largest |K~| in [128, 256); partial maxima first (kpart: [heads]
// [kKeyAmaxChunks]), then every element of kt [heads][k_rows][64] (bf16)
// rounded to nearest-even e4m3 into k8, and kexp[h] the exponent.
constexpr int kKeyAmaxChunks = 64;
hipError_t launch_quantize_keys(int heads, int k_rows, const void* kt, float* kpart, uint8_t* k8,
                                int32_t* kexp, hipStream_t stream);
// The FP8 main and exact attention kernels (called by launch_attention /
// launch_attention_tail when s.k8 is set).
int attention_fp8_per_round(int split);
hipError_t launch_attention_fp8(const AttnShape& s, const void* q, const void* vt, const int32_t* lenq, void* o,
                                hipStream_t stream);
hipError_t launch_attention_fp8_exact(const AttnShape& s, const void* q, const void* vt, const int32_t* lenq,
                                      void* o, hipStream_t stream);

// out[h][n] = o[slot[h][n]]
hipError_t launch_unmerge(int dtype, int heads, int N, const int32_t* slot, const void* o,
                          void* out, hipStream_t stream);

// Unmerged baseline inputs: kc = k * kscale ([h][pitch][64]); vt[h][c][n] =
// v[h][n][c]; both zero for n in [N, pitch).
hipError_t launch_prep_dense(int dtype, int heads, int N, int pitch, float kscale, const void* k,
                             const void* v, void* kc, void* vt, float* kmax, hipStream_t stream);


// Measured-peak micro-benchmark: `grid` workgroups of peak_threads() lanes,
// each lane `iters` (a multiple of 8) x 8 independent 16x16x32 bf16 MFMAs on
// pseudo-random operands scaled by a and b; out[grid * peak_threads()]
// receives each lane's accumulator sum (layout in k_peak.hip).
int peak_threads();
double peak_flop_per_iter_wg();
hipError_t launch_mfma_peak(int iters, int grid, float a, float b, float* out, hipStream_t stream);
// The same for v_mfma_scale_f32_32x32x64_f8f6f4 on e4m3 operands (4 chains
// per wave, `iters` a multiple of 4; layout in k_peak.hip).
double peak_flop_per_iter_wg_fp8();
hipError_t launch_mfma_peak_fp8(int iters, int grid, float* out, hipStream_t stream);

}  // namespace httm
