/*
 * httm.h -- C ABI of an MI355X (gfx950) implementation of HTTM's head-wise
 * temporal token-merged global-attention layer.
 *
 * What the layer computes ("HTTM: Head-wise Temporal Token Merging for Faster
 * VGGT", papernotes.org summary, "overall framework" and key designs 1-3):
 *
 *   1. temporal reordering: the patch tokens of one spatial region (n_s
 *      raster-order patches) in n_t adjacent frames form one merge block of
 *      n_b = n_s * n_t tokens (key design 2);
 *   2. per head and per stream (Q, then K), inside each block: cosine
 *      similarity of every source token to every destination token
 *      (RowNorm(S) RowNorm(D)^T), best destination per source, the r sources
 *      with the highest similarity merge into their destination, a merged
 *      token is the mean of its members; V follows K's groups (key design 1);
 *   3. queries only: L2 deviation of every query to its merged token, a single
 *      top-d% over all heads and tokens picks outliers, whose contribution is
 *      subtracted from their merged token and which are restored as separate
 *      tokens (key design 3);
 *   4. attention of the shortened, per-head ragged Q~ over K~ / V~;
 *   5. unmerge: each output row is copied back to every token it stands for,
 *      at its original index (key designs 1 and 2).
 *
 * The cached mode reuses the merge indices of an earlier layer ("LiteVGGT:
 * Boosting Vanilla VGGT via Geometry-aware Cached Token Merging",
 * papernotes.org summary, key design 3): only the means are recomputed.
 *
 * Conventions
 *   - q, k, v, out: device memory, contiguous [heads][N][64], N =
 *     frames * (n_special + grid_h * grid_w), token n = f*T + t with the first
 *     n_special slots of each frame special (never merged).  Element type is
 *     params.dtype (fp32 or bf16); out has the same type.  16-byte aligned.
 *   - Ownership: the caller owns every device buffer (inputs, output,
 *     workspace, index).  The library never allocates or frees device memory.
 *     Plans are host objects owned by the caller; they are immutable and may
 *     be shared between threads.
 *   - Asynchrony: httm_layer, httm_layer_cached and httm_attention_dense only
 *     enqueue kernels on `stream` (a hipStream_t; NULL = the default stream)
 *     and never synchronise.  Arguments are validated on the host before any
 *     launch; on an error nothing is enqueued and no output is written.  A
 *     launch failure returns HTTM_ERR_DEVICE; asynchronous device faults
 *     surface at the caller's next synchronisation.
 *   - Calls that share a workspace or index buffer must be ordered on one
 *     stream; concurrent calls need separate buffers.
 *   - httm_layer runs the key branch (K similarity, K selection, K/V merge)
 *     and httm_layer_cached the K/V merge on a library-owned stream of the
 *     current device (created on first use, default priority) that waits for
 *     the caller's stream and is joined back into it with events before the
 *     attention, so the caller sees one ordered stream.
 *     Enqueueing is serialised by an internal lock.
 *   - Sizes: validation requires heads * N < 2^31, N < 2^24 (32-bit offsets
 *     into a head's merged keys), n_s * n_t <= 4096 and heads <= 64
 *     (HTTM_ERR_UNSUPPORTED otherwise).
 */
#ifndef HTTM_H_
#define HTTM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HTTM_OK = 0,
  HTTM_ERR_INVALID_ARG = 1,    /* out-of-range parameter or NULL pointer */
  HTTM_ERR_UNSUPPORTED = 2,    /* d_head != 64, n_s * n_t > 4096, heads > 64, N >= 2^24,
                                  attn_fp8 on an fp32 layer; partitions 1 and 2: N >= 2^20, and
                                  for partition 1 more than 4096 patches per frame; a debug item
                                  that the plan's partition (or attn_fp8 = 0) does not produce */
  HTTM_ERR_WORKSPACE = 3,      /* workspace or index buffer smaller than required */
  HTTM_ERR_INDEX_MISMATCH = 4, /* index made by another plan, or never filled */
  HTTM_ERR_DEVICE = 5          /* a HIP call or a kernel launch failed */
} httm_status;

typedef enum { HTTM_F32 = 0, HTTM_BF16 = 1 } httm_dtype;

/* Layer parameters.  Ratios are binary64 so that r = floor(ratio * n) and
 * k_o = floor(d * h * N / 100) round exactly as written (0.9f would give
 * floor(0.9f * 3840) = 3455).  The HTTM page's settings are n_s = 128, n_t = 30, query
 * merge 90 % with 10 % outliers, key/value merge 70 % (HTTM page, "training
 * strategy / settings"). */
typedef struct {
  int32_t heads;         /* h >= 1 */
  int32_t d_head;        /* must be 64 */
  int32_t frames;        /* F >= 1 */
  int32_t grid_h, grid_w;/* patch grid per frame */
  int32_t n_special;     /* leading special tokens per frame (never merged) */
  int32_t n_s;           /* spatial run: consecutive raster-order patches per block */
  int32_t n_t;           /* temporal group: adjacent frames per block; last group may be shorter */
  double q_ratio;        /* fraction of each block's queries merged away, [0, 1) */
  double kv_ratio;       /* fraction of each block's keys merged away, [0, 1) */
  double outlier_pct;    /* d in [0, 100]: percent of heads*N queries restored */
  int32_t q_dst_stride;  /* destination stride for Q; 0 = max(4, ceil(1/(1-q_ratio))) */
  int32_t kv_dst_stride; /* destination stride for K; 0 = max(4, ceil(1/(1-kv_ratio))) */
  int32_t block_order;   /* stacking inside a block: 0 = frame-major, 1 = frame-minor */
  float softmax_scale;   /* 0 = 1/sqrt(d_head) */
  int32_t dtype;         /* httm_dtype of q, k, v, out */
  int32_t partition;     /* 0 = HTTM temporal blocks (default); 1 = geometry-aware three-class
                            partition (LiteVGGT page, key designs 1-3) of both streams, per
                            head: q_ratio, kv_ratio, strides and block_order do not apply
                            (n_s, n_t are still validated); the group count, and with it
                            the keys per head, varies by head and input, up to the bound
                            frames * n_special + H*W + (frames - 1) * (protected +
                            ceil(H/2) * ceil(W/2)) (at most N), which sizes q_groups and
                            kv_len in httm_plan_info.  Limits: at most 4096 patches per
                            frame and N < 2^20 */
                         /* 2 = one head-shared partition from global matching (the merging
                            the HTTM page contrasts itself with, research background and key
                            designs 1-2): the keys averaged over heads, every patch token in
                            original order as one block, every 4th a destination, the
                            floor(kv_ratio * patches) most similar sources merged; the same
                            groups serve the queries and keys of every head (deviation,
                            outlier restore, attention and unmerge per head as usual);
                            q_ratio, strides and block_order do not apply.  Limit: N < 2^20 */
  double protect_pct;    /* partition 1: percent of each frame's patches protected, [0, 100]
                            (the page uses 10); protected = floor(protect_pct / 100 * H*W) */
  int32_t attn_split;    /* bf16 attention: key ranges per query tile whose partial results are
                            combined in a fixed order; 0 = the library's choice (4), else 1, 2, 4
                            or 8 (fp32 layers always use 1).  Outputs agree to rounding */
  int32_t attn_fp8;      /* bf16 layers: 1 = attention scores from FP8 operands (LiteVGGT page,
                            training strategy and ablations: FP8 quantisation for inference;
                            our own OCP e4m3 form): every merged query row and every head's
                            merged keys get a power-of-two scale that puts their largest
                            magnitude in [128, 256), values round to nearest-even e4m3, the
                            products and sums are exact / fp32; probabilities and merged
                            values stay bf16.  0 = bf16 scores (default).  Merge indices do
                            not depend on it (an index serves both) */
} httm_params;

typedef struct httm_plan httm_plan;

/* Cached merge indices (LiteVGGT page, key design 3).  `dev` points to
 * caller-owned device memory of httm_index_size() bytes.  httm_layer fills it
 * when given and sets plan_id and valid; httm_layer_cached checks both on the
 * host. */
typedef struct {
  uint64_t plan_id;
  void* dev;
  size_t bytes;
  int32_t valid;
} httm_index;

/* Sizes that follow from the parameters alone (host-side, no device calls). */
typedef struct {
  int64_t n_tokens;      /* N */
  int64_t n_patch;       /* F * grid_h * grid_w */
  int32_t n_blocks;
  int32_t q_stride, kv_stride;
  int64_t q_groups;      /* G_q: query groups per head before outlier restore, specials included */
  int64_t kv_len;        /* L_k: merged keys per head, specials included */
  int64_t n_outliers;    /* k_o = floor(d * heads * N / 100) */
  int64_t q_capacity;    /* heads * G_q + k_o: upper bound of the packed Q~ rows */
  int64_t q_src, kv_src; /* source tokens per head (Q stream, K stream) */
  float softmax_scale;   /* resolved scale */
} httm_plan_info;

/* Per-block row of the host block table (temporal reordering, HTTM page key
 * design 2).  Blocks are ordered by temporal group, then spatial run; a
 * block's tokens occupy reordered positions [start, start + n). */
typedef struct {
  int32_t start, n;
  int32_t f0, nf;        /* frames f0 .. f0+nf-1 */
  int32_t j0, run;       /* patches j0 .. j0+run-1 of each frame */
  int32_t q_dst, q_src, q_r;   /* destinations, sources, merged sources (Q) */
  int32_t kv_dst, kv_src, kv_r;
  int32_t q_slot0, kv_slot0;   /* first merged slot of this block in its head */
  int32_t q_src0, kv_src0;     /* first source of this block in its head */
} httm_block;

/* Validate `params` and build a plan.  Host only; never touches the device.
 * Returns HTTM_ERR_INVALID_ARG / HTTM_ERR_UNSUPPORTED on bad parameters. */
httm_status httm_plan_create(const httm_params* params, httm_plan** out);
void httm_plan_destroy(httm_plan* plan);
httm_status httm_plan_get_info(const httm_plan* plan, httm_plan_info* info);
/* Copies min(n_blocks, cap) rows into `rows` (host memory). */
httm_status httm_plan_get_blocks(const httm_plan* plan, httm_block* rows, int32_t cap);

/* Device bytes the caller must provide as workspace / index buffer. */
httm_status httm_workspace_size(const httm_plan* plan, size_t* bytes);
httm_status httm_index_size(const httm_plan* plan, size_t* bytes);

/* One full HTTM layer: q, k, v -> out.  `index` may be NULL; if given, the
 * merge indices of this layer are written to index->dev for later
 * httm_layer_cached calls. */
httm_status httm_layer(const httm_plan* plan, void* ws, size_t ws_bytes,
                       const void* q, const void* k, const void* v, void* out,
                       httm_index* index, void* stream);

/* httm_layer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same layer, with no workspace argument and no merge index.  Its workspace
 * is a static device array of httm_noalloc_capacity() bytes (64 MiB) that
 * the library holds on every GPU it runs on until the process ends; a plan
 * whose httm_workspace_size() exceeds it gets HTTM_ERR_WORKSPACE before any
 * launch.  Every launch goes to `stream` (no library stream is created) and
 * nothing is allocated or freed.  All calls on one GPU share that GPU's
 * array, which keeps the last call's contents (the layer clears what it
 * needs zeroed): calls that may overlap on one GPU (other streams, other
 * threads' streams) race and must be ordered by the caller. */
httm_status httm_noalloc_capacity(size_t* bytes);
httm_status httm_layer_noalloc(const httm_plan* plan, const void* q, const void* k, const void* v, void* out,
                               void* stream);

/* A layer that reuses the reordering, final query partition and key
 * partition held in `index` (LiteVGGT page, key design 3): means of this
 * layer's q, k, v over the cached groups, attention, unmerge. */
httm_status httm_layer_cached(const httm_plan* plan, void* ws, size_t ws_bytes,
                              const httm_index* index,
                              const void* q, const void* k, const void* v, void* out,
                              void* stream);

/* Move a filled index through host memory (LiteVGGT page, key design 3:
 * the merge indices of one layer serve the following layers; exporting them
 * lets a caller keep or ship them).  Both synchronise `stream`.
 *
 * httm_index_export copies httm_index_size() bytes of `index` (filled by
 * httm_layer with this plan) into `host` (at least that many bytes).  The
 * bytes start with a header naming the plan's parameters and geometry.
 * HTTM_ERR_INDEX_MISMATCH if `index` was not filled with this plan.
 *
 * httm_index_import copies `host` (exactly httm_index_size() bytes, as
 * exported by a plan with the same parameters) into index->dev and marks the
 * index filled for this plan.  The header must match this plan and the
 * contents must stay in range (offsets rising from 0 to N, token ids below N,
 * packed rows inside their head), else HTTM_ERR_INDEX_MISMATCH and the index
 * is left unfilled.  index->dev is caller-owned device memory of at least
 * httm_index_size() bytes (HTTM_ERR_WORKSPACE otherwise). */
httm_status httm_index_export(const httm_plan* plan, const httm_index* index, void* host, size_t bytes,
                              void* stream);
/* The 64-byte header an index of this plan starts with, written to `host`
 * (at least 64 bytes; host only, no device calls): for callers that
 * assemble an index in host memory before httm_index_import. */
httm_status httm_index_header(const httm_plan* plan, void* host, size_t bytes);
httm_status httm_index_import(const httm_plan* plan, const void* host, size_t bytes, httm_index* index,
                              void* stream);

/* Exact softmax(scale q k^T) v per head with nothing merged, on the same
 * attention kernel (the unmerged baseline).  Needs
 * httm_dense_workspace_size() bytes of workspace. */
httm_status httm_dense_workspace_size(const httm_plan* plan, size_t* bytes);
httm_status httm_attention_dense(const httm_plan* plan, void* ws, size_t ws_bytes,
                                 const void* q, const void* k, const void* v, void* out,
                                 void* stream);

/* Intermediates of the last httm_layer on `ws`, for staged comparison with
 * an independent implementation.  Synchronises `stream` and copies to host
 * memory.  `index` is the index that call filled (NULL if it was given none):
 * HTTM_DBG_Q_SLOT and HTTM_DBG_CU_Q are read from it.  Layouts (per head h,
 * all int32 unless noted):
 *   HTTM_DBG_Q_MATCH / KV_MATCH: [h][src] matched destination as an original
 *       token id (sources ordered by block, then block position);
 *   HTTM_DBG_Q_SCORE / KV_SCORE: [h][src] float cosine of that match;
 *   HTTM_DBG_Q_GROUP / KV_GROUP: [h][N] merged slot of every token before
 *       outlier restore (query) / final (key);
 *   HTTM_DBG_DELTA: [h][N] float deviation;
 *   HTTM_DBG_OUTLIER: [h][N] uint8 outlier mask;
 *   HTTM_DBG_Q_SLOT: [h][N] packed row of Q~ that token n reads at unmerge;
 *   HTTM_DBG_CU_Q: [h+1] prefix of per-head Q~ lengths;
 *   HTTM_DBG_SELECT: [4] uint32 {threshold bits, count above, ties taken, k_o};
 *   HTTM_DBG_ATTN_FALLBACK: [1] int32 attention work units that the exact
 *       (running-max) kernel recomputed because their rows' probabilities
 *       underflowed against the norm bound.
 * Geometry-aware partition only (the four MATCH / SCORE items above return
 * HTTM_ERR_UNSUPPORTED there), [2][h][N] with stream 0 = Q, 1 = K:
 *   HTTM_DBG_GA_VAR: float token variance map (0 for special tokens);
 *   HTTM_DBG_GA_ROLE: uint8 class: 0 source, 1 destination, 2 protected,
 *       3 special;
 *   HTTM_DBG_GA_MATCH: matched destination token of every source, -1 for
 *       every other token;
 *   HTTM_DBG_GA_SCORE: float cosine of that match (0 for non-sources);
 *   HTTM_DBG_KV_LEN: [h] keys per head (the key stream's group count).
 * Merged rows, in the layer's element type (bf16 bit patterns or fp32), as
 * the attention kernel reads them (also after httm_layer_cached):
 *   HTTM_DBG_KT: [h][L_k padded to 64][64] merged keys, each the mean of its
 *       group multiplied by softmax_scale * log2(e) (rows past L_k are 0);
 *   HTTM_DBG_VT: [h][64][L_k padded to 64] merged values, transposed;
 *   HTTM_DBG_QT: [q_capacity][64] packed merged queries, head h's rows at
 *       [cu_q[h], cu_q[h+1]) (rows past cu_q[h] are unspecified).
 * Head-shared partition only (partition 2):
 *   HTTM_DBG_GM_METRIC: [N][64] the head-mean keys matched on (element type);
 *   HTTM_DBG_GM_MATCH: [N] int32 matched destination token of every source,
 *       -1 for every other token;
 *   HTTM_DBG_GM_SCORE: [N] float cosine of that match (0 for non-sources).
 * FP8 scores only (attn_fp8 = 1), the operands of the last layer's score
 * product as e4m3 bytes (value = code * 2^-exponent):
 *   HTTM_DBG_K8: [h][L_k padded to 64][64] merged keys (as HTTM_DBG_KT);
 *   HTTM_DBG_KEXP: [h] int32 key scale exponent per head;
 *   HTTM_DBG_Q8: [q_capacity][64] packed merged queries (as HTTM_DBG_QT);
 *   HTTM_DBG_QEXP: [q_capacity] int32 scale exponent per query row. */
typedef enum {
  HTTM_DBG_Q_MATCH = 0, HTTM_DBG_Q_SCORE, HTTM_DBG_KV_MATCH, HTTM_DBG_KV_SCORE,
  HTTM_DBG_Q_GROUP, HTTM_DBG_KV_GROUP, HTTM_DBG_DELTA, HTTM_DBG_OUTLIER,
  HTTM_DBG_Q_SLOT, HTTM_DBG_CU_Q, HTTM_DBG_SELECT, HTTM_DBG_ATTN_FALLBACK,
  HTTM_DBG_GA_VAR, HTTM_DBG_GA_ROLE, HTTM_DBG_GA_MATCH, HTTM_DBG_GA_SCORE, HTTM_DBG_KV_LEN,
  HTTM_DBG_KT, HTTM_DBG_VT, HTTM_DBG_QT,
  HTTM_DBG_GM_METRIC, HTTM_DBG_GM_MATCH, HTTM_DBG_GM_SCORE,
  HTTM_DBG_K8, HTTM_DBG_KEXP, HTTM_DBG_Q8, HTTM_DBG_QEXP,
  HTTM_DBG_COUNT
} httm_debug_item;
httm_status httm_debug_size(const httm_plan* plan, int32_t item, size_t* bytes);
httm_status httm_debug_read(const httm_plan* plan, const void* ws, const httm_index* index,
                            int32_t item, void* host, size_t bytes, void* stream);

/* Per-stage launch timing.  httm_set_timing(mask) records HIP events on the
 * call's stream around every stage whose bit (1 << httm_timing_stage) is set,
 * for the next calls of httm_layer / httm_layer_cached /
 * httm_attention_dense (a ring of 32 calls; 0 turns recording off and every
 * call resets the count).  httm_get_timing writes, per stage, the mean
 * milliseconds between the events over the recorded calls that ran that
 * stage (0 if none) and the number of recorded calls; it synchronises on
 * the events.  Host-side state, not thread-safe. */
/* In httm_layer the key branch (K similarity, K selection, K/V merge) runs on
 * the library stream concurrently with the query branch: HTTM_T_SIM_K,
 * HTTM_T_SELECT_K and HTTM_T_MERGE_KV time its three launches there,
 * HTTM_T_SIM and HTTM_T_SELECT the query stream's similarity and selection.
 * With partition = 1, HTTM_T_SIM times the whole geometry-aware partition of
 * both streams (on the caller's stream) and HTTM_T_GA_MATCH its global cosine
 * match alone (one launch); the two selection stages and HTTM_T_SIM_K are not
 * recorded.  With partition = 2 the same two stages time the head-shared
 * partition (metric, match, top-r, groups, per-head copies) and its global
 * match kernel.  httm_layer_cached records HTTM_T_MERGE_KV (its K/V merge, on the
 * library stream) and HTTM_T_MERGE_Q (its query means); httm_attention_dense
 * records HTTM_T_MERGE_KV for its input preparation. */
typedef enum {
  HTTM_T_SIM = 0, HTTM_T_SELECT, HTTM_T_MERGE_KV, HTTM_T_MERGE_Q, HTTM_T_OUTLIER,
  HTTM_T_RESTORE,
  HTTM_T_ATTN,       /* the main attention kernel (one launch) */
  HTTM_T_UNMERGE,
  HTTM_T_ATTN_TAIL,  /* exact recompute of queued units + combine of key splits */
  HTTM_T_GA_MATCH,   /* partition = 1: the global match kernel (one launch) */
  HTTM_T_SIM_K,      /* key stream similarity (library stream) */
  HTTM_T_SELECT_K,   /* key stream selection (library stream) */
  HTTM_T_KEY_FP8,    /* attn_fp8: the merged keys' scale and e4m3 rounding (two launches) */
  HTTM_T_COUNT
} httm_timing_stage;
/* With HTTM_TIMING_SERIAL in the mask (and at least one stage bit), the
 * timed httm_layer / httm_layer_cached calls enqueue every launch on the
 * caller's stream instead of forking the key branch onto the library
 * stream: each stage then times its kernels running alone on the GPU (for
 * per-kernel rooflines).  Results are bit-identical either way. */
#define HTTM_TIMING_SERIAL (1 << 30)
httm_status httm_set_timing(int32_t stage_mask);
httm_status httm_get_timing(float* ms, int32_t n, int32_t* calls);

/* Test hook of the error path: the n-th launch that the library checks
 * after this call (counting over all following calls; 0 turns it off)
 * reports HTTM_ERR_DEVICE ("forced launch failure") instead of being
 * enqueued, once.  The launches before it are enqueued as usual, so a
 * layer can fail part way; later calls run normally.  Not thread-safe. */
httm_status httm_debug_fail_launch(int32_t n);

/* Measured-peak micro-benchmark (not part of a layer): `grid` workgroups of
 * 256 lanes, every lane `iters` x 8 independent v_mfma_f32_16x16x32_bf16,
 * with no memory traffic in the loop, enqueued on `stream`.  Operands: lane
 * g (global id) holds 8 pairs (A_j, B_j) of 8 bf16 values; with
 * h = hash(64 g + 8 j + e) (the xorshift-multiply hash in k_peak.hip),
 * A_j[e] = bf16(a * ((h & 0xffff) - 32768) / 32768) and
 * B_j[e] = bf16(b * ((h >> 16) - 32768) / 32768); in every group of 8
 * iterations, step s accumulates A_j times B_((j + s) mod 8) into chain j
 * (operands change from one MFMA to the next, as real data does).  `out`
 * (device, caller-owned) receives grid * 256 floats, each lane's sum of its
 * 8 chains' 4 accumulator elements.  *flop (nullable) = the launch's MFMA
 * FLOP (grid * iters * 524,288).  Warm launches of tens of milliseconds
 * measure the matrix rate the GPU sustains, against which kernel fractions
 * are also reported.  iters a multiple of 8 in [8, 2^30], grid in
 * [1, 2^20]; else HTTM_ERR_INVALID_ARG, with nothing enqueued. */
httm_status httm_peak_mfma(int32_t iters, int32_t grid, float a, float b, float* out, void* stream,
                           double* flop);

/* The FP8 counterpart: every lane `iters` x 4 independent
 * v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, unit E8M0 scales).  Lane g
 * holds 4 pairs (A_j, B_j) of 32 bytes: dword w of A_j is
 * hash(128 g + 16 j + w) and of B_j hash(128 g + 16 j + 8 + w), each byte
 * with bit 6 cleared (no NaN codes); in every group of 4 iterations, step s
 * accumulates A_j times B_((j + s) mod 4) into chain j.  `out` receives each
 * lane's sum of its 4 chains' 16 accumulator elements.  *flop (nullable) =
 * grid * iters * 524,288.  iters a multiple of 4 in [4, 2^30], grid in
 * [1, 2^20]; else HTTM_ERR_INVALID_ARG, with nothing enqueued. */
httm_status httm_peak_mfma_fp8(int32_t iters, int32_t grid, float* out, void* stream, double* flop);

const char* httm_status_string(httm_status s);
/* Last error detail recorded on this thread (empty if none). */
const char* httm_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HTTM_H_ */
