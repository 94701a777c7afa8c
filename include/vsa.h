/*
 * vsa.h -- C ABI of the MI355X (gfx950) two-branch video sparse attention
 * forward over a packed "conditioning prefix + video" token sequence.
 *
 * What the calls compute (pages cited by title and section):
 *  - "Ref2VA VSA : noeud d'attention sparse pour le Ref2VA H3", section
 *    "Le correctif d'attention a deux niveaux", items 1-3: a geometry mapper
 *    puts text, reference-image and reference-audio tokens in tiles of their
 *    own that top-k never prunes; top-k prunes only video key tiles; a gate
 *    (to_gate_compress) scales the compressed branch.
 *  - "ComfyUI-Ref2VA-VSA: Ultra-Fast Character Video Generation", sections
 *    "Technical Architecture" and "The Solution": 4x4x4 spatio-temporal video
 *    tiles; segment-pure prefix tiles that stay dense.
 *  - "BSAI FastH3 Native VSA (recipe)", sections "The mechanism, briefly" and
 *    "The inputs that matter": 64-token video blocks are scored and only the
 *    top share runs exact attention; BF16 with head_dim 128; the patch needs
 *    the packed segment layout; sink_conditioning exact_kv /
 *    exact_kv_and_rows; ambiguous cases must not silently run dense.
 *  - "ComfyUI Agrega Nodo Central de Atencion Dispersa y Compilador Comfy",
 *    section "Atencion dispersa por bloques: un nodo, tres backends": each
 *    query block goes to a chosen subset of key blocks; top-k at a fixed keep
 *    share; Sol-Attn per-head threshold in sigmas of the score distribution;
 *    VSA = cubic tiling plus a coarse compression branch.
 *  - "Spark-H3: atencion dispersa por bloques acelera MiniMax-H3 en ComfyUI",
 *    section "Que cambia Spark-Attn": an exact branch over the top-ranked
 *    blocks and a compressed branch over mean-pooled summaries; a log-mass
 *    bias anchored at the mean video query restores the mass that mean
 *    pooling loses.
 *
 * Conventions for every call:
 *  - Every function returns an int status: VSA_OK (0) or a negative
 *    vsa_status.  Nothing aborts, throws or prints (unless the environment
 *    variable VSA_LOG=1, which writes one line per forward to stderr).
 *  - Device pointers are HIP device addresses on the current device.  The
 *    caller owns every device buffer (inputs, output, workspace) and the
 *    stream.  The library owns only the host-side plan.
 *  - Streams are passed as void* holding a hipStream_t (NULL = null stream).
 *
 * Tensor layout (q, k, v, g, o): bf16, [batch, N, heads, 128] contiguous in
 * packed token order, heads interleaved; 16-byte aligned.
 *
 * Tile numbering used by every output of the library: the P prefix tiles
 * first (segments in packed order, 64 consecutive tokens per tile, the last
 * tile of a segment possibly partial), then the Vt video tiles in raster
 * order (tt, th, tw) over the (T/4, H/4, W/4) tile grid.  Inside a video tile
 * the 64 tokens are raster (dt, dh, dw).  Video tokens are packed raster
 * (t, h, w), w fastest.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSA_OK = 0,
  VSA_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad spans, negative sizes, aliasing */
  VSA_ERR_UNSUPPORTED = -2,      /* outside what the kernels implement: head_dim != 128,
                                    grid dims not multiples of 4, not exactly one video span,
                                    keep outside (0, 100], > 4096 video tiles or candidate
                                    key tiles, > 65535 tiles in all, > 16 prefix
                                    segments, a sparse row list longer than 2048 tiles
                                    (P + k, or P + Vt in TAU mode; k, or Tq, with sink
                                    off), N * heads * head_dim
                                    >= 2^30 (one batch item's Q, K or V is addressed
                                    with 32-bit byte offsets), unknown mode, device
                                    not gfx950.  The caller
                                    decides explicitly what to run instead. */
  VSA_ERR_WORKSPACE = -3,        /* workspace pointer null or smaller than required */
  VSA_ERR_HIP = -4,              /* a HIP runtime call or kernel launch failed */
  VSA_ERR_NO_MEMORY = -5         /* host allocation of the plan failed */
} vsa_status;

typedef enum {
  VSA_SEG_TEXT = 0,
  VSA_SEG_REF_IMAGE = 1,
  VSA_SEG_REF_AUDIO = 2,
  VSA_SEG_OTHER_PREFIX = 3,
  VSA_SEG_VIDEO = 4
} vsa_seg_kind;

/* One span of the packed token axis, [start, start + length). */
typedef struct {
  int64_t start;
  int64_t length;
  int32_t kind;    /* vsa_seg_kind */
  int32_t reserved;
} vsa_segment;

/* sink_conditioning ("BSAI FastH3 Native VSA (recipe)", "The inputs that
 * matter"): EXACT_KV keeps every prefix key tile in every query tile's list;
 * EXACT_KV_AND_ROWS also runs prefix query tiles dense (all key tiles, no
 * coarse term).  OFF protects nothing: the prefix tiles become candidate key
 * tiles like the video tiles (coarse branch, bias and selection run over all
 * Tq tiles, a partial prefix tile summarised over its valid tokens) and every
 * query tile is a sparse row. */
typedef enum {
  VSA_SINK_OFF = 0,
  VSA_SINK_EXACT_KV = 1,
  VSA_SINK_EXACT_KV_AND_ROWS = 2
} vsa_sink;

/* Candidate key tile selection (the Kc candidates are the video tiles, or
 * every tile with VSA_SINK_OFF): TOPK keeps the k = ceil(keep * Kc / 100)
 * largest coarse logits of each sparse query tile (ties to the lowest tile
 * index); TAU keeps every candidate whose logit exceeds mean + tau * std of
 * all the (sparse query tile, candidate) logits of its (batch, head)
 * (Sol-Attn, "un nodo, tres backends").
 * DENSE is the explicit dense call the schedule makes outside its window
 * ("ComfyUI Agrega Nodo Central de Atencion Dispersa y Compilador Comfy", schedule
 * paragraph: outside the start/end window the ordinary dense attention runs): every
 * query tile attends to every key tile exactly, no pooling, coarse branch or
 * selection runs, g is ignored (no coarse term), and keep_percent, sink, coarse
 * and tau are ignored; extra_tokens must be 0 (else VSA_ERR_UNSUPPORTED). */
typedef enum { VSA_SELECT_TOPK = 0, VSA_SELECT_TAU = 1, VSA_SELECT_DENSE = 2 } vsa_select;

/* Coarse logits: MEAN is s * qbar . kbar; MEAN_LOGMASS adds the per candidate
 * tile bias b_j = log(mean_{t in j} exp(s q_a . (k_t - kbar_j))) with q_a the
 * mean video query of the (batch, head) ("Que cambia Spark-Attn",
 * Spark-Reweight).  WEIGHTED_LOGMASS (same item: weighted summaries in place of
 * the means) replaces kbar_j and vbar_j by the anchor's attention over the
 * tile, ktil_j = sum_t w_t k_t and vtil_j = sum_t w_t v_t with
 * w_t = softmax_{t in j}(s q_a . k_t), and takes
 * b_j = log(mean_t exp(s q_a . k_t)) - s q_a . ktil_j.  s = 1/sqrt(128). */
typedef enum {
  VSA_COARSE_MEAN = 0,
  VSA_COARSE_MEAN_LOGMASS = 1,
  VSA_COARSE_WEIGHTED_LOGMASS = 2
} vsa_coarse;

typedef struct {
  int32_t sink;    /* vsa_sink */
  int32_t select;  /* vsa_select */
  int32_t coarse;  /* vsa_coarse */
  float tau;       /* TAU mode threshold in standard deviations */
  /* extra_tokens ("ComfyUI Agrega Nodo Central de Atencion Dispersa y Compilador
   * Comfy", schedule paragraph: the best-scoring tokens beyond the selected blocks
   * are added): 0 (off) .. 64.  Each sparse query tile i also attends to the
   * extra_tokens valid key tokens outside its listed tiles with the largest
   * s * qbar_i . k_t (ties to the lower packed token index; all of them if fewer
   * remain).  Dense rows take none.  > 64 is VSA_ERR_UNSUPPORTED, < 0
   * VSA_ERR_INVALID_ARGUMENT. */
  int32_t extra_tokens;
  /* reblock ("Spark-H3: atencion dispersa por bloques acelera MiniMax-H3 en ComfyUI",
   * "Que cambia Spark-Attn", Spark-Reblock item; reblock_layout=q_reuse_k in its
   * "Flujos de trabajo"): 0 = the fixed 4x4x4 video tiles; 1 = an adaptive
   * partition of each (batch, head)'s video tokens into 64-token tiles, computed
   * on the GPU every forward.  M = mean over the video keys of k k^T; queries are
   * compared by the cosine in the metric M (the cosine of their score patterns over
   * the keys).  A group of m tiles splits along its principal axis (three power
   * steps on the centred covariance of q / sqrt(q^T M q), from z = 1): the
   * 64 floor(m/2) tokens lowest by (projection, token id) form its first floor(m/2)
   * tiles.  Video tile j is then the tree's j-th leaf, tokens ascending; key tiles
   * reuse the query partition; prefix tiles are unchanged.  Not with extra_tokens
   * or the DENSE mode (VSA_ERR_UNSUPPORTED). */
  int32_t reblock;
} vsa_options;

typedef struct vsa_plan vsa_plan; /* opaque, host-only, immutable after creation */

/* Shape facts of a plan. */
typedef struct {
  int32_t batch, heads, head_dim;
  int64_t n_tokens;        /* N */
  int32_t n_prefix_tiles;  /* P */
  int32_t n_video_tiles;   /* Vt */
  int32_t n_tiles;         /* Tq = P + Vt */
  int32_t k;               /* candidate tiles kept per sparse row (TOPK); 0 in TAU mode */
  int32_t n_dense_rows;    /* query tiles per (batch, head) that run dense */
  int32_t n_sparse_rows;   /* query tiles per (batch, head) that select (Qs) */
  int32_t list_capacity;   /* entries reserved per sparse row in the list buffer */
  vsa_options options;
  float keep_percent;
  int32_t first_candidate; /* candidate key tiles are [first_candidate, first_candidate + */
  int32_t n_candidates;    /* n_candidates): P and Vt, or 0 and Tq with VSA_SINK_OFF */
} vsa_plan_desc;

/* Counters of one forward ("BSAI FastH3 Native VSA (recipe)", "Where it goes
 * wrong": read the stats and check sparse work is above zero). */
typedef struct {
  int64_t executed_pairs;   /* (query tile, key tile) pairs run by the fine branch, all (batch, head) */
  int64_t dense_pairs;      /* pairs a dense run would execute: batch * heads * Tq * Tq */
  int64_t sparse_rows;      /* sparse query tiles, all (batch, head) */
  int64_t dense_rows;       /* dense query tiles, all (batch, head) */
  int64_t kept_video_tiles; /* candidate tiles kept over all sparse rows (video tiles
                               unless VSA_SINK_OFF) */
  int32_t k;                /* as in vsa_plan_desc */
  int32_t reserved;
  int64_t extra_tokens;     /* extra tokens attended over all sparse rows (executed_pairs
                               counts each row's extra-token tile as one pair) */
} vsa_stats;

/* Byte offsets into the workspace of the intermediates of the last forward
 * that used it (all row-major, fp32 unless noted):
 *   qbar  [batch, heads, Tq, 128]   mean of the valid Q tokens of each tile
 *   kbar  [batch, heads, Kc, 128]   K summary of each candidate tile (Kc = n_candidates)
 *   vbar  [batch, heads, Kc, 128]   V summary of each candidate tile
 *   bias  [batch, heads, Kc]        log-mass bias (zeros in MEAN mode)
 *   anchor[batch, heads, 128]       mean video query (LOGMASS modes only)
 *   scores[batch, heads, Qs, Kc]    coarse logits of the sparse rows
 *   ocoarse[batch, heads, Qs, 128]  coarse output of the sparse rows
 *   thr   [batch, heads]            TAU threshold (TAU mode only)
 *   lists [batch, heads, Qs, list_capacity] int32 tile ids, ascending (the protected
 *                                   prefix tiles, then the kept candidates)
 *   counts[batch, heads, Qs]        int32 valid entries of each list
 *   xtok  [batch, heads, Qs, 64]    int32 extra token ids, ascending (extra_tokens > 0)
 *   xcnt  [batch, heads, Qs]        int32 extra tokens of each sparse row
 *   tiles [batch, heads, Vt, 64]    int32 packed token ids of each video tile (reblock = 1)
 * Sparse row s of a (batch, head) is query tile s + n_dense_rows. */
typedef struct {
  size_t qbar, kbar, vbar, bias, anchor, scores, ocoarse, thr, lists, counts;
  size_t xtok, xcnt, tiles;
  size_t total_bytes;
} vsa_debug;

/* Build the plan for one packed layout ("BSAI FastH3 Native VSA (recipe)",
 * "The mechanism, briefly": the patch reads where the video span starts and
 * ends).  segs: n_segs spans that must partition [0, N) (any order; sorted by
 * start inside), exactly one of kind VSA_SEG_VIDEO with length
 * video_T * video_H * video_W, each dim a multiple of 4, at most 16 prefix
 * spans.  keep_percent in (0, 100] is used in TOPK mode.  opts may be NULL
 * ({EXACT_KV, TOPK, MEAN, tau 0, extra_tokens 0, reblock 0}).  On success *out owns a new plan (free with
 * vsa_plan_destroy); on error *out is NULL.  Host only, no device work. */
int vsa_plan_geometry(const vsa_segment* segs, int n_segs, int batch, int video_T, int video_H,
                      int video_W, int heads, int head_dim, float keep_percent,
                      const vsa_options* opts, vsa_plan** out);

/* Bytes of device workspace vsa_forward needs for this plan. */
int vsa_plan_workspace_bytes(const vsa_plan* plan, size_t* bytes);

/* Shape facts of the plan. */
int vsa_plan_describe(const vsa_plan* plan, vsa_plan_desc* out);

/* Enqueue the whole forward on `stream`: geometry gather + mean pooling,
 * [anchor + log-mass bias], coarse logits, coarse softmax + O_coarse,
 * [tau statistics], selection, [extra-token scoring and staging],
 * block-sparse fine attention with the gated
 * combine O = O_fine + G * O_coarse written in packed order.
 * Defined by "BSAI FastH3 Native VSA (recipe)", "The mechanism, briefly"
 * (64-token blocks scored, only the top share attended exactly), and by
 * "Spark-H3: atencion dispersa por bloques acelera MiniMax-H3 en ComfyUI",
 * "Que cambia Spark-Attn" (an exact branch over the top-ranked key/value
 * blocks plus a compressed branch over the pooled summaries); the gate is
 * "Ref2VA VSA : noeud d'attention sparse pour le Ref2VA H3", item 3.
 * q, k, v, o: [batch, N, heads, 128] bf16 device buffers; g: same shape or
 * NULL (no coarse term in O).  o must not overlap q, k, v, g or the
 * workspace.  workspace: >= vsa_plan_workspace_bytes, 256-byte aligned,
 * device memory the call may overwrite.  Arguments are checked before
 * anything is enqueued; the call returns without waiting for the GPU.
 * Deterministic: the same inputs give bitwise the same o. */
int vsa_forward(const vsa_plan* plan, const void* q, const void* k, const void* v, const void* g,
                void* o, void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): vsa_forward with the
 * workspace taken from a library-owned device array of VSA_NOALLOC_SCRATCH_BYTES
 * (160 MiB) on each GPU, instead of a caller buffer.  The array is a static
 * device variable of the library: each GPU the call runs on holds its own copy
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine); the first call on a device only looks up the
 * array's address there.  Plans whose workspace exceeds the array are rejected
 * with VSA_ERR_WORKSPACE before anything is enqueued (vsa_last_error names both
 * sizes).  Every call on one GPU shares that GPU's array and leaves the last
 * call's intermediates in it: calls that overlap on one GPU (other streams, other
 * threads) race, so order them on one stream.  No kernel needs the array cleared
 * (every intermediate is written before it is read).  Other arguments, checks and
 * results as vsa_forward; vsa_read_stats does not apply (it reads a caller
 * workspace). */
#define VSA_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
int vsa_forward_noalloc(const vsa_plan* plan, const void* q, const void* k, const void* v,
                        const void* g, void* o, void* stream);

/* Counters of the last forward that used `workspace` (reads the list counts
 * back; synchronises `stream`). */
int vsa_read_stats(const vsa_plan* plan, const void* workspace, void* stream, vsa_stats* out);

/* Offsets of the intermediates inside the workspace (host only). */
int vsa_debug_views(const vsa_plan* plan, vsa_debug* out);

int vsa_plan_destroy(vsa_plan* plan);

/* Static string for a status code (never NULL). */
const char* vsa_status_string(int status);

/* Detail of the last VSA_ERR_HIP returned on the calling thread (the step and
 * the HIP error name and text), or of the last VSA_ERR_WORKSPACE returned by
 * vsa_forward_noalloc (the sizes); "" if none.  Valid until the next call on the
 * same thread. */
const char* vsa_last_error(void);

/* ---- kernel timing for measurement -------------------------------------
 * A timer records a HIP event pair around every kernel that
 * vsa_forward_timed enqueues, on the same stream, and sums the elapsed times
 * per kernel.  Not thread-safe; one timer per stream. */
typedef struct vsa_timer vsa_timer;

typedef struct {
  char name[32];       /* kernel name */
  int32_t launches;    /* launches recorded since the last reset */
  double total_ms;     /* summed event-to-event time */
} vsa_kernel_time;

int vsa_timer_create(vsa_timer** out);
int vsa_timer_destroy(vsa_timer* timer);
int vsa_timer_reset(vsa_timer* timer);
/* Same as vsa_forward, plus event records around each kernel. */
int vsa_forward_timed(const vsa_plan* plan, const void* q, const void* k, const void* v,
                      const void* g, void* o, void* workspace, size_t workspace_bytes,
                      void* stream, vsa_timer* timer);
/* Waits for the recorded events, then fills up to `max` entries (one per
 * kernel name) and sets *n to their number. */
int vsa_timer_read(vsa_timer* timer, vsa_kernel_time* out, int max, int* n);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
