/*
 * sfa.h -- C ABI of the frame-aligned window-sparse attention library (gfx950).
 *
 * The operation ("HeyGen x Google Cloud: Bringing Avatar IV to TPUs"):
 *   - tokens are frame-major: frame 0 is the global reference frame, frames
 *     1..F are video frames, each of T tokens; S = (F + 1) * T;
 *   - a query of video frame v sees the keys of the reference frame and of
 *     the video frames max(1, v - w) .. min(F, v + w); a reference-frame query
 *     sees the reference frame only (section "Deleting the mask", Fig. 3);
 *   - O_i = sum_j softmax_j(scale * <q_i, k_j>) v_j over the visible keys;
 *   - heads whose Cauchy-Schwarz bound  scale * max_i ||q_i|| * max_j ||k_j - mu||
 *     (mu = per-head key mean) is <= bound_limit use that bound as a fixed
 *     softmax maximum; the others use the online (running-maximum) softmax in
 *     the same kernel (section "Unchaining softmax", Fig. 4);
 *   - QK^T and PV run on bf16 MFMA with fp32 accumulation; P is rounded to
 *     bf16 before PV (section "Proving pixels unchanged").
 *
 * Conventions for every entry point:
 *   - returns an int status (SFA_OK = 0 or a negative SFA_ERR_*), never throws,
 *     never aborts; on error nothing has been enqueued;
 *   - device pointers (tensor data, workspace) are owned by the caller; the
 *     library never allocates or frees device memory;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream); work
 *     is enqueued asynchronously on it; only the sfa_read_* calls synchronise;
 *   - a plan owns host memory only, is immutable after creation and may be
 *     shared by threads.
 */
#ifndef SFA_H
#define SFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFA_OK 0
#define SFA_ERR_INVALID (-1)     /* null pointer, bad size, too-small workspace */
#define SFA_ERR_UNSUPPORTED (-2) /* T % 16 != 0, head_dim not 64/128, misaligned data */
#define SFA_ERR_HIP (-3)         /* HIP launch/runtime error (see sfa_status_str) */
#define SFA_ERR_NOMEM (-4)       /* host allocation failed */
#define SFA_ERR_TOO_LARGE (-5)   /* sfa_attention_static: workspace beyond its 64 MiB */

/* Attention geometry. One plan per geometry (section "Workload and porting":
 * every attention is dispatched to a kernel shaped for it). */
typedef struct sfa_geometry {
  int32_t batch;            /* B >= 1 */
  int32_t heads;            /* H >= 1 */
  int32_t head_dim;         /* d: 64 or 128 */
  int32_t frames;           /* F >= 0 video frames; the reference frame is extra */
  int32_t tokens_per_frame; /* T >= 16, T % 16 == 0 */
  int32_t window;           /* w >= 0 */
  float scale;              /* softmax scale; 0 selects 1/sqrt(d) */
  float bound_limit;        /* fixed-max eligibility threshold (40 in the workloads), at most
                               126 / (2 log2 e) = 43.668 (SFA_ERR_UNSUPPORTED above: a fixed
                               maximum up to 2 * bound_limit above a row's largest logit
                               must leave its largest weight a normal float); a negative
                               value makes every head use the online path */
} sfa_geometry;

/* A bf16 tensor [B, S, H, d] addressed as
 * data + b*stride_b + s*stride_s + h*stride_h + e  (strides in elements, d contiguous).
 * data must be 16-byte aligned, every stride a multiple of 8 and stride_s at
 * most 2^24 (SFA_ERR_UNSUPPORTED otherwise). */
typedef struct sfa_tensor {
  void* data;
  int64_t stride_b;
  int64_t stride_s;
  int64_t stride_h;
} sfa_tensor;

typedef struct sfa_plan sfa_plan;

typedef struct sfa_plan_info {
  int32_t block_q;          /* query rows per work item, a multiple of 16; the last item
                               of each frame holds the T mod block_q rows left, if any */
  int32_t granule;          /* token granule of the key loop (16) */
  int32_t waves_per_item;   /* 64-lane waves in one workgroup */
  int32_t items;            /* work items = B * H * (F + 1 + split_frames) *
                               ceil(T / block_q) */
  int64_t active_pairs;     /* visible (query, key) pairs summed over B and H */
  double active_flops;      /* 4 * d * active_pairs (q.k and p.v, 2 flops per MAC) */
  int64_t io_bytes;         /* q, k, v read once and o written once: 8 * B * S * H * d */
  size_t workspace_bytes;   /* device workspace needed by sfa_norms / sfa_fwd */
  int32_t bound_mode;       /* the plan's bound_mode (see sfa_plan_options) */
  int32_t split_frames;     /* query frames whose work items run as two key halves (see
                               sfa_plan_options.key_split) */
  int32_t wave_rows;        /* query rows per wave (32 or 64) */
} sfa_plan_info;

/* Validates the geometry and builds the work decomposition (host only, no HIP
 * call, no device memory). *out is set to NULL on error. */
int sfa_plan_create(const sfa_geometry* geom, sfa_plan** out);

/* Tuning overrides for sfa_plan_create_ex; 0 in a field selects the default. */
typedef struct sfa_plan_options {
  int32_t block_q;        /* query rows per work item: a multiple of 16, at most
                             waves_per_item * wave_rows, cut to T (default: that maximum;
                             when it gives fewer work items than 256 compute units, each
                             frame is cut into the most blocks of balanced size that keep
                             the items at 256 or fewer, not below wave_rows); when it does
                             not divide T, the last item of each frame takes the rows left */
  int32_t waves_per_item; /* 8 (default: two waves per SIMD), 12 (three per SIMD, 32 query
                             rows each, 96-key LDS stages) or 4 (one wave per SIMD, 512
                             registers, 64 query rows per wave) */
  int32_t lds_stages;     /* K/V stages in LDS: 2, 3 or 4 (2 or 3 with 12 waves; default 3).
                             With 8 waves of 32 rows, 3 and 4 select the software-pipelined
                             loop, with 1 or 2 stages in flight while one is read */
  int32_t bound_mode;     /* how the fixed maximum is bounded (section "Unchaining
                             softmax": query norm times the largest mean-centred key norm):
                             0 (default) per (b, h): the largest key norm of the head, one
                             eligibility flag per head;
                             1 per (b, h, query frame): the largest key norm over the frames
                             that query frame sees (reference frame + window, section
                             "Deleting the mask"), one flag per query frame. Never looser
                             than 0; the output is the same softmax either way. */
  int32_t key_split;      /* 0 (default): with 8 waves per item, the items of the query
                             frames that see the fewest frames (more than one) run as two
                             key halves, whose partial outputs and row sums the later
                             finisher merges (section "Unchaining softmax": with a shared
                             fixed maximum the halves simply add); they are the last long
                             items of the largest-first order, so the launch's tail gets
                             shorter. -1: never split. */
  int32_t wave_rows;      /* query rows per wave with 8 waves: 32 (default: one 32-row
                             query tile, 256-row work items, software-pipelined loop) or 64
                             (two tiles, so every K or V^T operand read from LDS feeds two
                             MFMAs; 512-row items; measured slower on MI355X: the 256
                             registers of a wave leave no room to overlap its softmax with
                             its MFMAs). 4 waves: 64 only; 12 waves: 32 only. */
} sfa_plan_options;

/* sfa_plan_create with overrides (options may be NULL). Values outside the
 * ranges above give SFA_ERR_UNSUPPORTED. */
int sfa_plan_create_ex(const sfa_geometry* geom, const sfa_plan_options* options,
                       sfa_plan** out);

void sfa_plan_destroy(sfa_plan* plan);

int sfa_plan_get_info(const sfa_plan* plan, sfa_plan_info* out);

/* Key token ranges seen by queries of `query_frame` (0 = reference frame), as
 * half-open [start, end) pairs in ranges[0..2*n). Adjacent ranges are merged,
 * so n is 1 or 2. Section "Deleting the mask": every range is a whole number of
 * frames, hence a whole number of 16-token granules. */
int sfa_plan_key_ranges(const sfa_plan* plan, int32_t query_frame, int32_t ranges[4],
                        int32_t* n);

/* Work item scheduled at position `index` of the launch (0 <= index < items):
 * writes {batch, head, query_frame, query_block}. Items are ordered by
 * decreasing key count (largest first) and grouped so that the items sharing
 * one (batch, head, frame) key stream land on one XCD. */
int sfa_plan_item(const sfa_plan* plan, int32_t index, int32_t item[4]);

/* Keys of the work item at `index`: *half is -1 for an item that covers every visible
 * key of its query frame, 0 or 1 for the first or second key half of a split one (the
 * visible frames, reference frame first, cut after the first ceil(n/2)); its key token
 * ranges as half-open [start, end) pairs in ranges[0..2*n), n = 1 or 2. */
int sfa_plan_item_keys(const sfa_plan* plan, int32_t index, int32_t* half, int32_t ranges[4],
                       int32_t* n);

/* Memory-bound prologue of the attention, written into `workspace` only:
 *  - the norm array of the fixed maximum (section "Unchaining softmax"): per
 *    (b, h) the key mean mu, max_j ||k_j - mu||, max_i ||q_i||, the bound and
 *    the eligibility flag; per (b, h, query frame) the key-norm maximum, bound
 *    and flag the plan's bound_mode selects; per row ||q_i|| and <q_i, mu>
 *    (fp32; q read once, k three times, v once; fixed reduction order, no
 *    atomics, so bit-deterministic);
 *  - k and v staged in bf16 in the layout of the attention kernel's LDS stages
 *    (per (b, h), 16-token granules of 32 * d bytes: k as [granule][8-element
 *    chunk][16 keys][8], v as [granule][d][16 keys] with the two 8-key halves of
 *    each row swapped when (d / 8) is odd), see sfa_read_staged.
 * Must run on the current q, k and v before sfa_fwd. */
int sfa_norms(const sfa_plan* plan, sfa_tensor q, sfa_tensor k, sfa_tensor v, void* workspace,
              size_t workspace_bytes, void* stream);

/* The attention kernel (one launch): one pass over each query block's
 * reference-frame and window key granules, with the fixed maximum for eligible
 * heads and the online softmax for the others. Reads q from its tensor and the
 * staged copies of k and v from the workspace, so sfa_norms must have run on the
 * same q, k, v and workspace earlier on the stream; k and v themselves are only
 * validated. o may not alias q, k or v. The launch is persistent (at most one workgroup per
 * CU) and takes its work items from counters in the workspace, which sfa_norms
 * zeroes and every launch leaves at zero: sfa_fwd may run any number of times
 * after one sfa_norms, but two calls in flight at once on one workspace race.
 * The key halves of split items (sfa_plan_options.key_split) meet through partial
 * results and counters in the same workspace; the output does not depend on which
 * half finishes first. */
int sfa_fwd(const sfa_plan* plan, sfa_tensor q, sfa_tensor k, sfa_tensor v, sfa_tensor o,
            void* workspace, size_t workspace_bytes, void* stream);

/* sfa_norms followed by sfa_fwd. */
int sfa_attention(const sfa_plan* plan, sfa_tensor q, sfa_tensor k, sfa_tensor v,
                  sfa_tensor o, void* workspace, size_t workspace_bytes, void* stream);

/* sfa_attention without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a fixed 64 MiB array in the library, one per GPU, held
 * from the first call on that GPU until the process ends. The call allocates nothing.
 * Plans whose workspace_bytes exceed 64 MiB get SFA_ERR_TOO_LARGE (e.g. 8 heads of d =
 * 128 over S = 8192 tokens fit; the 720p-shaped layer does not). `stream` must run on the
 * current device (SFA_ERR_INVALID otherwise). Every call on a GPU uses that GPU's one
 * array, so calls that overlap on one GPU (other streams, other threads) race; calls
 * ordered on one stream are safe, and nothing left in the array by an earlier call is
 * read. */
int sfa_attention_static(const sfa_plan* plan, sfa_tensor q, sfa_tensor k, sfa_tensor v,
                         sfa_tensor o, void* stream);

/* Head-group split (section "Hiding collectives": heads are independent and the
 * mask does not depend on them, so they can be processed in groups, each group
 * a pipeline step of its own). Runs sfa_attention on `groups` consecutive head
 * groups of q, k, v, o, each of `group_plan`'s geometry (its `heads` is the group
 * size; the tensors hold groups * heads heads, group g being heads
 * [g*heads, (g+1)*heads)). Group g uses workspace bytes [g*W, (g+1)*W) with W =
 * the group plan's workspace_bytes (so workspace_bytes >= groups * W) and is
 * launched on group_streams[g % nstreams] (or on `stream` when nstreams is 0).
 * The group streams first wait for the work already queued on `stream`, and
 * `stream` then waits for every group, so callers order against `stream` only.
 * Results are bitwise identical to one sfa_attention over all heads. The events
 * that order the streams are created and released inside the call. */
int sfa_attention_groups(const sfa_plan* group_plan, int32_t groups, sfa_tensor q, sfa_tensor k,
                         sfa_tensor v, sfa_tensor o, void* workspace, size_t workspace_bytes,
                         void* stream, void* const* group_streams, int32_t nstreams);

/* The sfa_read_* calls copy parts of a workspace that sfa_norms has filled to host
 * memory and synchronise the stream. workspace_bytes is the size of the workspace
 * (SFA_ERR_INVALID below the plan's workspace_bytes: nothing is copied). */

/* Per-head statistics. Each output pointer is host memory of B*H entries (mu: B*H*d)
 * or NULL to skip it. bound = scale * max_i ||q_i|| * max_j ||k_j - mu|| (per head in
 * both bound modes); eligible = 1 when every query frame of the head takes the
 * fixed-maximum path. */
int sfa_read_head_stats(const sfa_plan* plan, const void* workspace, size_t workspace_bytes,
                        float* mu, float* kmax, float* qmax, float* bound, uint8_t* eligible,
                        void* stream);

/* The per-row half of the norm array: qnorm[b][h][s] = ||q_s|| and
 * qmu[b][h][s] = <q_s, mu_bh>, B*H*S floats each, host memory, either may be NULL. The
 * attention kernel derives the fixed row maximum from them as
 * M = scale * (qmu + qnorm * kvis[b][h][frame(s)]). */
int sfa_read_row_norms(const sfa_plan* plan, const void* workspace, size_t workspace_bytes,
                       float* qnorm, float* qmu, void* stream);

/* The per-(b, h, query frame) half of the norm array; each output is host memory of
 * B*H*(F+1) entries, index [b][h][g], or NULL to skip it:
 *   kvis[g]     key-norm maximum the rows of query frame g use: bound_mode 0 the
 *               head's max_j ||k_j - mu||; bound_mode 1 the maximum over the frames
 *               g sees of max ||k_j - mu|| within the frame;
 *   bound[g]    scale * (max ||q_i|| over the head, mode 0, or over frame g, mode 1) * kvis[g];
 *   eligible[g] bound[g] <= bound_limit (0 for every frame when bound_limit < 0): the
 *               work items of frame g take the fixed-maximum path. */
int sfa_read_frame_stats(const sfa_plan* plan, const void* workspace, size_t workspace_bytes,
                         float* kvis, float* bound, uint8_t* eligible, void* stream);

/* The staged copies of k and v the attention kernel reads (layouts at sfa_norms),
 * B*H*S*d bf16 each, host memory, either may be NULL. */
int sfa_read_staged(const sfa_plan* plan, const void* workspace, size_t workspace_bytes,
                    uint16_t* k_staged, uint16_t* v_staged, void* stream);

/* ---- Fused attention prologue (section "Layout as ABI", Fig. 5) ----
 * The chain that produces the attention's inputs -- normalisation, projection,
 * rotary embedding, head packing -- as one MFMA kernel that writes q, k, v
 * straight into the sfa_tensor layout sfa_norms / sfa_fwd read:
 *   xn = x / sqrt(mean_c x^2 + eps) * gamma          (RMSNorm over C)
 *   [q | k | v] = xn . W^T,  W stored [3*H*d][C]     (row n: tensor n / (H*d),
 *                                                     head (n / d) % H, element n % d)
 *   q, k: pairs (e, e + d/2), e < d/2, rotated by cos[s][e], sin[s][e].
 * gamma is folded into W once (sfa_prologue_fold); the kernel sums each token's
 * squares from the x operands it stages anyway and scales the token's outputs by
 * the inverse RMS. bf16 in and out, fp32 accumulation, no workspace. */
typedef struct sfa_prologue_geometry {
  int32_t batch;
  int32_t seq;        /* S tokens per batch entry */
  int32_t model_dim;  /* C: a multiple of 64 */
  int32_t heads;      /* H; heads * head_dim must be a multiple of 256 */
  int32_t head_dim;   /* 64 or 128 */
  float eps;          /* RMSNorm epsilon, >= 0 */
} sfa_prologue_geometry;

/* W' = bf16(gamma[c] * W[n][c]) for bf16 W [rows][cols] and gamma [cols] (device
 * pointers, 16-byte aligned, cols even). Run once per weight. */
int sfa_prologue_fold(const void* w, const void* gamma, void* w_folded, int32_t rows,
                      int32_t cols, void* stream);
/* x: bf16 [B][S][C] (stride_b, stride_s in elements, C contiguous, stride_s <= 2^22;
 * stride_h ignored). w_folded: bf16 [3*H*d][C] from sfa_prologue_fold. cos, sin:
 * fp32 [S][d/2]. q, k, v: bf16 [B][S][H][d] in any sfa_tensor strides (they must
 * not overlap x, and share no element with each other; interleaved views of one
 * [B][S][3][H][d] buffer are fine). Fewer than 2^31 tiles of 256 x 256. One launch on `stream`. Returns SFA_ERR_INVALID for null or
 * overlapping arguments, SFA_ERR_UNSUPPORTED for shapes, strides or alignments
 * outside the rules above (data pointers 16-byte aligned, strides multiples of 8). */
int sfa_qkv_prologue(const sfa_prologue_geometry* geom, sfa_tensor x, const void* w_folded,
                     const float* cos_table, const float* sin_table, sfa_tensor q, sfa_tensor k,
                     sfa_tensor v, void* stream);

/* ---- Ablation: generic block-sparse attention (measured, not the product path) ----
 * The design the pages started from (section "Deleting the mask": splash-style
 * block-sparse attention with generic tile sizes that ignore frame
 * boundaries): query blocks of 256 rows and key blocks of 128 keys over the
 * padded sequence, each (query block, key block) classified as empty, full or
 * partial from the frame mask, partial blocks masked element by element, the
 * window keys and the reference-frame keys processed as two separate
 * online-softmax passes whose normalised outputs are merged through their
 * log-sum-exp. Computes the same attention as sfa_attention (online softmax
 * everywhere, no norm array); it exists to measure what the frame-aligned
 * single-pass design saves on this hardware. */
typedef struct sfa_generic sfa_generic;

typedef struct sfa_generic_info {
  int32_t block_q;          /* 256 */
  int32_t block_k;          /* 128 */
  int32_t query_blocks;     /* per (b, h): ceil(S / block_q) */
  int32_t key_blocks;       /* per (b, h): ceil(S / block_k) */
  int64_t full_blocks;      /* per (b, h), both passes */
  int64_t partial_blocks;   /* per (b, h), both passes */
  int64_t computed_pairs;   /* (query rows incl. padding) x (keys of visited blocks), all (b, h) */
  size_t workspace_bytes;   /* device workspace of sfa_generic_attention */
} sfa_generic_info;

/* Host only; the block lists are built here. *out is NULL on error. */
int sfa_generic_create(const sfa_geometry* geom, sfa_generic** out);
void sfa_generic_destroy(sfa_generic* g);
int sfa_generic_get_info(const sfa_generic* g, sfa_generic_info* out);
/* Block class of (pass, query block, key block): 0 empty, 1 full, 2 partial;
 * pass 0 = window keys, pass 1 = reference-frame keys. */
int sfa_generic_block_class(const sfa_generic* g, int32_t pass, int32_t query_block,
                            int32_t key_block, int32_t* cls);
/* V^T staging, both passes (one launch) and the merge, on `stream`; all
 * scratch (V^T, block lists, per-pass outputs and log-sum-exps) lives in
 * `workspace`. Same tensor rules as sfa_fwd. */
int sfa_generic_attention(const sfa_generic* g, sfa_tensor q, sfa_tensor k, sfa_tensor v,
                          sfa_tensor o, void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable text for a status code (includes the last HIP error of the
 * calling thread for SFA_ERR_HIP). */
const char* sfa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* SFA_H */
