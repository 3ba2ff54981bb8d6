/*
 * rs.h — C ABI of the Representation Shift hot path on MI355X (gfx950).
 *
 * The method: "Representation Shift: Unifying Token Compression with FlashAttention"
 * (arXiv HTML page).  A pre-LN Vision/Video Transformer block (Sec. 3.3, Eqs. (5) and
 * (6)) runs fused attention that never stores the attention map (Sec. 3.1, Eq. (1);
 * Sec. 1 on fused attention), then its MLP sublayer; every token is scored by the
 * MLP-sublayer representation shift || MLP(LN(x')) - x' ||_2 (Sec. 3.2, Eq. (4), with
 * Sec. 3.3 case ii and the L2 distance); the lowest-scoring tokens are dropped, the
 * same number in every sample (Sec. 3.2, toy experiments; Sec. 4.1 and 4.2 settings).
 *
 * Conventions shared by every entry point
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library never
 *    allocates or frees device memory; scratch space is the caller's `workspace`.
 *  - Every tensor is dense row-major.  Activations are [B][L][C] (sample, token,
 *    channel).  A Linear layer's weight is [out][in] and computes z W^T + b.
 *  - Enumerated arguments (rs_dtype, rs_shift_op, rs_dist, rs_pool) are passed as int
 *    and validated; an unknown value is RS_ERR_INVALID_ARG.
 *  - Element type: RS_F32 (float) or RS_BF16 (bfloat16 storage; all accumulation,
 *    softmax, LayerNorm statistics and scores are fp32).  Scores are always fp32,
 *    indices int32.
 *  - Every data pointer must be 16-byte aligned; `workspace` 256-byte aligned.
 *  - All work is enqueued on `stream` (0 = the null stream) and is asynchronous; the
 *    call returns once it is enqueued.  Synchronise the stream before reading outputs.
 *  - Validation is synchronous and happens before anything is enqueued: on an error
 *    nothing is enqueued, no output is touched and the code is returned.  A failed
 *    kernel launch returns RS_ERR_HIP (earlier launches of the call may have run).
 *    Nothing is printed, nothing aborts, no C++ exception crosses the ABI.
 *    rs_last_error() returns a message for the calling thread's last failure.
 *  - Calls are re-entrant; concurrent calls need distinct workspaces and outputs.
 *  - No call works in place: outputs and the workspace must not overlap the inputs or
 *    each other (overlapping buffers give undefined results; this is not checked).
 *  - Limits (else RS_ERR_UNSUPPORTED): head dim 64 (C == heads*64), C % 64 == 0,
 *    C <= RS_MAX_WIDTH, hidden % 64 == 0, 1 <= L <= RS_MAX_TOKENS, and
 *    B*L*max(3C, hidden) < 2^31.
 */
#ifndef RS_H_
#define RS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RS_MAX_TOKENS 16384
#define RS_MAX_WIDTH 1024

typedef enum {
  RS_OK = 0,
  RS_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, bad schedule */
  RS_ERR_UNSUPPORTED = 2,   /* shape outside the limits listed above */
  RS_ERR_WORKSPACE = 3,     /* workspace smaller than rs_workspace_bytes() */
  RS_ERR_HIP = 4            /* a HIP call or kernel launch failed */
} rs_status;

typedef enum { RS_F32 = 0, RS_BF16 = 1 } rs_dtype;

/* Which score ranks the tokens.  A representation shift (Sec. 3.3, "Operation choice"):
 * D(F(z), z) through the MLP sublayer, F(z) = MLP(LN(z)) at z = x' (the method), through
 * the attention sublayer, F = SA(LN(.)) (after the output projection and its bias) at
 * z = x, or through the whole block, D(x_hat, x).  Or, as the comparison baselines of
 * Sec. 3.1, the block's attention map averaged over heads: the class token's attention
 * row (Eq. (2); needs desc->has_cls) or the mean of all queries' attention rows
 * (Eq. (3)).  The map scores run the pruning blocks' attention with the map-forming
 * kernel (two passes over the keys); score_dist does not apply to them. */
typedef enum {
  RS_SHIFT_MLP = 0,
  RS_SHIFT_ATTN = 1,
  RS_SHIFT_BLOCK = 2,
  RS_MAP_CLS = 3,
  RS_MAP_MEAN = 4
} rs_shift_op;
/* Distance D per token (Sec. 3.3, "Distance metrics"): L2 norm of the difference (the
 * method), L1 norm of the difference, or cosine distance 1 - a.b / max(|a| |b|, 1e-8). */
typedef enum { RS_DIST_L2 = 0, RS_DIST_L1 = 1, RS_DIST_COS = 2 } rs_dist;

/* Shape of one encoder: width C, heads (head dim C/heads = 64), MLP hidden width,
 * LayerNorm epsilon (biased variance), element type, whether token 0 is a class token
 * that selection always keeps, the score (operation and distance; 0, 0 = the method's
 * MLP-sublayer L2 shift), and attn_map: 0 = attention never stores its map (fused;
 * blocks scored from the map form it in registers only), 1 = every block's attention
 * forms its map and stores it to HBM ([B][H][L][L rounded up to 8] in the workspace), as
 * a non-fused attention does -- the comparison setting of the pages' Base and Attn rows. */
typedef struct {
  int C;
  int heads;
  int hidden;
  float ln_eps;
  int dtype;              /* an rs_dtype */
  int has_cls;
  int score_op;           /* an rs_shift_op */
  int score_dist;         /* an rs_dist */
  int attn_map;
} rs_model_desc;

/* Weights of one pre-LN block (Sec. 3.3, Eqs. (5) and (6)), all of desc.dtype.
 * w_qkv rows 0..C-1 produce Q, rows C..2C-1 K, rows 2C..3C-1 V; head h uses rows
 * h*64 .. h*64+63 of each (Eq. (1) applied per head with scale 1/sqrt(64)).
 * MLP = fc2(GELU(fc1(.))) with the exact (erf) GELU. */
typedef struct {
  const void *ln1_g, *ln1_b;    /* [C]                  */
  const void *w_qkv, *b_qkv;    /* [3C][C], [3C]        */
  const void *w_proj, *b_proj;  /* [C][C], [C]          */
  const void *ln2_g, *ln2_b;    /* [C]                  */
  const void *w_fc1, *b_fc1;    /* [hidden][C], [hidden] */
  const void *w_fc2, *b_fc2;    /* [C][hidden], [C]     */
} rs_block_weights;

/* One block plus selection (Eqs. (5), (6), the MLP-sublayer shift of Eq. (4) and the
 * per-sample drop of the lowest scores).
 *  x        [B][L][C]   block input.
 *  keep_k   tokens kept per sample, 1 <= keep_k <= L (keep_k == L keeps all; the
 *           class token, when desc->has_cls, counts towards keep_k and is kept).
 *  y        [B][L][C]   block output x_hat (Eq. (6)); nullable (then not written).
 *  scores   [B][L]      fp32 per-token shift (desc->score_op, desc->score_dist; the
 *                       method: || MLP(LN(x')) - x' ||_2); nullable.
 *  kept_idx [B][keep_k] kept token indices of each sample, ascending.  Order used to
 *           choose: score descending, ties to the lower index, NaN lowest.
 *  y_kept   [B][keep_k][C] rows of x_hat at kept_idx (class token first when present).
 *  workspace/ws_bytes   >= rs_workspace_bytes(desc, 1, B, L). */
rs_status rs_block_forward(const rs_model_desc* desc, const rs_block_weights* w,
                           const void* x, int B, int L, int keep_k,
                           void* y, float* scores, int32_t* kept_idx, void* y_kept,
                           void* workspace, size_t ws_bytes, hipStream_t stream);

/* Representation shift with the L2 distance (Eq. (4)) of given tensors:
 * scores[r] = || fx[r,:] - x[r,:] ||_2 for every row r of [B*L][C]. */
rs_status rs_score(const void* fx, const void* x, int B, int L, int C, int dtype,
                   float* scores, hipStream_t stream);
/* Same with the distance of Sec. 3.3 chosen: scores[r] = D(fx[r,:], x[r,:]). */
rs_status rs_score_dist(const void* fx, const void* x, int B, int L, int C, int dtype,
                        int dist, float* scores, hipStream_t stream);

/* Multi-head attention alone (Sec. 3.1, Eq. (1), heads of 64 consecutive columns, scale
 * 1/8): qkv [B][L][3C] (Q | K | V, as the block's QKV projection writes them) ->
 * out [B][L][C].  With map, score_cls and score_mean all null it is the fused kernel
 * that never forms the map.  Otherwise the map-forming kernel runs and writes what is
 * asked: map [B][H][L][Lpad] (Lpad = L rounded up to a multiple of 8; row i holds query
 * i's attention over the keys, padding keys 0), score_cls [B][L] = Eq. (2) averaged over
 * heads (the class token's row; query 0), score_mean [B][L] = Eq. (3) averaged over
 * heads.  desc supplies C, heads and dtype.  workspace/ws_bytes >=
 * rs_attention_workspace_bytes(desc, B, L) (may be 0 / null when no score is asked). */
rs_status rs_attention(const rs_model_desc* desc, const void* qkv, int B, int L, void* out,
                       void* map, float* score_cls, float* score_mean, void* workspace,
                       size_t ws_bytes, hipStream_t stream);
size_t rs_attention_workspace_bytes(const rs_model_desc* desc, int B, int L);

/* rs_attention without a workspace, for callers that cannot allocate device memory
 * (work under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, validation and results as rs_attention; the score sums live in a
 * fixed scratch array of RS_NOALLOC_SCRATCH_BYTES inside the library, one per device
 * (held from the library's first use on that device until the process ends).  No call
 * allocates or frees memory.  A call that asks for a score whose sums exceed the limit
 * (rs_attention_workspace_bytes(desc, B, L) > RS_NOALLOC_SCRATCH_BYTES) returns
 * RS_ERR_UNSUPPORTED and enqueues nothing.  Every call on one device shares that array
 * and fully overwrites the part it uses: calls whose work may overlap in time on the same
 * device (concurrent streams, or host threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe. */
#define RS_NOALLOC_SCRATCH_BYTES (16u << 20)
rs_status rs_attention_noalloc(const rs_model_desc* desc, const void* qkv, int B, int L,
                               void* out, void* map, float* score_cls, float* score_mean,
                               hipStream_t stream);

/* Per-sample selection and compaction: keep the keep_k highest scores of each sample
 * (ties to the lower index, NaN lowest, token 0 always kept if has_cls), write their
 * indices ascending to kept_idx [B][keep_k] and, if x_kept is not null, the rows
 * x[b, kept_idx[b, j], :] to x_kept [B][keep_k][C].  x may be null when x_kept is. */
rs_status rs_topk_gather(const float* scores, const void* x, int B, int L, int C,
                         int dtype, int keep_k, int has_cls,
                         int32_t* kept_idx, void* x_kept, hipStream_t stream);

/* Whole encoder with progressive pruning (Sec. 4.1 and 4.2 settings): blocks 0..depth-1
 * in order; after each block listed in prune_layers (0-based, strictly ascending) the
 * block's output is compacted to the floor(r*L + 1/2) highest-scoring tokens of the
 * current L (r = the matching keep_ratios entry, 0 < r <= 1, evaluated in IEEE
 * double), the score being that block's representation shift (desc->score_op,
 * desc->score_dist).
 *  blocks   [depth] weight sets.
 *  out      [B][L_final][C] encoder output (L_final from rs_encoder_out_len).
 *  out_idx  [B][L_final] original token index of every output row.
 *  workspace/ws_bytes   >= rs_workspace_bytes(desc, depth, B, L).
 * Concurrency: the batch runs as n lanes, n the largest count up to the process-wide
 * maximum (rs_set_max_lanes) for which every lane keeps >= 512 rows after the last
 * pruning (floor(B/n) * L_final >= 512) -- lane i takes a contiguous share of the
 * samples, floor(B/n) or one more (the first B mod n lanes); lane 0 runs on `stream`, the
 * others on streams the library owns (default priority), forked from and joined back
 * into `stream` with events -- so one lane's memory-bound phases overlap another's
 * matrix work.  Per-sample results do not depend on the lane split except through a
 * GEMM's split over K, which depends on its row count.  All work is ordered after prior
 * work on `stream` and before later work; the call can be captured into a HIP graph. */
rs_status rs_encoder_forward(const rs_model_desc* desc, const rs_block_weights* blocks,
                             int depth, const void* x, int B, int L,
                             const int* prune_layers, const double* keep_ratios, int n_prune,
                             void* out, int32_t* out_idx,
                             void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---- the steps either side of the encoder --------------------------------------------
 * Tokenisation (Sec. 3.1): an H x W image is cut into N = (H/P)(W/P) patches of P x P
 * pixels; a clip of `frames` images is tokenised frame by frame.  The patch embedding is
 * the P x P, stride-P convolution with bias, computed as one GEMM whose A operand is
 * gathered from the images inside the kernel; tokens are the patches in raster order of
 * the grid, frame after frame, preceded by the class token when desc->has_cls, plus a
 * position table.  The encoder output ends in a final LayerNorm, a pooling (the class
 * token's row, or the mean over tokens) and a Linear head.  The pages run these steps
 * unchanged from the DeiT / UMT models; they bracket the pruned encoder in a whole
 * forward pass. */

/* Pixel input geometry.  frames >= 1 (1 for an image), in_chans >= 1, patch P in
 * {8, 16, 32}, height and width positive multiples of P.  Tokens per sample:
 * L = desc->has_cls + frames * (height/P) * (width/P). */
typedef struct {
  int frames;
  int in_chans;
  int height;
  int width;
  int patch;
} rs_image_desc;

/* Patch embedding weights, all of desc->dtype:
 *  w_patch [C][in_chans*P*P]  the convolution weight, each output channel's kernel
 *                             flattened as (input channel, row, column);
 *  b_patch [C];
 *  cls     [C]   class token (read only when desc->has_cls; may be null otherwise);
 *  pos     [L][C] position table, row 0 the class token's when present. */
typedef struct {
  const void* w_patch;
  const void* b_patch;
  const void* cls;
  const void* pos;
} rs_embed_weights;

typedef enum { RS_POOL_CLS = 0, RS_POOL_MEAN = 1 } rs_pool;

/* Final LayerNorm (ln_g, ln_b [C], eps = desc->ln_eps) and head (w_head [n_out][C],
 * b_head [n_out]), all of desc->dtype; n_out >= 8 and n_out % 8 == 0.  pool:
 * RS_POOL_CLS takes token 0's normalised row (requires desc->has_cls), RS_POOL_MEAN the
 * mean of all tokens' normalised rows. */
typedef struct {
  const void* ln_g;
  const void* ln_b;
  const void* w_head;
  const void* b_head;
  int n_out;
  int pool;               /* an rs_pool */
} rs_head_weights;

/* Patch embedding: images [B][frames][in_chans][height][width] (desc->dtype) ->
 * tokens [B][L][C].  No workspace. */
rs_status rs_patch_embed(const rs_model_desc* desc, const rs_image_desc* img,
                         const rs_embed_weights* emb, const void* images, int B,
                         void* tokens, hipStream_t stream);

/* Final LayerNorm, pooling and head of x [B][L][C]: features [B][C] (the pooled,
 * normalised, affine-transformed row, desc->dtype) and logits [B][n_out] (desc->dtype).
 * workspace/ws_bytes >= rs_head_workspace_bytes(B, L, C): fp32 partial sums of the
 * pooling over blocks of rows. */
rs_status rs_head(const rs_model_desc* desc, const rs_head_weights* head, const void* x,
                  int B, int L, void* features, void* logits, void* workspace, size_t ws_bytes,
                  hipStream_t stream);
/* Host only: workspace bytes of rs_head (0 for sizes outside the limits). */
size_t rs_head_workspace_bytes(int B, int L, int C);

/* Whole forward pass: rs_patch_embed, then rs_encoder_forward with the schedule, then
 * rs_head on the encoder output (whose class token, when present, is its row 0); equal
 * bit for bit to that chain of calls.  The first block's LayerNorm statistics come from
 * the patch embedding's epilogue.
 *  features [B][C], logits [B][n_out]: as rs_head.
 *  out_idx  [B][L_final] original token index of every encoder output row; nullable.
 *  workspace/ws_bytes   >= rs_vit_workspace_bytes(desc, img, depth, B). */
rs_status rs_vit_forward(const rs_model_desc* desc, const rs_image_desc* img,
                         const rs_embed_weights* emb, const rs_block_weights* blocks, int depth,
                         const rs_head_weights* head, const void* images, int B,
                         const int* prune_layers, const double* keep_ratios, int n_prune,
                         void* features, void* logits, int32_t* out_idx,
                         void* workspace, size_t ws_bytes, hipStream_t stream);

/* Host only: workspace bytes that suffice for rs_vit_forward at batch B (any schedule).
 * Returns 0 for an invalid description or geometry. */
size_t rs_vit_workspace_bytes(const rs_model_desc* desc, const rs_image_desc* img, int depth,
                              int B);

/* Host only: token count after the schedule (same rule as rs_encoder_forward). */
rs_status rs_encoder_out_len(int depth, int L, const int* prune_layers,
                             const double* keep_ratios, int n_prune, int* L_final);

/* Host only: workspace bytes that suffice for rs_block_forward and for
 * rs_encoder_forward (any depth >= 1) at batch B and input length L.  Returns 0 for an
 * invalid description. */
size_t rs_workspace_bytes(const rs_model_desc* desc, int depth, int B, int L);

/* Host only: most lanes rs_encoder_forward may use (1 .. 4; default 2).  1 keeps every
 * launch on the caller's stream.  Process-wide; affects calls made after it returns
 * (rs_workspace_bytes covers every lane count). */
rs_status rs_set_max_lanes(int lanes);
/* Host only: the current most-lanes setting (what rs_set_max_lanes last stored, else 2). */
int rs_get_max_lanes(void);

/* Message for the calling thread's last failed call ("" if none); valid until the next
 * call on that thread. */
const char* rs_last_error(void);

/* ---- kernel timing (measurement support; not part of the method) -------------------
 * Between rs_timing_begin(kernel) and rs_timing_end(), every launch of that kernel
 * class made by this library is bracketed by HIP events recorded on the stream it is
 * launched on.  rs_timing_end() waits for those events and returns the summed kernel
 * time (launches of the two encoder lanes may overlap, and each then includes the time
 * it shared the GPU), the number of launches and the summed algorithmic work of those launches
 * (flop for the GEMM and attention kernels, bytes for the memory-bound ones).
 * LayerNorm has no pass of its own: it is applied inside the kernel that consumes it (the
 * QKV kernel and the fused MLP for bf16 widths up to 384, folded into the QKV and fc1 GEMMs
 * otherwise), from row statistics written by the producing kernel; RS_KERNEL_LN_PREP times
 * the remaining preparation (statistics of the encoder input, per-call weight folding and
 * packing).
 * One timing session at a time per process. */
typedef enum {
  RS_KERNEL_LN_PREP = 0,      /* LayerNorm statistics, weight folding and packing */
  RS_KERNEL_QKV = 1,          /* LayerNorm 1 + QKV projection (weight-streaming kernel for
                                 bf16, C <= 384; GEMM otherwise) */
  RS_KERNEL_ATTENTION = 2,
  RS_KERNEL_PROJ = 3,         /* attention output projection (weight-streaming kernel when
                                 the MLP is fused and the attention-sublayer shift is not
                                 the score; GEMM otherwise) */
  RS_KERNEL_FC1 = 4,
  RS_KERNEL_FC2_SCORE = 5,
  RS_KERNEL_TOPK = 6,
  RS_KERNEL_GATHER = 7,       /* reserved: kept rows are copied inside the top-k launch */
  RS_KERNEL_SCORE = 8,
  RS_KERNEL_PATCH = 9,        /* patch-embedding GEMM and class-token rows */
  RS_KERNEL_HEAD = 10,        /* final LayerNorm + pooling, and the head GEMM */
  RS_KERNEL_MAP_SCORE = 11,   /* Eq. (2) / Eq. (3) scores from the attention kernel's sums */
  RS_KERNEL_MLP = 12,         /* the MLP sublayer in one kernel (bf16, C <= 384): LayerNorm 2,
                                 fc1, GELU, fc2, residual and score partials; replaces
                                 RS_KERNEL_FC1 + RS_KERNEL_FC2_SCORE for those widths */
  RS_KERNEL_COUNT = 13
} rs_kernel_id;

rs_status rs_timing_begin(int kernel_id);
rs_status rs_timing_end(float* total_ms, int* launches, double* work);

/* ---- throughput probe (measurement support; not part of the method) ---------------
 * Runs `workgroups` workgroups of 256 threads of a probe kernel on `stream`; each wave
 * iterates `iters` times over the body of `mode` on register data:
 *   0  16 independent hardware exp2          1  16 independent fp32 FMAs
 *   2  the fused attention's softmax of one 64-key x 16-query tile (each lane's 16
 *      scores: maximum, rescale test, exp2, running sum, bf16 packing of P)
 *   3  16 MFMA 16x16x32 bf16 (the matrix work of that tile)
 *   4  the bodies of 2 and 3 interleaved in one wave on independent registers
 *   5  8 LDS reads of 16 bytes per lane (1 KiB per wave, contiguous, conflict free)
 *   6  8 such LDS reads and 8 MFMA 16x16x32 bf16, one fragment per product (the operand
 *      pattern of the fused MLP kernel's weight fragments)
 * Their rates bound the attention kernel: per tile, the matrix cores need the mode-3 time
 * and the vector units the mode-2 time, and mode 4 shows how far one wave overlaps them.
 * sink: device, workgroups * 256 floats, caller-owned; receives one value per thread so
 * the work is kept.  Asynchronous.  RS_ERR_INVALID_ARG for a mode outside 0..6,
 * workgroups < 1, iters < 1 or a null sink. */
rs_status rs_probe_throughput(int mode, int workgroups, int iters, float* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* RS_H_ */
