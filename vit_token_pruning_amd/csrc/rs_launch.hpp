// Internal launch interface between the host library (rs_api.cpp) and the gfx950
// kernels.  Every function enqueues on `stream` and returns the launch status; none
// validates its arguments (rs_api.cpp does that before anything is enqueued).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace rs {

enum Dtype { kF32 = 0, kBF16 = 1 };

// Row tile of every GEMM: 128 activation rows x 128 output columns.
constexpr int kGemmTile = 128;
// Score partials per token written by the fc2 epilogue: one per 64-column wave slice
// of each 128-column tile.
inline int score_parts(int C) { return 2 * ((C + kGemmTile - 1) / kGemmTile); }

// LayerNorm is folded into the GEMM that consumes it:
//   LN(z) W^T + b = rstd * (z W'^T - mu * c) + d,  W' = W diag(gamma), c = W' 1, d = W beta + b
// Row statistics travel as partials over 64-column slices: (slice mean, slice sum of squared
// deviations from it), merged exactly by the consumer.  A row of partials is padded to an
// even number of slices (16-byte rows).
__host__ __device__ constexpr int stat_slices(int C) { return C / 64; }
__host__ __device__ constexpr int stat_stride(int C) { return (C / 64 + 1) / 2 * 2; }  // float2 per row

enum GemmEpilogue {
  kEpiQKV = 0,   // LN1 folded; Q|K|V -> qkv [M][3C]
  kEpiProj = 1,  // p = acc + b -> out; (x' - a) * gamma2 -> out2 with x' = x + p and a the
                 // row mean of x (from stats_in; 0 if null); LN2 slice partials of x' - a
  kEpiGelu = 2,  // LN2 folded, GELU -> out [M][N]                 (fc1)
  kEpiFc2 = 3,   // y = acc + b2; out = (x + p) + y; score partials; LN1 slice partials of out
  kEpiPatch = 4, // patch embedding: A gathered from images; out row = acc + b + pos, placed
                 // after the sample's class-token row; LN1 slice partials of out
  kEpiBias = 5   // out = acc + b (the head)
};

struct GemmEpiArgs {
  const void* bias = nullptr;  // [N]
  void* out = nullptr;         // row stride ldo
  int ldo = 0;
  // kEpiProj / kEpiFc2: x' = x + p is re-formed in fp32 from the block input and the
  // attention branch
  const void* x = nullptr;
  const void* p = nullptr;
  void* out2 = nullptr;        // kEpiProj: x' * gamma2 in the storage type (fc1's A operand)
  const void* gamma = nullptr; // kEpiProj: LayerNorm 2 gamma [N]
  // representation-shift partials per 64-column slice, or null (no scoring): kEpiProj
  // the attention-sublayer shift D(p, x), kEpiFc2 the MLP-sublayer D(y, x') or, with
  // shift_block, the whole-block D(x_hat, x).  part [M][pstride]; quantity q of slice s at
  // q * nparts + s: L2 sum of squares, L1 sum of magnitudes, cosine (a.b, a.a, b.b).
  float* part = nullptr;
  int nparts = 0, pstride = 0;
  int dist = 0;                // 0 L2, 1 L1, 2 cosine
  int shift_block = 0;
  // folded LayerNorm of the A operand rows (kEpiQKV, kEpiGelu)
  const float* stats_in = nullptr;  // [M][stat_stride] float2 slice partials
  const float* fold_c = nullptr;    // [N]
  const float* fold_d = nullptr;    // [N]
  float eps = 1e-6f;
  int C = 0;                        // LayerNorm width (= K of the consuming GEMM)
  // slice partials of the output rows (kEpiProj: of x'; kEpiFc2: of x_hat)
  float* stats_out = nullptr;
  // split-K partial tiles, kSplitWsBytes; null disables splitting
  float* split_ws = nullptr;
  // kEpiPatch: A is images [frames][K >> 2*patch_log2][img_h][img_w]; GEMM row m is patch
  // m % frame_patches of frame m / frame_patches (raster order, grid_w patches per row),
  // its K columns the patch's pixels in (channel, row, column) order.  Output row of m:
  // m + cls_rows * (m / sample_patches + 1); pos [L][N] is indexed by the row within its
  // sample.
  const void* pos = nullptr;
  int img_h = 0, img_w = 0, patch_log2 = 0, grid_w = 0, frame_patches = 0;
  int sample_patches = 0, cls_rows = 0;
};

// Split-K.  A GEMM with fewer output tiles than kSplitBelow leaves CUs idle (each tile
// is one workgroup); it is then cut into S ranges of K: S * tiles workgroups each write
// an fp32 partial tile, and one reduction workgroup per tile sums the S partials in a
// fixed order and runs the epilogue.  S * tiles <= kSplitTarget <= kSplitMaxTiles, and
// every range keeps at least kSplitMinStages K stages.  The choice depends only on
// (dtype, M, N, K), so equal problems give bit-identical results.
#ifndef RS_SPLIT_BELOW
#define RS_SPLIT_BELOW 256
#endif
#ifndef RS_SPLIT_TARGET
#define RS_SPLIT_TARGET 512
#endif
#ifndef RS_SPLIT_MIN_STAGES
#define RS_SPLIT_MIN_STAGES 8
#endif
#ifndef RS_SPLIT_MAX
#define RS_SPLIT_MAX 16
#endif
constexpr int kSplitBelow = RS_SPLIT_BELOW, kSplitTarget = RS_SPLIT_TARGET;
constexpr int kSplitMinStages = RS_SPLIT_MIN_STAGES, kSplitMaxTiles = 512, kSplitMax = RS_SPLIT_MAX;
static_assert(kSplitTarget <= kSplitMaxTiles, "split buffer is sized for kSplitMaxTiles tiles");
constexpr size_t kSplitWsBytes = (size_t)kSplitMaxTiles * kGemmTile * kGemmTile * 4;
inline int gemm_splits(Dtype dt, int M, int N, int K) {
  const int tiles = ((M + kGemmTile - 1) / kGemmTile) * ((N + kGemmTile - 1) / kGemmTile);
  if (tiles >= kSplitBelow) return 1;
  const int stages = K / (dt == kBF16 ? 64 : 32);
  int s = kSplitTarget / tiles;
  if (s > stages / kSplitMinStages) s = stages / kSplitMinStages;
  if (s > kSplitMax) s = kSplitMax;
  return s < 2 ? 1 : s;
}

// Y = A W^T (+ epilogue).  A [M][K], W [N][K]; K % 64 == 0 (bf16) / % 32 (f32).
hipError_t launch_gemm(Dtype dt, GemmEpilogue epi, const void* A, const void* W, int M, int N,
                       int K, const GemmEpiArgs& ep, hipStream_t stream);

// The MLP sublayer in one kernel (rs_mlp.hip), bf16 and C <= kMlpMaxWidth: LayerNorm 2 of
// x' = x + p, fc1, GELU, fc2, x_hat = x' + MLP(LN(x')) -> out, and the same score partials
// (part, as kEpiFc2) and x_hat slice statistics (stats_out) as the fc2 epilogue.  The
// hidden activations stay in registers.  `out` may alias `x`.
constexpr int kMlpMaxWidth = 384;
struct MlpArgs {
  const void* x = nullptr;      // [M][C] block input
  const void* p = nullptr;      // [M][C] attention branch (x' = x + p)
  const void* ln_g = nullptr;   // [C] LayerNorm 2
  const void* ln_b = nullptr;
  const void* wpack = nullptr;  // W1 and W2 packed by launch_mlp_pack (mlp_pack_bytes)
  const void* b1 = nullptr;     // [hidden]
  const void* b2 = nullptr;     // [C]
  void* out = nullptr;          // [M][C]
  float* part = nullptr;        // nullable; layout of GemmEpiArgs::part
  int nparts = 0, pstride = 0, dist = 0, shift_block = 0;
  float* stats_out = nullptr;   // nullable; [M][stat_stride(C)] float2
  float eps = 1e-6f;
};
bool mlp_fused_supported(Dtype dt, int C, int hidden);
hipError_t launch_mlp(Dtype dt, const MlpArgs& a, int M, int C, int hidden, hipStream_t stream);
// The fused kernel's weight layout: for each 32-unit slice of the hidden layer, the
// slice's W1 rows then its W2 columns, each as the 1 KiB register fragments of the matrix
// products in lane order, so every staging load reads 1 KiB of consecutive bytes.  Packed
// per call (the weights are the caller's, in their own layout) into the workspace.
inline size_t mlp_pack_bytes(int C, int hidden) { return (size_t)2 * C * hidden * 2; }
struct MlpPackJob {
  const void* w1;   // [hidden][C]
  const void* w2;   // [C][hidden]
  void* out;        // mlp_pack_bytes(C, hidden)
};
constexpr int kMaxPackJobs = 16;
hipError_t launch_mlp_pack(const MlpPackJob* jobs, int njobs, int C, int hidden, hipStream_t stream);

// Weight-streaming linear layer (rs_lin.hip), bf16, K = C <= kMlpMaxWidth, N <= kLinMaxN:
// out[m][n] = A'[m] . W'[n] + b'[n].  With `stats` (the rows' slice partials, as
// GemmEpiArgs::stats_in), A' = (A row - mean) * rstd rounded to bf16, W' = W diag(gamma)
// (packed with gamma) and b' = bias_f (fp32: b + W beta), i.e. LayerNorm(A) W^T + b;
// without, A' = A, W' = W and b' = bias (bf16).  The QKV projection with LayerNorm 1 and
// the attention output projection.
constexpr int kLinMaxN = 1536;
struct LinArgs {
  const void* a = nullptr;      // [M][K]
  const float* stats = nullptr; // [M][stat_stride(K)] float2, or null (no LayerNorm)
  const void* wpack = nullptr;  // W' packed by a packed fold job (lin_pack_bytes)
  const void* bias = nullptr;   // [N] bf16 (no LayerNorm)
  const float* bias_f = nullptr;// [N] fp32 (LayerNorm)
  void* out = nullptr;          // [M][ldo]
  int ldo = 0;
  float eps = 1e-6f;
};
bool lin_supported(Dtype dt, int K, int N);
hipError_t launch_lin(Dtype dt, const LinArgs& a, int M, int K, int N, hipStream_t stream);
// W [N][K] (times diag(gamma) when given, rounded to bf16) in the kernel's layout, written
// by launch_fold's packed jobs: per 32-row slice of W, its 1 KiB MFMA register fragments in
// lane order (rows permuted within the slice so that each lane's eight results are eight
// consecutive output columns).
inline size_t lin_pack_bytes(int K, int N) { return (size_t)K * N * 2; }

// Class-token rows of the patch embedding: out[b][0] = cls + pos[0] for b < B (rows of
// L tokens) and their slice partials stats[b * L].
hipError_t launch_cls_rows(Dtype dt, const void* cls, const void* pos, void* out, float* stats,
                           int B, int L, int C, hipStream_t stream);

// Final LayerNorm and pooling of x [B][L][C]: mode 0 the class token's normalised row,
// mode 1 the mean of all rows' normalised rows; feat [B][C] = gamma * pooled + beta.
// part: pool_parts(L, mode) * B * C floats of scratch (sums over blocks of kPoolRows rows).
constexpr int kPoolRows = 32;
inline int pool_parts(int L, int mode) { return mode == 0 ? 1 : (L + kPoolRows - 1) / kPoolRows; }
hipError_t launch_pool(Dtype dt, const void* x, const void* gamma, const void* beta, float eps,
                       int B, int L, int C, int mode, float* part, void* feat, hipStream_t stream);

// Slice partials of every row of x [M][C] -> stats [M][stat_stride(C)] float2.
hipError_t launch_row_stats(Dtype dt, const void* x, float* stats, int M, int C, hipStream_t stream);

// One weight to fold: W [rows][C] with the LayerNorm gamma/beta [C] and Linear bias [rows]
// -> c [rows], d [rows] (fp32) and, if w_out is not null, W' = W diag(gamma) [rows][C] in
// the storage type with c = W' 1 (else c = W gamma).
struct FoldJob {
  const void* w;
  const void* gamma;   // null: W copied unchanged (w_out), no c, d
  const void* beta;
  const void* bias;
  void* w_out;         // nullable
  float* c;
  float* d;
  int rows;
  int packed = 0;      // bf16: w_out in the weight-streaming kernel's layout (lin_pack_bytes)
};
constexpr int kMaxFoldJobs = 32;   // 16 blocks per launch; the arguments stay under 4 KiB
hipError_t launch_fold(Dtype dt, const FoldJob* jobs, int njobs, int C, hipStream_t stream);

// Fused attention, one (sample, head, 64-query block) per workgroup.
// qkv [B*L][3C] (Q at columns h*64.., K at C + h*64.., V at 2C + h*64..) -> out [B*L][C].
hipError_t launch_attention(Dtype dt, const void* qkv, void* out, int B, int L, int H,
                            hipStream_t stream);

// Attention that forms the normalised map (two passes over the keys): out as
// launch_attention; map [B][H][L][Lpad] (nullable; Lpad % 8 == 0, padding keys 0),
// cls [B][H][L] query 0's row (nullable), colsum [B][H][ceil(L/64)][L] per 64-query
// block column sums (nullable).
hipError_t launch_attention_map(Dtype dt, const void* qkv, void* out, int B, int L, int H,
                                void* map, int Lpad, float* cls, float* colsum,
                                hipStream_t stream);
// scores [B][L]: mode 0 mean over heads of cls; mode 1 mean over heads and queries of the
// column sums.
hipError_t launch_map_scores(const float* cls, const float* colsum, int B, int L, int H, int mode,
                             float* scores, hipStream_t stream);
inline int map_pad(int L) { return (L + 7) / 8 * 8; }

// scores[r] = D(fx[r], x[r]) over C; dist 0 L2, 1 L1, 2 cosine.
hipError_t launch_score_rows(Dtype dt, const void* fx, const void* x, float* scores, int M, int C,
                             int dist, hipStream_t stream);

// Per-sample exact top-k (one workgroup per sample, or topk_copy_split(B) when copying
// rows).  Score source: `scores` [B][L], or
// when `part` is not null the fp32 shift partials [B*L][dist_quantities(dist)][P] of the
// GEMM epilogues, finished per distance (L2: sqrt of the sum; L1: the sum; cosine:
// 1 - sum(a.b) / max(sqrt(sum a.a) sqrt(sum b.b), 1e-8)).  Writes the scores (if
// scores_out), kept indices ascending [B][k], and (if ids_out) the composed original ids
// ids_out[b][j] = ids_in ? ids_in[b][kept] : kept.  Then copies the kept rows of up to two
// row sets: dst[b][j] = src[b][kept[b][j]], rows of row_bytes (a multiple of 16).
struct TopkCopy {
  const void* src;
  void* dst;
  int row_bytes;
};
hipError_t launch_topk(const float* scores, const float* part, int P, int dist, int B, int L,
                       int k, int has_cls, float* scores_out, int32_t* kept,
                       const int32_t* ids_in, int32_t* ids_out, const TopkCopy* copies,
                       int ncopies, hipStream_t stream);
// partial quantities per slice of each distance (cosine: a.b, a.a, b.b)
inline int dist_quantities(int dist) { return dist == 2 ? 3 : 1; }
// With row sets to copy, the top-k launch runs topk_copy_split(B) workgroups per sample:
// each makes the same selection and copies its share of the kept rows, so that every batch
// size spreads the copy over about kTopkTargetWgs workgroups (two per CU: one workgroup's
// selection overlaps another's copy; the selection is a few passes over one sample's L
// keys, the copy is what needs the bandwidth).
constexpr int kTopkTargetWgs = 512, kTopkMaxSplit = 128;
inline int topk_copy_split(int B) {
  const int g = (kTopkTargetWgs + B - 1) / B;
  return g < 1 ? 1 : (g > kTopkMaxSplit ? kTopkMaxSplit : g);
}

// Throughput probe (rs_probe.hip): `workgroups` x 256 threads, body `mode`, `iters` times.
hipError_t launch_probe(int mode, int workgroups, int iters, float* sink, hipStream_t stream);

// ids[b][i] = i
hipError_t launch_iota(int32_t* ids, int B, int L, hipStream_t stream);

// Scratch of the entry points that allocate nothing: a device array of this many bytes
// in the library's code object, one per device.  noalloc_scratch() returns the current
// device's copy (its address is looked up once per device and kept).
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void** out);

}  // namespace rs
