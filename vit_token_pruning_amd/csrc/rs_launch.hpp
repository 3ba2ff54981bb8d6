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
// Padded key length of the transposed V buffer (whole 64-key tiles).
inline int padded_len(int L) { return (L + 63) / 64 * 64; }

enum GemmEpilogue {
  kEpiQKV = 0,   // + b_qkv; Q|K -> qk [M][2C]; V -> vt [B][H][64][Lp] (transposed per head)
  kEpiBias = 1,  // + bias -> out [M][N]                          (attention projection)
  kEpiGelu = 2,  // GELU(+ bias) -> out [M][N]                      (fc1)
  kEpiFc2 = 3    // y = acc + b2; out = (x + p) + y; part += sum((y - (x + p))^2)
};

struct GemmEpiArgs {
  const void* bias = nullptr;  // [N]
  void* out = nullptr;         // row stride ldo
  int ldo = 0;
  // kEpiQKV: output columns >= vcol0 (= 2C, a multiple of the tile width) are V
  void* vt = nullptr;
  int vcol0 = 0, L = 1, Lp = 64, heads = 1;
  // kEpiFc2: x' = x + p is re-formed in fp32 from the block input and the attention branch
  const void* x = nullptr;
  const void* p = nullptr;
  float* part = nullptr;       // [M][nparts] or null (no scoring)
  int nparts = 0;
};

// Y = A W^T (+ epilogue).  A [M][K], W [N][K]; K % 64 == 0 (bf16) / % 32 (f32).
hipError_t launch_gemm(Dtype dt, GemmEpilogue epi, const void* A, const void* W, int M, int N,
                       int K, const GemmEpiArgs& ep, hipStream_t stream);

// out = LN(x (+ p)) over C per row; p nullable.  C % 8 == 0, C <= 1024.
hipError_t launch_layernorm(Dtype dt, const void* x, const void* p, const void* g, const void* b,
                            float eps, void* out, int M, int C, hipStream_t stream);

// Fused attention, one (sample, head, 64-query block) per workgroup.
// qk [B*L][2C] (Q at columns h*64.., K at C + h*64..), vt [B][H][64][Lp] -> out [B*L][C].
hipError_t launch_attention(Dtype dt, const void* qk, const void* vt, void* out, int B, int L,
                            int H, int Lp, hipStream_t stream);

// scores[r] = || fx[r] - x[r] ||_2 over C.
hipError_t launch_score_rows(Dtype dt, const void* fx, const void* x, float* scores, int M, int C,
                             hipStream_t stream);

// Per-sample exact top-k.  Score source: `scores` [B][L], or when `part` is not null the
// fp32 partial sums of squares [B*L][P] (score = sqrt of their sum).  Writes the
// scores (if scores_out), kept indices ascending [B][k], and (if ids_out) the composed
// original ids ids_out[b][j] = ids_in ? ids_in[b][kept] : kept.
hipError_t launch_topk(const float* scores, const float* part, int P, int B, int L, int k,
                       int has_cls, float* scores_out, int32_t* kept, const int32_t* ids_in,
                       int32_t* ids_out, hipStream_t stream);

// out[b][j][:] = x[b][kept[b][j]][:], rows of row_bytes (multiple of 16).
hipError_t launch_gather(const void* x, const int32_t* kept, void* out, int B, int L, int k,
                         int row_bytes, hipStream_t stream);

// ids[b][i] = i
hipError_t launch_iota(int32_t* ids, int B, int L, hipStream_t stream);

}  // namespace rs
