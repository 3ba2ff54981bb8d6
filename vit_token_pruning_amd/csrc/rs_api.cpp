// Host side of the C ABI declared in include/rs.h: argument validation (complete
// before anything is enqueued), workspace carving, the per-block launch sequence, the
// encoder's pruning schedule, and optional per-kernel event timing.
//
// The schedule follows "Representation Shift: Unifying Token Compression with
// FlashAttention" (arXiv HTML): tokens are pruned after the listed blocks, each time
// keeping a fraction of the *current* tokens (Sec. 4.1 and 4.2 settings); the kept count
// is floor(r*L + 1/2) evaluated in IEEE double.  This file is compiled with
// -ffp-contract=off so that r*L + 1/2 is two correctly rounded operations.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rs.h"
#include "rs_launch.hpp"

static_assert(RS_NOALLOC_SCRATCH_BYTES == rs::kNoallocScratchBytes,
              "the header's scratch limit must match the library's array");

namespace {

thread_local std::string g_err;

rs_status fail(rs_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t esize(int dt) { return dt == RS_BF16 ? 2 : 4; }
bool map_score(const rs_model_desc& d) {
  return d.score_op == RS_MAP_CLS || d.score_op == RS_MAP_MEAN;
}

// floats of score partials per token: one per 64-column slice and partial quantity (map
// scores keep one score per token in the same buffer)
size_t part_stride(const rs_model_desc& d) {
  return (size_t)rs::score_parts(d.C) * rs::dist_quantities((int)d.score_dist);
}
size_t up256(size_t n) { return (n + 255) & ~size_t(255); }

// ------------------------------------------------------------------ kernel timing
std::atomic<int> g_timed_kernel{-1};
std::mutex g_tmu;
std::vector<hipEvent_t> g_ev;  // start/end pairs, reused across sessions
size_t g_ev_used = 0;
double g_work = 0.0;
hipError_t g_timing_err = hipSuccess;

template <class F>
hipError_t timed(int kid, double work, hipStream_t st, F&& launch) {
  if (g_timed_kernel.load(std::memory_order_relaxed) != kid) return launch();
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_ev_used + 2 > g_ev.size()) {
    for (int i = 0; i < 2; ++i) {
      hipEvent_t e;
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) {
        g_timing_err = err;
        return launch();
      }
      g_ev.push_back(e);
    }
  }
  hipEvent_t a = g_ev[g_ev_used], b = g_ev[g_ev_used + 1];
  hipError_t e1 = hipEventRecord(a, st);
  hipError_t err = launch();
  hipError_t e2 = hipEventRecord(b, st);
  if (e1 != hipSuccess || e2 != hipSuccess) g_timing_err = e1 != hipSuccess ? e1 : e2;
  g_ev_used += 2;
  g_work += work;
  return err;
}

// ------------------------------------------------------------------ validation
rs_status check_desc(const rs_model_desc* d) {
  if (!d) return fail(RS_ERR_INVALID_ARG, "desc is null");
  if (d->dtype != RS_F32 && d->dtype != RS_BF16) return fail(RS_ERR_INVALID_ARG, "unknown dtype");
  if (d->C <= 0 || d->heads <= 0 || d->hidden <= 0)
    return fail(RS_ERR_INVALID_ARG, "C, heads and hidden must be positive");
  if (d->C % 64 != 0 || d->heads * 64 != d->C)
    return fail(RS_ERR_UNSUPPORTED, "head dim must be 64 (C == heads*64, C % 64 == 0)");
  if (d->C > 1024) return fail(RS_ERR_UNSUPPORTED, "C > 1024");
  if (d->hidden % 64 != 0) return fail(RS_ERR_UNSUPPORTED, "hidden % 64 != 0");
  if (!(d->ln_eps > 0.0f) || !isfinite(d->ln_eps)) return fail(RS_ERR_INVALID_ARG, "ln_eps must be > 0");
  if (d->has_cls != 0 && d->has_cls != 1) return fail(RS_ERR_INVALID_ARG, "has_cls must be 0 or 1");
  if (d->score_op < RS_SHIFT_MLP || d->score_op > RS_MAP_MEAN)
    return fail(RS_ERR_INVALID_ARG, "unknown score_op");
  if (d->score_op == RS_MAP_CLS && !d->has_cls)
    return fail(RS_ERR_INVALID_ARG, "the class-token attention score needs a class token");
  if (d->attn_map != 0 && d->attn_map != 1) return fail(RS_ERR_INVALID_ARG, "attn_map must be 0 or 1");
  if (d->score_dist != RS_DIST_L2 && d->score_dist != RS_DIST_L1 && d->score_dist != RS_DIST_COS)
    return fail(RS_ERR_INVALID_ARG, "unknown score_dist");
  return RS_OK;
}

rs_status check_BL(int B, int L, int C, int wide) {
  if (B < 1 || L < 1) return fail(RS_ERR_INVALID_ARG, "B and L must be >= 1");
  if (L > RS_MAX_TOKENS) return fail(RS_ERR_UNSUPPORTED, "L > RS_MAX_TOKENS");
  const long long M = (long long)B * L;
  if (M * (long long)(wide > C ? wide : C) >= (1LL << 31))
    return fail(RS_ERR_UNSUPPORTED, "B*L*width must stay below 2^31");
  return RS_OK;
}

rs_status check_ptr(const void* p, const char* name, size_t align = 16) {
  if (!p) return fail(RS_ERR_INVALID_ARG, std::string(name) + " is null");
  if (!aligned(p, align))
    return fail(RS_ERR_INVALID_ARG, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return RS_OK;
}

rs_status check_weights(const rs_block_weights* w) {
  if (!w) return fail(RS_ERR_INVALID_ARG, "weights are null");
  const void* ps[12] = {w->ln1_g, w->ln1_b, w->w_qkv, w->b_qkv, w->w_proj, w->b_proj,
                        w->ln2_g, w->ln2_b, w->w_fc1, w->b_fc1, w->w_fc2, w->b_fc2};
  static const char* names[12] = {"ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj",
                                  "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2"};
  for (int i = 0; i < 12; ++i) {
    rs_status s = check_ptr(ps[i], names[i]);
    if (s != RS_OK) return s;
  }
  return RS_OK;
}

// kept count at a prune block: floor(r * L + 1/2), both steps rounded in double
bool keep_count(double r, int L, int* k) {
  if (!(r > 0.0) || !(r <= 1.0)) return false;
  const double prod = r * (double)L;
  const double kk = floor(prod + 0.5);
  if (kk < 1.0 || kk > (double)L) return false;
  *k = (int)kk;
  return true;
}

rs_status check_schedule(int depth, int L, const int* prune, const double* ratios, int n,
                         int* L_final, std::vector<int>* ks) {
  if (depth < 1) return fail(RS_ERR_INVALID_ARG, "depth must be >= 1");
  if (n < 0) return fail(RS_ERR_INVALID_ARG, "n_prune < 0");
  if (n > 0 && (!prune || !ratios)) return fail(RS_ERR_INVALID_ARG, "prune_layers/keep_ratios null");
  int cur = L;
  for (int i = 0; i < n; ++i) {
    if (prune[i] < 0 || prune[i] >= depth)
      return fail(RS_ERR_INVALID_ARG, "prune layer outside [0, depth)");
    if (i > 0 && prune[i] <= prune[i - 1])
      return fail(RS_ERR_INVALID_ARG, "prune_layers must be strictly ascending");
    int k;
    if (!keep_count(ratios[i], cur, &k))
      return fail(RS_ERR_INVALID_ARG, "keep ratio must be in (0, 1] and keep >= 1 token");
    if (ks) ks->push_back(k);
    cur = k;
  }
  *L_final = cur;
  return RS_OK;
}

// ------------------------------------------------------------------ workspace
struct BlockWs {
  void *qkv, *o, *p, *xp, *h, *xhat;
  float* part;    // score partials of x_hat rows
  float* st_x;    // slice partials of the block input rows (LayerNorm 1)
  float* st_xp;   // slice partials of x' rows (LayerNorm 2)
  float* st_xhat; // slice partials of x_hat rows (next block's LayerNorm 1)
  float* split;   // split-K partial tiles (rs::kSplitWsBytes)
  void* map;      // attention maps [B][H][L][map_pad(L)] (desc.attn_map only)
  float* mapsum;  // Eq. (2) rows [B][H][L] or Eq. (3) column sums [B][H][nq][L] (map scores)
};
struct FoldWs {   // LayerNorm folding of one block: W_qkv diag(gamma1); c, d of QKV and fc1
  void* wq;       // (weight-streaming QKV: W_qkv packed for that kernel instead)
  float *cq, *dq, *c1, *d1;
  void* wpack;    // the fused MLP kernel's packed W1 / W2 (null when the block runs unfused)
  void* ppack;    // W_proj packed for the weight-streaming kernel (null when not used)
};

size_t carve_seq(char* base, const size_t* sizes, int n, void** ptrs) {
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    ptrs[i] = base ? base + off : nullptr;
    off += up256(sizes[i]);
  }
  return off;
}

// Carves the per-block buffers for (B, L) from `base` (or only sizes them if null).
size_t carve_block(const rs_model_desc& d, int B, int L, char* base, BlockWs* ws) {
  const size_t e = esize(d.dtype), M = (size_t)B * L, C = d.C;
  const size_t st = M * rs::stat_stride(d.C) * 8;
  const size_t H = (size_t)d.heads, nq = ((size_t)L + 63) / 64;
  const size_t map_bytes = d.attn_map ? (size_t)B * H * L * rs::map_pad(L) * e : 0;
  const size_t mapsum_bytes = d.score_op == RS_MAP_CLS ? (size_t)B * H * L * 4
                              : d.score_op == RS_MAP_MEAN ? (size_t)B * H * nq * L * 4 : 0;
  const size_t sizes[13] = {
      M * 3 * C * e,                                     // qkv: Q | K | V
      M * C * e,                                         // o: attention output
      M * C * e,                                         // p: attention branch (proj out)
      M * C * e,                                         // xp: x' * gamma2 (fc1 input)
      M * (size_t)d.hidden * e,                          // h: GELU(fc1)
      M * C * e,                                         // xhat: block output
      M * part_stride(d) * 4,                            // part: score partials
      st, st, st,                                        // slice partials
      rs::kSplitWsBytes,                                 // split-K partial tiles
      map_bytes, mapsum_bytes,                           // attention maps, map-score sums
  };
  void* p[13];
  const size_t off = carve_seq(base, sizes, 13, p);
  if (ws) {
    ws->qkv = p[0]; ws->o = p[1]; ws->p = p[2]; ws->xp = p[3]; ws->h = p[4];
    ws->xhat = p[5]; ws->part = static_cast<float*>(p[6]);
    ws->st_x = static_cast<float*>(p[7]); ws->st_xp = static_cast<float*>(p[8]);
    ws->st_xhat = static_cast<float*>(p[9]);
    ws->split = static_cast<float*>(p[10]);
    ws->map = p[11];
    ws->mapsum = static_cast<float*>(p[12]);
  }
  return off;
}

rs::Dtype dtype_of(const rs_model_desc& d);

#ifndef RS_USE_LIN
#define RS_USE_LIN 3
#endif
// The QKV projection runs on the weight-streaming kernel (LayerNorm 1 in the kernel, W_qkv
// packed per call) where it supports the width; the attention projection too when the MLP
// sublayer is fused (the unfused fc1 needs the projection's LayerNorm-2 epilogue).
bool lin_qkv(const rs_model_desc& d) {
  return (RS_USE_LIN & 1) && rs::lin_supported(dtype_of(d), d.C, 3 * d.C);
}
bool lin_proj_packed(const rs_model_desc& d) {
  return (RS_USE_LIN & 2) && rs::lin_supported(dtype_of(d), d.C, d.C) &&
         rs::mlp_fused_supported(dtype_of(d), d.C, d.hidden);
}

size_t carve_fold(const rs_model_desc& d, char* base, FoldWs* fw) {
  const size_t e = esize(d.dtype), C = d.C, Hd = d.hidden;
  const bool fused = rs::mlp_fused_supported(dtype_of(d), d.C, d.hidden);
  const bool pp = lin_proj_packed(d);
  const size_t sizes[7] = {3 * C * C * e, 3 * C * 4, 3 * C * 4, Hd * 4, Hd * 4,
                           fused ? rs::mlp_pack_bytes(d.C, d.hidden) : 0,
                           pp ? rs::lin_pack_bytes(d.C, d.C) : 0};
  void* p[7];
  const size_t off = carve_seq(base, sizes, 7, p);
  if (fw) {
    fw->wq = p[0];
    fw->cq = static_cast<float*>(p[1]); fw->dq = static_cast<float*>(p[2]);
    fw->c1 = static_cast<float*>(p[3]); fw->d1 = static_cast<float*>(p[4]);
    fw->wpack = fused ? p[5] : nullptr;
    fw->ppack = pp ? p[6] : nullptr;
  }
  return off;
}

// One lane of the encoder: the per-block buffers and the running activations for a
// contiguous share of the batch.
struct LaneWs {
  BlockWs blk;
  void* act;      // [B][L][C] running activations
  int32_t* kept;  // [B][L]
  int32_t* ids[2];
};

size_t carve_lane(const rs_model_desc& d, int B, int L, char* base, LaneWs* ws) {
  size_t off = carve_block(d, B, L, base, ws ? &ws->blk : nullptr);
  const size_t sizes[4] = {(size_t)B * L * d.C * esize(d.dtype), (size_t)B * L * 4,
                           (size_t)B * L * 4, (size_t)B * L * 4};
  void* p[4];
  off += carve_seq(base ? base + off : nullptr, sizes, 4, p);
  if (ws) {
    ws->act = p[0];
    ws->kept = static_cast<int32_t*>(p[1]);
    ws->ids[0] = static_cast<int32_t*>(p[2]);
    ws->ids[1] = static_cast<int32_t*>(p[3]);
  }
  return off;
}

// The encoder runs its batch as up to g_max_lanes lanes on as many streams (lane 0 on the
// caller's stream, the others on library streams; lane i takes a contiguous share of
// the samples, the first B % n lanes one sample more) when every lane keeps at least
// kLaneMinRows rows after the last pruning, so one lane's memory-bound epilogues and
// partial last rounds of workgroups overlap another lane's matrix work.  Smaller lanes
// lose more to per-launch latency and extra K splits than the overlap gains (measured:
// UMT-L at 2 x 98 final rows per lane 6.6 % slower, DeiT-S at 128 x 68 5.9 % faster,
// UMT-B at 4 x 196 2.2 % faster).
// rs_block_forward uses one lane.
constexpr int kMaxLanes = 4;
constexpr long kLaneMinRows = 512;
#ifndef RS_DEFAULT_LANES
#define RS_DEFAULT_LANES 2
#endif
std::atomic<int> g_max_lanes{RS_DEFAULT_LANES};
int encoder_lanes(int B, int L_final) {
  int n = g_max_lanes.load();
  while (n > 1 && (B < n || (long)(B / n) * L_final < kLaneMinRows)) --n;
  return n;
}
int lane_batch(int B, int nlanes, int i) { return B / nlanes + (i < B % nlanes ? 1 : 0); }

struct EncWs {
  int nlanes;
  LaneWs lane[kMaxLanes];
  char* fold;     // nfold x carve_fold
};

// Workspace of rs_block_forward (nfold = 1, one lane) and rs_encoder_forward (nfold =
// depth, encoder_lanes(B) lanes).
size_t carve_encoder(const rs_model_desc& d, int nfold, int nlanes, int B, int L, char* base,
                     EncWs* ws) {
  size_t off = 0;
  for (int i = 0; i < nlanes; ++i)
    off += carve_lane(d, lane_batch(B, nlanes, i), L, base ? base + off : nullptr,
                      ws ? &ws->lane[i] : nullptr);
  if (ws) {
    ws->nlanes = nlanes;
    ws->fold = base + off;
  }
  return off + (size_t)nfold * carve_fold(d, nullptr, nullptr);
}

FoldWs fold_of(const rs_model_desc& d, const EncWs& ws, int b) {
  FoldWs fw;
  carve_fold(d, ws.fold + (size_t)b * carve_fold(d, nullptr, nullptr), &fw);
  return fw;
}

// The other lanes' streams and the fork / join events, one set per device, created on
// first use (default priority, non-blocking).  g_lane_mu is held while an encoder call
// enqueues, so calls from several host threads cannot interleave their event records.
struct LaneStreams {
  bool ready = false;
  hipStream_t s[kMaxLanes - 1] = {};
  hipEvent_t fork = nullptr, join[kMaxLanes - 1] = {};
};
std::mutex g_lane_mu;
std::vector<LaneStreams> g_lanes;

// ------------------------------------------------------------------ launch sequence
#define RS_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess) return fail(RS_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

rs::Dtype dtype_of(const rs_model_desc& d) { return d.dtype == RS_BF16 ? rs::kBF16 : rs::kF32; }

// LayerNorm folding of blocks [b0, b0 + n): W_qkv diag(gamma1) with its c, d, and c, d of
// fc1 against gamma2/beta2; up to kMaxFoldJobs / 2 blocks per launch.
rs_status run_fold(const rs_model_desc& d, const rs_block_weights* blocks, const EncWs& ws, int b0,
                   int n, hipStream_t st) {
  for (int b = b0; b < b0 + n; b += rs::kMaxFoldJobs / 2) {
    rs::FoldJob jobs[rs::kMaxFoldJobs];
    int nj = 0;
    double bytes = 0.0;
    for (int i = b; i < b0 + n && i < b + rs::kMaxFoldJobs / 2; ++i) {
      const rs_block_weights& w = blocks[i];
      const FoldWs fw = fold_of(d, ws, i);
      // QKV against LayerNorm 1: W_qkv diag(gamma1) row-major with c, d for the GEMM, or
      // packed for the weight-streaming kernel (which takes d as its bias)
      const bool pq = lin_qkv(d);
      jobs[nj++] = {w.w_qkv, w.ln1_g, w.ln1_b, w.b_qkv, fw.wq, fw.cq, fw.dq, 3 * d.C, pq ? 1 : 0};
      bytes += 2.0 * 3.0 * d.C * d.C * esize(d.dtype);
      // fc1 against LayerNorm 2 (c, d vectors), unless the fused MLP kernel normalises x'
      // itself; then W_proj packed for the weight-streaming kernel (a copy job: no gamma).
      // At most two jobs per block: the packed projection comes only with the fused MLP.
      if (!rs::mlp_fused_supported(dtype_of(d), d.C, d.hidden)) {
        jobs[nj++] = {w.w_fc1, w.ln2_g, w.ln2_b, w.b_fc1, nullptr, fw.c1, fw.d1, d.hidden};
        bytes += (double)d.hidden * d.C * esize(d.dtype);
      } else if (lin_proj_packed(d)) {
        jobs[nj++] = {w.w_proj, nullptr, nullptr, nullptr, fw.ppack, nullptr, nullptr, d.C, 1};
        bytes += 2.0 * d.C * d.C * esize(d.dtype);
      }
    }
    RS_HIP(timed(RS_KERNEL_LN_PREP, bytes, st, [&] {
      return rs::launch_fold(dtype_of(d), jobs, nj, d.C, st);
    }));
  }
  // the fused MLP kernel's packed weights (same blocks, up to kMaxPackJobs per launch)
  if (rs::mlp_fused_supported(dtype_of(d), d.C, d.hidden)) {
    for (int b = b0; b < b0 + n; b += rs::kMaxPackJobs) {
      rs::MlpPackJob jobs[rs::kMaxPackJobs];
      int nj = 0;
      for (int i = b; i < b0 + n && i < b + rs::kMaxPackJobs; ++i)
        jobs[nj++] = {blocks[i].w_fc1, blocks[i].w_fc2, fold_of(d, ws, i).wpack};
      const double bytes = 2.0 * nj * rs::mlp_pack_bytes(d.C, d.hidden);
      RS_HIP(timed(RS_KERNEL_LN_PREP, bytes, st, [&] {
        return rs::launch_mlp_pack(jobs, nj, d.C, d.hidden, st);
      }));
    }
  }
  return RS_OK;
}

rs_status run_row_stats(const rs_model_desc& d, const void* x, float* stats, int M, hipStream_t st) {
  RS_HIP(timed(RS_KERNEL_LN_PREP, (double)M * d.C * esize(d.dtype), st, [&] {
    return rs::launch_row_stats(dtype_of(d), x, stats, M, d.C, st);
  }));
  return RS_OK;
}

// One block: Eq. (5) then Eq. (6), LayerNorms folded.  st_x holds the slice partials of
// the rows of x.  The fc2 epilogue writes x_hat to `out`; the score partials go to `part`
// (nullable; [M][part_stride], from the projection epilogue for the attention-sublayer
// shift, from the fc2 epilogue otherwise) and the slice partials of x_hat to `st_out` (nullable; may alias st_x, which
// nothing reads after the QKV epilogue).  `out` may alias `x` (the fc2 epilogue reads each
// element of x before it writes it, and nothing reads x after that).
void set_score(rs::GemmEpiArgs& ep, const rs_model_desc& d, float* part) {
  ep.part = part;
  ep.nparts = rs::score_parts(d.C);
  ep.pstride = (int)part_stride(d);
  ep.dist = (int)d.score_dist;
  ep.shift_block = d.score_op == RS_SHIFT_BLOCK;
}

rs_status run_block(const rs_model_desc& d, const rs_block_weights& w, const FoldWs& fw,
                    const void* x, const float* st_x, int B, int L, void* out, float* part,
                    float* st_out, const BlockWs& ws, hipStream_t st) {
  const rs::Dtype dt = dtype_of(d);
  const int M = B * L, C = d.C, Hd = d.hidden;
  const double Md = M, Cd = C;
  if (lin_qkv(d)) {
    rs::LinArgs la;
    la.a = x; la.stats = st_x; la.wpack = fw.wq; la.bias_f = fw.dq;
    la.out = ws.qkv; la.ldo = 3 * C; la.eps = d.ln_eps;
    RS_HIP(timed(RS_KERNEL_QKV, 2.0 * Md * 3 * Cd * Cd, st, [&] {
      return rs::launch_lin(dt, la, M, C, 3 * C, st);
    }));
  } else {
    rs::GemmEpiArgs ep;
    ep.out = ws.qkv; ep.ldo = 3 * C;
    ep.stats_in = st_x; ep.fold_c = fw.cq; ep.fold_d = fw.dq; ep.eps = d.ln_eps; ep.C = C;
    ep.split_ws = ws.split;
    RS_HIP(timed(RS_KERNEL_QKV, 2.0 * Md * 3 * Cd * Cd, st, [&] {
      return rs::launch_gemm(dt, rs::kEpiQKV, x, fw.wq, M, 3 * C, C, ep, st);
    }));
  }
  const bool by_map = part && map_score(d);   // this block is scored from its attention map
  if (d.attn_map || by_map) {
    float* cls = by_map && d.score_op == RS_MAP_CLS ? ws.mapsum : nullptr;
    float* colsum = by_map && d.score_op == RS_MAP_MEAN ? ws.mapsum : nullptr;
    RS_HIP(timed(RS_KERNEL_ATTENTION, 4.0 * B * (double)L * L * Cd, st, [&] {
      return rs::launch_attention_map(dt, ws.qkv, ws.o, B, L, d.heads,
                                      d.attn_map ? ws.map : nullptr, rs::map_pad(L), cls, colsum, st);
    }));
  } else {
    RS_HIP(timed(RS_KERNEL_ATTENTION, 4.0 * B * (double)L * L * Cd, st, [&] {
      return rs::launch_attention(dt, ws.qkv, ws.o, B, L, d.heads, st);
    }));
  }
  // The MLP sublayer: one fused kernel (LayerNorm 2, fc1, GELU, fc2, residual, score
  // partials; the hidden activations stay in registers) where the width allows, else fc1
  // with LayerNorm 2 folded and fc2 with the score epilogue.
  const bool fused = rs::mlp_fused_supported(dt, C, Hd);
  if (fw.ppack && !(part && d.score_op == RS_SHIFT_ATTN)) {
    // p alone (no epilogue work): the weight-streaming kernel
    rs::LinArgs la;
    la.a = ws.o; la.wpack = fw.ppack; la.bias = w.b_proj; la.out = ws.p; la.ldo = C;
    RS_HIP(timed(RS_KERNEL_PROJ, 2.0 * Md * Cd * Cd, st, [&] {
      return rs::launch_lin(dt, la, M, C, C, st);
    }));
  } else {
    rs::GemmEpiArgs ep;
    ep.bias = w.b_proj; ep.out = ws.p; ep.ldo = C;
    ep.x = x; ep.C = C;
    if (!fused) {
      // fc1's operand (x' - mean(x)) * gamma2 and LayerNorm 2's slice partials
      ep.out2 = ws.xp; ep.gamma = w.ln2_g; ep.stats_out = ws.st_xp;
      ep.stats_in = st_x;
    }
    ep.split_ws = ws.split;
    if (part && d.score_op == RS_SHIFT_ATTN) set_score(ep, d, part);   // D(p, x)
    RS_HIP(timed(RS_KERNEL_PROJ, 2.0 * Md * Cd * Cd, st, [&] {
      return rs::launch_gemm(dt, rs::kEpiProj, ws.o, w.w_proj, M, C, C, ep, st);
    }));
  }
  const bool mlp_scored = part && (d.score_op == RS_SHIFT_MLP || d.score_op == RS_SHIFT_BLOCK);
  if (fused) {
    rs::MlpArgs ma;
    ma.x = x; ma.p = ws.p; ma.ln_g = w.ln2_g; ma.ln_b = w.ln2_b;
    ma.wpack = fw.wpack; ma.b1 = w.b_fc1; ma.b2 = w.b_fc2;
    ma.out = out; ma.stats_out = st_out; ma.eps = d.ln_eps;
    if (mlp_scored) {
      ma.part = part;
      ma.nparts = rs::score_parts(C);
      ma.pstride = (int)part_stride(d);
      ma.dist = (int)d.score_dist;
      ma.shift_block = d.score_op == RS_SHIFT_BLOCK;
    }
    RS_HIP(timed(RS_KERNEL_MLP, 4.0 * Md * Cd * Hd, st, [&] {
      return rs::launch_mlp(dt, ma, M, C, Hd, st);
    }));
  } else {
    {
      rs::GemmEpiArgs ep;
      ep.out = ws.h; ep.ldo = Hd;
      ep.stats_in = ws.st_xp; ep.fold_c = fw.c1; ep.fold_d = fw.d1; ep.eps = d.ln_eps; ep.C = C;
      ep.split_ws = ws.split;
      RS_HIP(timed(RS_KERNEL_FC1, 2.0 * Md * Cd * Hd, st, [&] {
        return rs::launch_gemm(dt, rs::kEpiGelu, ws.xp, w.w_fc1, M, Hd, C, ep, st);
      }));
    }
    {
      rs::GemmEpiArgs ep;
      ep.bias = w.b_fc2; ep.out = out; ep.ldo = C;
      ep.x = x; ep.p = ws.p;
      if (mlp_scored) set_score(ep, d, part);
      ep.stats_out = st_out; ep.C = C;
      ep.split_ws = ws.split;
      RS_HIP(timed(RS_KERNEL_FC2_SCORE, 2.0 * Md * Cd * Hd, st, [&] {
        return rs::launch_gemm(dt, rs::kEpiFc2, ws.h, w.w_fc2, M, C, Hd, ep, st);
      }));
    }
  }
  if (by_map) {
    // Eq. (2) / Eq. (3) per token into part[0 .. M) (the scores run_select reads)
    const int mode = d.score_op == RS_MAP_CLS ? 0 : 1;
    const double rd = mode == 0 ? (double)B * d.heads * L : (double)B * d.heads * ((L + 63) / 64) * L;
    RS_HIP(timed(RS_KERNEL_MAP_SCORE, rd * 4.0 + Md * 4.0, st, [&] {
      return rs::launch_map_scores(ws.mapsum, ws.mapsum, B, L, d.heads, mode, part, st);
    }));
  }
  return RS_OK;
}

// Top-k of each sample and compaction of the kept rows of x (-> x_kept, nullable) and of
// an optional second row set (x2 -> x2_kept, e.g. the rows' LayerNorm statistics), in one
// launch.
rs_status run_select(int B, int L, int k, int has_cls, const float* scores, const float* part,
                     int P, int dist, float* scores_out, int32_t* kept, const int32_t* ids_in,
                     int32_t* ids_out, const void* x, void* x_kept, size_t row_bytes,
                     hipStream_t st, const void* x2 = nullptr, void* x2_kept = nullptr,
                     size_t row_bytes2 = 0) {
  const double topk_bytes = (double)B * L * 4.0 * (part ? P * rs::dist_quantities(dist) : 1) +
                            (scores_out ? B * L * 4.0 : 0.0) +
                            (double)B * k * 4.0 * (ids_out ? 2 : 1);
  rs::TopkCopy cp[2];
  int nc = 0;
  double copy_bytes = 0.0;
  if (x_kept) {
    cp[nc++] = {x, x_kept, (int)row_bytes};
    copy_bytes += 2.0 * B * k * (double)row_bytes;
  }
  if (x2_kept) {
    cp[nc++] = {x2, x2_kept, (int)row_bytes2};
    copy_bytes += 2.0 * B * k * (double)row_bytes2;
  }
  RS_HIP(timed(RS_KERNEL_TOPK, topk_bytes + copy_bytes, st, [&] {
    return rs::launch_topk(scores, part, P, dist, B, L, k, has_cls, scores_out, kept, ids_in,
                           ids_out, cp, nc, st);
  }));
  return RS_OK;
}

// Lane streams and events of the current device (g_lane_mu held by the caller).
rs_status lane_streams(LaneStreams** out) {
  int dev = 0;
  RS_HIP(hipGetDevice(&dev));
  if ((int)g_lanes.size() <= dev) g_lanes.resize(dev + 1);
  LaneStreams& l = g_lanes[dev];
  if (!l.ready) {
    for (int i = 0; i < kMaxLanes - 1; ++i) {
      RS_HIP(hipStreamCreateWithFlags(&l.s[i], hipStreamNonBlocking));
      RS_HIP(hipEventCreateWithFlags(&l.join[i], hipEventDisableTiming));
    }
    RS_HIP(hipEventCreateWithFlags(&l.fork, hipEventDisableTiming));
    l.ready = true;
  }
  *out = &l;
  return RS_OK;
}

// The encoder over one lane's samples, one block per call of block(): Eq. (5)/(6) blocks,
// scoring and top-k selection after the pruning blocks, kept rows and their LayerNorm
// statistics gathered for the next block.
struct LaneRun {
  const rs_model_desc* d;
  const rs_block_weights* blocks;
  const EncWs* enc;
  const LaneWs* ws;
  int depth, B, L, n_prune;
  const int* prune_layers;
  const std::vector<int>* ks;
  const void* x;
  void* out;
  int32_t* out_idx;
  hipStream_t st;
  const float* x_st = nullptr;  // slice partials of x's rows if already computed (nullable)
  // progress
  const void* cur = nullptr;     // block input
  const float* cur_st = nullptr; // its slice partials (x_st, then ws->blk.st_x)
  int curL = 0, pi = 0;
  const int32_t* ids = nullptr;  // original ids of the current rows (null = identity)

  rs_status begin() {
    cur = x;
    curL = L;
    if (x_st) {
      cur_st = x_st;
      return RS_OK;
    }
    cur_st = ws->blk.st_x;
    return run_row_stats(*d, x, ws->blk.st_x, B * L, st);
  }
  rs_status block(int b) {
    rs_status s;
    const BlockWs& bw = ws->blk;
    const bool prune = pi < n_prune && prune_layers[pi] == b;
    const bool last = b == depth - 1;
    const FoldWs fw = fold_of(*d, *enc, b);
    if (!prune) {
      void* dst = last ? out : ws->act;
      if ((s = run_block(*d, blocks[b], fw, cur, cur_st, B, curL, dst, nullptr,
                         last ? nullptr : bw.st_x, bw, st)) != RS_OK)
        return s;
      cur = dst;
      cur_st = bw.st_x;
      return RS_OK;
    }
    const int k = (*ks)[pi];
    const bool last_prune = pi == n_prune - 1;
    int32_t* ids_out = last_prune ? out_idx : ws->ids[pi & 1];
    void* dst = last ? out : ws->act;
    const size_t row_bytes = (size_t)d->C * esize(d->dtype);
    if ((s = run_block(*d, blocks[b], fw, cur, cur_st, B, curL, bw.xhat, bw.part,
                       last ? nullptr : bw.st_xhat, bw, st)) != RS_OK)
      return s;
    // the kept rows and, unless this is the last block, their LayerNorm statistics
    const size_t stat_bytes = (size_t)rs::stat_stride(d->C) * 8;
    const bool by_map = map_score(*d);
    if ((s = run_select(B, curL, k, d->has_cls, by_map ? bw.part : nullptr,
                        by_map ? nullptr : bw.part, rs::score_parts(d->C),
                        (int)d->score_dist, nullptr,
                        ws->kept, ids, ids_out, bw.xhat, dst, row_bytes, st,
                        last ? nullptr : bw.st_xhat, last ? nullptr : bw.st_x, stat_bytes)) != RS_OK)
      return s;
    cur = dst;
    cur_st = bw.st_x;
    ids = ids_out;
    curL = k;
    ++pi;
    return RS_OK;
  }
  rs_status end() {
    if (n_prune == 0) RS_HIP(rs::launch_iota(out_idx, B, L, st));
    return RS_OK;
  }
  rs_status all() {
    rs_status s;
    if ((s = begin()) != RS_OK) return s;
    for (int b = 0; b < depth; ++b)
      if ((s = block(b)) != RS_OK) return s;
    return end();
  }
};

// The encoder on `x` [B][L][C] (x_st: its rows' slice partials, or null to compute
// them): LayerNorm folding of every block, then the blocks as one or two lanes.
rs_status run_encoder(const rs_model_desc& d, const rs_block_weights* blocks, int depth,
                      const void* x, const float* x_st, int B, int L, const int* prune_layers,
                      int n_prune, const std::vector<int>& ks, int L_final, void* out,
                      int32_t* out_idx, EncWs& enc, hipStream_t stream) {
  rs_status s;
  const int nlanes = enc.nlanes;
  if ((s = run_fold(d, blocks, enc, 0, depth, stream)) != RS_OK) return s;
  const size_t row_bytes = (size_t)d.C * esize(d.dtype);
  LaneRun run[kMaxLanes];
  for (int i = 0, b0 = 0; i < nlanes; ++i) {
    const int Bl = lane_batch(B, nlanes, i);
    LaneRun& r = run[i];
    r.d = &d; r.blocks = blocks; r.enc = &enc; r.ws = &enc.lane[i];
    r.depth = depth; r.B = Bl; r.L = L; r.prune_layers = prune_layers; r.n_prune = n_prune; r.ks = &ks;
    r.x_st = x_st ? x_st + (size_t)b0 * L * rs::stat_stride(d.C) * 2 : nullptr;
    r.x = static_cast<const char*>(x) + (size_t)b0 * L * row_bytes;
    r.out = static_cast<char*>(out) + (size_t)b0 * L_final * row_bytes;
    r.out_idx = out_idx + (size_t)b0 * L_final;
    b0 += Bl;
  }
  if (nlanes == 1) {
    run[0].st = stream;
    return run[0].all();
  }
  // fork the other lanes off the caller's stream, interleave the lanes' launches block by
  // block, and join them back
  std::lock_guard<std::mutex> lk(g_lane_mu);
  LaneStreams* ls = nullptr;
  if ((s = lane_streams(&ls)) != RS_OK) return s;
  run[0].st = stream;
  RS_HIP(hipEventRecord(ls->fork, stream));
  for (int i = 1; i < nlanes; ++i) {
    run[i].st = ls->s[i - 1];
    RS_HIP(hipStreamWaitEvent(ls->s[i - 1], ls->fork, 0));
  }
  for (int i = 0; i < nlanes; ++i)
    if ((s = run[i].begin()) != RS_OK) return s;
  for (int blk = 0; blk < depth; ++blk)
    for (int i = 0; i < nlanes; ++i)
      if ((s = run[i].block(blk)) != RS_OK) return s;
  for (int i = 0; i < nlanes; ++i)
    if ((s = run[i].end()) != RS_OK) return s;
  for (int i = 1; i < nlanes; ++i) {
    RS_HIP(hipEventRecord(ls->join[i - 1], ls->s[i - 1]));
    RS_HIP(hipStreamWaitEvent(stream, ls->join[i - 1], 0));
  }
  return RS_OK;
}

// ------------------------------------------------------------------ around the encoder
// Geometry of the pixel input: tokens per sample L, patch rows per frame, log2 of P.
struct ImageGeom {
  int L, frame_patches, grid_w, lp, K;
};

rs_status check_image(const rs_model_desc& d, const rs_image_desc* img, ImageGeom* g) {
  if (!img) return fail(RS_ERR_INVALID_ARG, "image description is null");
  if (img->frames < 1 || img->in_chans < 1 || img->height < 1 || img->width < 1)
    return fail(RS_ERR_INVALID_ARG, "frames, in_chans, height and width must be >= 1");
  int lp = -1;
  for (int q = 3; q <= 5; ++q)
    if (img->patch == (1 << q)) lp = q;
  if (lp < 0) return fail(RS_ERR_UNSUPPORTED, "patch must be 8, 16 or 32");
  const int P = img->patch;
  if (img->height % P || img->width % P)
    return fail(RS_ERR_INVALID_ARG, "height and width must be multiples of the patch size");
  const long long fp = (long long)(img->height / P) * (img->width / P);
  const long long L = (d.has_cls ? 1 : 0) + (long long)img->frames * fp;
  const long long K = (long long)img->in_chans * P * P;
  if (L > RS_MAX_TOKENS) return fail(RS_ERR_UNSUPPORTED, "tokens per sample > RS_MAX_TOKENS");
  if (K > (1 << 20)) return fail(RS_ERR_UNSUPPORTED, "in_chans * patch^2 too large");
  const long long pix = (long long)img->frames * img->in_chans * img->height * img->width;
  if (pix >= (1LL << 31)) return fail(RS_ERR_UNSUPPORTED, "pixels per sample must stay below 2^31");
  g->L = (int)L;
  g->frame_patches = (int)fp;
  g->grid_w = img->width / P;
  g->lp = lp;
  g->K = (int)K;
  return RS_OK;
}

rs_status check_embed(const rs_model_desc& d, const rs_embed_weights* e) {
  if (!e) return fail(RS_ERR_INVALID_ARG, "embedding weights are null");
  rs_status s;
  if ((s = check_ptr(e->w_patch, "w_patch")) != RS_OK) return s;
  if ((s = check_ptr(e->b_patch, "b_patch")) != RS_OK) return s;
  if ((s = check_ptr(e->pos, "pos")) != RS_OK) return s;
  if (d.has_cls && (s = check_ptr(e->cls, "cls")) != RS_OK) return s;
  return RS_OK;
}

rs_status check_head(const rs_model_desc& d, const rs_head_weights* h) {
  if (!h) return fail(RS_ERR_INVALID_ARG, "head weights are null");
  rs_status s;
  if ((s = check_ptr(h->ln_g, "ln_g")) != RS_OK) return s;
  if ((s = check_ptr(h->ln_b, "ln_b")) != RS_OK) return s;
  if ((s = check_ptr(h->w_head, "w_head")) != RS_OK) return s;
  if ((s = check_ptr(h->b_head, "b_head")) != RS_OK) return s;
  if (h->n_out < 8 || h->n_out % 8 != 0) return fail(RS_ERR_UNSUPPORTED, "n_out must be a positive multiple of 8");
  if (h->pool != RS_POOL_CLS && h->pool != RS_POOL_MEAN) return fail(RS_ERR_INVALID_ARG, "unknown pool");
  if (h->pool == RS_POOL_CLS && !d.has_cls)
    return fail(RS_ERR_INVALID_ARG, "class-token pooling needs a class token (desc->has_cls)");
  return RS_OK;
}

// Patch embedding of B samples into tokens [B][L][C]; the tokens' slice partials to
// `stats` (nullable).  The class-token rows count no work in the timing.
rs_status run_patch(const rs_model_desc& d, const rs_image_desc& img, const ImageGeom& g,
                    const rs_embed_weights& e, const void* images, int B, void* tokens,
                    float* stats, float* split_ws, hipStream_t st) {
  const int C = d.C, Ns = img.frames * g.frame_patches, M = B * Ns;
  rs::GemmEpiArgs ep;
  ep.bias = e.b_patch; ep.out = tokens; ep.ldo = C; ep.pos = e.pos;
  ep.img_h = img.height; ep.img_w = img.width; ep.patch_log2 = g.lp; ep.grid_w = g.grid_w;
  ep.frame_patches = g.frame_patches; ep.sample_patches = Ns; ep.cls_rows = d.has_cls;
  ep.stats_out = stats; ep.C = C; ep.split_ws = split_ws;
  RS_HIP(timed(RS_KERNEL_PATCH, 2.0 * M * (double)C * g.K, st, [&] {
    return rs::launch_gemm(dtype_of(d), rs::kEpiPatch, images, e.w_patch, M, C, g.K, ep, st);
  }));
  if (d.has_cls) {
    RS_HIP(timed(RS_KERNEL_PATCH, 0.0, st, [&] {
      return rs::launch_cls_rows(dtype_of(d), e.cls, e.pos, tokens, stats, B, g.L, C, st);
    }));
  }
  return RS_OK;
}

// Scratch of the head: the pooling's partial sums (room for either pooling).
size_t head_ws_bytes(int B, int L, int C) {
  return up256((size_t)rs::pool_parts(L, 1) * B * C * 4);
}

// Final LayerNorm, pooling and head of x [B][L][C].  The pooling counts no work.
rs_status run_head(const rs_model_desc& d, const rs_head_weights& h, const void* x, int B, int L,
                   void* features, void* logits, float* pool_ws, float* split_ws, hipStream_t st) {
  RS_HIP(timed(RS_KERNEL_HEAD, 0.0, st, [&] {
    return rs::launch_pool(dtype_of(d), x, h.ln_g, h.ln_b, d.ln_eps, B, L, d.C, (int)h.pool,
                           pool_ws, features, st);
  }));
  rs::GemmEpiArgs ep;
  ep.bias = h.b_head; ep.out = logits; ep.ldo = h.n_out; ep.split_ws = split_ws;
  RS_HIP(timed(RS_KERNEL_HEAD, 2.0 * B * (double)h.n_out * d.C, st, [&] {
    return rs::launch_gemm(dtype_of(d), rs::kEpiBias, features, h.w_head, B, h.n_out, d.C, ep, st);
  }));
  return RS_OK;
}

// Workspace of rs_vit_forward: tokens and their slice partials, the encoder output and
// its ids (worst case: no pruning), the head's scratch, then the encoder's own workspace.
struct VitWs {
  void* tokens;
  float* stats;
  void* enc_out;
  int32_t* idx;
  float* head;
  char* enc;
};
size_t carve_vit(const rs_model_desc& d, int depth, int nlanes, int B, int L, char* base, VitWs* ws) {
  const size_t M = (size_t)B * L;
  const size_t sizes[5] = {M * d.C * esize(d.dtype), M * rs::stat_stride(d.C) * 8,
                           M * d.C * esize(d.dtype), M * 4, head_ws_bytes(B, L, d.C)};
  void* p[5];
  const size_t off = carve_seq(base, sizes, 5, p);
  if (ws) {
    ws->tokens = p[0];
    ws->stats = static_cast<float*>(p[1]);
    ws->enc_out = p[2];
    ws->idx = static_cast<int32_t*>(p[3]);
    ws->head = static_cast<float*>(p[4]);
    ws->enc = base + off;
  }
  return off + carve_encoder(d, depth, nlanes, B, L, nullptr, nullptr);
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

const char* rs_last_error(void) { return g_err.c_str(); }

size_t rs_workspace_bytes(const rs_model_desc* desc, int depth, int B, int L) {
  std::string saved = g_err;
  if (check_desc(desc) != RS_OK || depth < 1 || B < 1 || L < 1) {
    g_err = saved;
    return 0;
  }
  // enough for any lane count the encoder may choose
  size_t need = 0;
  for (int n = 1; n <= kMaxLanes && n <= B; ++n) {
    const size_t w = carve_encoder(*desc, depth, n, B, L, nullptr, nullptr);
    if (w > need) need = w;
  }
  return need;
}

rs_status rs_encoder_out_len(int depth, int L, const int* prune_layers, const double* keep_ratios,
                             int n_prune, int* L_final) {
  if (!L_final) return fail(RS_ERR_INVALID_ARG, "L_final is null");
  if (L < 1) return fail(RS_ERR_INVALID_ARG, "L must be >= 1");
  return check_schedule(depth, L, prune_layers, keep_ratios, n_prune, L_final, nullptr);
}

rs_status rs_block_forward(const rs_model_desc* desc, const rs_block_weights* w, const void* x,
                           int B, int L, int keep_k, void* y, float* scores, int32_t* kept_idx,
                           void* y_kept, void* workspace, size_t ws_bytes, hipStream_t stream) {
  rs_status s;
  if ((s = check_desc(desc)) != RS_OK) return s;
  if ((s = check_weights(w)) != RS_OK) return s;
  if ((s = check_BL(B, L, desc->C, desc->hidden > 3 * desc->C ? desc->hidden : 3 * desc->C)) != RS_OK) return s;
  if (keep_k < 1 || keep_k > L) return fail(RS_ERR_INVALID_ARG, "keep_k outside [1, L]");
  if ((s = check_ptr(x, "x")) != RS_OK) return s;
  if (y && (s = check_ptr(y, "y")) != RS_OK) return s;
  if (scores && (s = check_ptr(scores, "scores")) != RS_OK) return s;
  if ((s = check_ptr(kept_idx, "kept_idx")) != RS_OK) return s;
  if ((s = check_ptr(y_kept, "y_kept")) != RS_OK) return s;
  if ((s = check_ptr(workspace, "workspace", 256)) != RS_OK) return s;
  const size_t need = carve_encoder(*desc, 1, 1, B, L, nullptr, nullptr);
  if (ws_bytes < need)
    return fail(RS_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");

  EncWs enc;
  carve_encoder(*desc, 1, 1, B, L, static_cast<char*>(workspace), &enc);
  const LaneWs& ws = enc.lane[0];
  void* xhat = y ? y : ws.blk.xhat;
  if ((s = run_fold(*desc, w, enc, 0, 1, stream)) != RS_OK) return s;
  if ((s = run_row_stats(*desc, x, ws.blk.st_x, B * L, stream)) != RS_OK) return s;
  if ((s = run_block(*desc, *w, fold_of(*desc, enc, 0), x, ws.blk.st_x, B, L, xhat, ws.blk.part,
                     nullptr, ws.blk, stream)) != RS_OK)
    return s;
  const bool by_map = map_score(*desc);
  return run_select(B, L, keep_k, desc->has_cls, by_map ? ws.blk.part : nullptr,
                    by_map ? nullptr : ws.blk.part, rs::score_parts(desc->C),
                    (int)desc->score_dist, scores, kept_idx, nullptr, nullptr, xhat, y_kept,
                    (size_t)desc->C * esize(desc->dtype), stream);
}

rs_status rs_score(const void* fx, const void* x, int B, int L, int C, int dtype, float* scores,
                   hipStream_t stream) {
  return rs_score_dist(fx, x, B, L, C, dtype, RS_DIST_L2, scores, stream);
}

rs_status rs_score_dist(const void* fx, const void* x, int B, int L, int C, int dtype,
                        int dist, float* scores, hipStream_t stream) {
  rs_status s;
  if (dtype != RS_F32 && dtype != RS_BF16) return fail(RS_ERR_INVALID_ARG, "unknown dtype");
  if (dist != RS_DIST_L2 && dist != RS_DIST_L1 && dist != RS_DIST_COS)
    return fail(RS_ERR_INVALID_ARG, "unknown dist");
  if (C < 8 || C % 8 != 0) return fail(RS_ERR_UNSUPPORTED, "C must be a positive multiple of 8");
  if ((s = check_BL(B, L, C, C)) != RS_OK) return s;
  if ((s = check_ptr(fx, "fx")) != RS_OK) return s;
  if ((s = check_ptr(x, "x")) != RS_OK) return s;
  if ((s = check_ptr(scores, "scores")) != RS_OK) return s;
  const int M = B * L;
  RS_HIP(timed(RS_KERNEL_SCORE, (double)M * C * esize(dtype) * 2 + M * 4.0, stream, [&] {
    return rs::launch_score_rows(dtype == RS_BF16 ? rs::kBF16 : rs::kF32, fx, x, scores, M, C,
                                 (int)dist, stream);
  }));
  return RS_OK;
}

size_t rs_attention_workspace_bytes(const rs_model_desc* desc, int B, int L) {
  std::string saved = g_err;
  if (check_desc(desc) != RS_OK || B < 1 || L < 1 || L > RS_MAX_TOKENS) {
    g_err = saved;
    return 0;
  }
  const size_t bhl = (size_t)B * desc->heads * L;
  return up256(bhl * 4) + up256(bhl * ((L + 63) / 64) * 4);
}

}  // extern "C"

namespace {

// rs_attention after its pointer checks, with the scratch of the score sums at `ws`
// (ws_bytes available; none needed when no score is asked).
rs_status run_attention(const rs_model_desc* desc, const void* qkv, int B, int L, void* out,
                        void* map, float* score_cls, float* score_mean, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  const rs::Dtype dt = dtype_of(*desc);
  const double flop = 4.0 * B * (double)L * L * desc->C;
  const size_t bhl = (size_t)B * desc->heads * L;
  if (!map && !score_cls && !score_mean) {
    RS_HIP(timed(RS_KERNEL_ATTENTION, flop, stream, [&] {
      return rs::launch_attention(dt, qkv, out, B, L, desc->heads, stream);
    }));
    return RS_OK;
  }
  float *cls = nullptr, *colsum = nullptr;
  if (score_cls || score_mean) {
    if (ws_bytes < rs_attention_workspace_bytes(desc, B, L))
      return fail(RS_ERR_WORKSPACE, "workspace too small: need " +
                                        std::to_string(rs_attention_workspace_bytes(desc, B, L)) + " bytes");
    if (score_cls) cls = static_cast<float*>(ws);
    if (score_mean) colsum = reinterpret_cast<float*>(static_cast<char*>(ws) + up256(bhl * 4));
  }
  RS_HIP(timed(RS_KERNEL_ATTENTION, flop, stream, [&] {
    return rs::launch_attention_map(dt, qkv, out, B, L, desc->heads, map, rs::map_pad(L), cls,
                                    colsum, stream);
  }));
  if (score_cls)
    RS_HIP(timed(RS_KERNEL_MAP_SCORE, bhl * 4.0 + B * L * 4.0, stream, [&] {
      return rs::launch_map_scores(cls, nullptr, B, L, desc->heads, 0, score_cls, stream);
    }));
  if (score_mean)
    RS_HIP(timed(RS_KERNEL_MAP_SCORE, bhl * ((L + 63) / 64) * 4.0 + B * L * 4.0, stream, [&] {
      return rs::launch_map_scores(nullptr, colsum, B, L, desc->heads, 1, score_mean, stream);
    }));
  return RS_OK;
}

rs_status check_attention(const rs_model_desc* desc, const void* qkv, int B, int L, const void* out,
                          const void* map, const float* score_cls, const float* score_mean) {
  rs_status s;
  if ((s = check_desc(desc)) != RS_OK) return s;
  if ((s = check_BL(B, L, desc->C, 3 * desc->C)) != RS_OK) return s;
  if ((s = check_ptr(qkv, "qkv")) != RS_OK) return s;
  if ((s = check_ptr(out, "out")) != RS_OK) return s;
  if (map && (s = check_ptr(map, "map")) != RS_OK) return s;
  if (score_cls && (s = check_ptr(score_cls, "score_cls", 4)) != RS_OK) return s;
  if (score_mean && (s = check_ptr(score_mean, "score_mean", 4)) != RS_OK) return s;
  return RS_OK;
}

}  // namespace

extern "C" {

rs_status rs_attention(const rs_model_desc* desc, const void* qkv, int B, int L, void* out,
                       void* map, float* score_cls, float* score_mean, void* workspace,
                       size_t ws_bytes, hipStream_t stream) {
  rs_status s;
  if ((s = check_attention(desc, qkv, B, L, out, map, score_cls, score_mean)) != RS_OK) return s;
  if ((score_cls || score_mean) && (s = check_ptr(workspace, "workspace", 256)) != RS_OK) return s;
  return run_attention(desc, qkv, B, L, out, map, score_cls, score_mean, workspace, ws_bytes, stream);
}

rs_status rs_attention_noalloc(const rs_model_desc* desc, const void* qkv, int B, int L, void* out,
                               void* map, float* score_cls, float* score_mean, hipStream_t stream) {
  rs_status s;
  if ((s = check_attention(desc, qkv, B, L, out, map, score_cls, score_mean)) != RS_OK) return s;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (score_cls || score_mean) {
    const size_t need = rs_attention_workspace_bytes(desc, B, L);
    if (need > rs::kNoallocScratchBytes)
      return fail(RS_ERR_UNSUPPORTED, "the score sums need " + std::to_string(need) +
                                          " bytes of scratch, more than the library's fixed " +
                                          std::to_string(rs::kNoallocScratchBytes) +
                                          " (use rs_attention with a workspace)");
    RS_HIP(rs::noalloc_scratch(&ws));
    ws_bytes = rs::kNoallocScratchBytes;
  }
  return run_attention(desc, qkv, B, L, out, map, score_cls, score_mean, ws, ws_bytes, stream);
}

rs_status rs_topk_gather(const float* scores, const void* x, int B, int L, int C, int dtype,
                         int keep_k, int has_cls, int32_t* kept_idx, void* x_kept,
                         hipStream_t stream) {
  rs_status s;
  if (dtype != RS_F32 && dtype != RS_BF16) return fail(RS_ERR_INVALID_ARG, "unknown dtype");
  if (has_cls != 0 && has_cls != 1) return fail(RS_ERR_INVALID_ARG, "has_cls must be 0 or 1");
  if (x_kept && (C < 1 || (C * esize(dtype)) % 16 != 0))
    return fail(RS_ERR_UNSUPPORTED, "row bytes must be a multiple of 16");
  if ((s = check_BL(B, L, C > 0 ? C : 1, C > 0 ? C : 1)) != RS_OK) return s;
  if (keep_k < 1 || keep_k > L) return fail(RS_ERR_INVALID_ARG, "keep_k outside [1, L]");
  if ((s = check_ptr(scores, "scores", 4)) != RS_OK) return s;
  if ((s = check_ptr(kept_idx, "kept_idx", 4)) != RS_OK) return s;
  if (x_kept) {
    if ((s = check_ptr(x, "x")) != RS_OK) return s;
    if ((s = check_ptr(x_kept, "x_kept")) != RS_OK) return s;
  }
  return run_select(B, L, keep_k, has_cls, scores, nullptr, 0, 0, nullptr, kept_idx, nullptr, nullptr, x,
                    x_kept, (size_t)C * esize(dtype), stream);
}

rs_status rs_encoder_forward(const rs_model_desc* desc, const rs_block_weights* blocks, int depth,
                             const void* x, int B, int L, const int* prune_layers,
                             const double* keep_ratios, int n_prune, void* out, int32_t* out_idx,
                             void* workspace, size_t ws_bytes, hipStream_t stream) {
  rs_status s;
  if ((s = check_desc(desc)) != RS_OK) return s;
  if (!blocks) return fail(RS_ERR_INVALID_ARG, "blocks is null");
  if ((s = check_BL(B, L, desc->C, desc->hidden > 3 * desc->C ? desc->hidden : 3 * desc->C)) != RS_OK) return s;
  int L_final = 0;
  std::vector<int> ks;
  if ((s = check_schedule(depth, L, prune_layers, keep_ratios, n_prune, &L_final, &ks)) != RS_OK) return s;
  for (int b = 0; b < depth; ++b)
    if ((s = check_weights(&blocks[b])) != RS_OK)
      return fail(s, "block " + std::to_string(b) + ": " + g_err);
  if ((s = check_ptr(x, "x")) != RS_OK) return s;
  if ((s = check_ptr(out, "out")) != RS_OK) return s;
  if ((s = check_ptr(out_idx, "out_idx", 4)) != RS_OK) return s;
  if ((s = check_ptr(workspace, "workspace", 256)) != RS_OK) return s;
  const int nlanes = encoder_lanes(B, L_final);
  const size_t need = carve_encoder(*desc, depth, nlanes, B, L, nullptr, nullptr);
  if (ws_bytes < need)
    return fail(RS_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");

  EncWs enc;
  carve_encoder(*desc, depth, nlanes, B, L, static_cast<char*>(workspace), &enc);
  return run_encoder(*desc, blocks, depth, x, nullptr, B, L, prune_layers, n_prune, ks, L_final,
                     out, out_idx, enc, stream);
}

rs_status rs_patch_embed(const rs_model_desc* desc, const rs_image_desc* img,
                         const rs_embed_weights* emb, const void* images, int B, void* tokens,
                         hipStream_t stream) {
  rs_status s;
  if ((s = check_desc(desc)) != RS_OK) return s;
  ImageGeom g;
  if ((s = check_image(*desc, img, &g)) != RS_OK) return s;
  if ((s = check_embed(*desc, emb)) != RS_OK) return s;
  if ((s = check_BL(B, g.L, desc->C, g.K > desc->C ? g.K : desc->C)) != RS_OK) return s;
  if ((s = check_ptr(images, "images")) != RS_OK) return s;
  if ((s = check_ptr(tokens, "tokens")) != RS_OK) return s;
  return run_patch(*desc, *img, g, *emb, images, B, tokens, nullptr, nullptr, stream);
}

rs_status rs_head(const rs_model_desc* desc, const rs_head_weights* head, const void* x, int B,
                  int L, void* features, void* logits, void* workspace, size_t ws_bytes,
                  hipStream_t stream) {
  rs_status s;
  if ((s = check_desc(desc)) != RS_OK) return s;
  if ((s = check_head(*desc, head)) != RS_OK) return s;
  if ((s = check_BL(B, L, desc->C, head->n_out > desc->C ? head->n_out : desc->C)) != RS_OK) return s;
  if ((s = check_ptr(x, "x")) != RS_OK) return s;
  if ((s = check_ptr(features, "features")) != RS_OK) return s;
  if ((s = check_ptr(logits, "logits")) != RS_OK) return s;
  if ((s = check_ptr(workspace, "workspace", 256)) != RS_OK) return s;
  if (ws_bytes < head_ws_bytes(B, L, desc->C))
    return fail(RS_ERR_WORKSPACE, "workspace too small: need " +
                                      std::to_string(head_ws_bytes(B, L, desc->C)) + " bytes");
  return run_head(*desc, *head, x, B, L, features, logits, static_cast<float*>(workspace),
                  nullptr, stream);
}

size_t rs_head_workspace_bytes(int B, int L, int C) {
  if (B < 1 || L < 1 || L > RS_MAX_TOKENS || C < 64 || C > RS_MAX_WIDTH || C % 64) return 0;
  return head_ws_bytes(B, L, C);
}

size_t rs_vit_workspace_bytes(const rs_model_desc* desc, const rs_image_desc* img, int depth,
                              int B) {
  std::string saved = g_err;
  ImageGeom g;
  if (check_desc(desc) != RS_OK || depth < 1 || B < 1 || check_image(*desc, img, &g) != RS_OK) {
    g_err = saved;
    return 0;
  }
  size_t need = 0;
  for (int n = 1; n <= kMaxLanes && n <= B; ++n) {
    const size_t w = carve_vit(*desc, depth, n, B, g.L, nullptr, nullptr);
    if (w > need) need = w;
  }
  return need;
}

rs_status rs_vit_forward(const rs_model_desc* desc, const rs_image_desc* img,
                         const rs_embed_weights* emb, const rs_block_weights* blocks, int depth,
                         const rs_head_weights* head, const void* images, int B,
                         const int* prune_layers, const double* keep_ratios, int n_prune,
                         void* features, void* logits, int32_t* out_idx, void* workspace,
                         size_t ws_bytes, hipStream_t stream) {
  rs_status s;
  if ((s = check_desc(desc)) != RS_OK) return s;
  ImageGeom g;
  if ((s = check_image(*desc, img, &g)) != RS_OK) return s;
  if ((s = check_embed(*desc, emb)) != RS_OK) return s;
  if ((s = check_head(*desc, head)) != RS_OK) return s;
  if (!blocks) return fail(RS_ERR_INVALID_ARG, "blocks is null");
  int wide = desc->hidden > 3 * desc->C ? desc->hidden : 3 * desc->C;
  if (g.K > wide) wide = g.K;
  if ((s = check_BL(B, g.L, desc->C, wide)) != RS_OK) return s;
  int L_final = 0;
  std::vector<int> ks;
  if ((s = check_schedule(depth, g.L, prune_layers, keep_ratios, n_prune, &L_final, &ks)) != RS_OK)
    return s;
  for (int b = 0; b < depth; ++b)
    if ((s = check_weights(&blocks[b])) != RS_OK)
      return fail(s, "block " + std::to_string(b) + ": " + g_err);
  if ((s = check_ptr(images, "images")) != RS_OK) return s;
  if ((s = check_ptr(features, "features")) != RS_OK) return s;
  if ((s = check_ptr(logits, "logits")) != RS_OK) return s;
  if (out_idx && (s = check_ptr(out_idx, "out_idx", 4)) != RS_OK) return s;
  if ((s = check_ptr(workspace, "workspace", 256)) != RS_OK) return s;
  const int nlanes = encoder_lanes(B, L_final);
  const size_t need = carve_vit(*desc, depth, nlanes, B, g.L, nullptr, nullptr);
  if (ws_bytes < need)
    return fail(RS_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");

  VitWs vw;
  carve_vit(*desc, depth, nlanes, B, g.L, static_cast<char*>(workspace), &vw);
  EncWs enc;
  carve_encoder(*desc, depth, nlanes, B, g.L, vw.enc, &enc);
  // The patch and head GEMMs never split over K, as in rs_patch_embed and rs_head (which
  // have no workspace), so the whole pass equals the chain of those calls bit for bit.
  if ((s = run_patch(*desc, *img, g, *emb, images, B, vw.tokens, vw.stats, nullptr, stream)) != RS_OK)
    return s;
  if ((s = run_encoder(*desc, blocks, depth, vw.tokens, vw.stats, B, g.L, prune_layers, n_prune,
                       ks, L_final, vw.enc_out, out_idx ? out_idx : vw.idx, enc, stream)) != RS_OK)
    return s;
  return run_head(*desc, *head, vw.enc_out, B, L_final, features, logits, vw.head, nullptr, stream);
}

rs_status rs_probe_throughput(int mode, int workgroups, int iters, float* sink,
                              hipStream_t stream) {
  if (mode < 0 || mode > 6) return fail(RS_ERR_INVALID_ARG, "probe mode must be 0 .. 6");
  if (workgroups < 1 || iters < 1) return fail(RS_ERR_INVALID_ARG, "workgroups and iters must be >= 1");
  rs_status s;
  if ((s = check_ptr(sink, "sink")) != RS_OK) return s;
  RS_HIP(rs::launch_probe(mode, workgroups, iters, sink, stream));
  return RS_OK;
}

rs_status rs_set_max_lanes(int lanes) {
  if (lanes < 1 || lanes > kMaxLanes) return fail(RS_ERR_INVALID_ARG, "lanes must be 1 .. 4");
  g_max_lanes.store(lanes);
  return RS_OK;
}

int rs_get_max_lanes(void) { return g_max_lanes.load(); }

rs_status rs_timing_begin(int kernel_id) {
  if (kernel_id < 0 || kernel_id >= RS_KERNEL_COUNT) return fail(RS_ERR_INVALID_ARG, "bad kernel id");
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_timed_kernel.load() != -1) return fail(RS_ERR_INVALID_ARG, "a timing session is open");
  g_ev_used = 0;
  g_work = 0.0;
  g_timing_err = hipSuccess;
  g_timed_kernel.store(kernel_id);
  return RS_OK;
}

rs_status rs_timing_end(float* total_ms, int* launches, double* work) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (g_timed_kernel.load() == -1) return fail(RS_ERR_INVALID_ARG, "no timing session is open");
  g_timed_kernel.store(-1);
  if (g_timing_err != hipSuccess)
    return fail(RS_ERR_HIP, std::string("timing event: ") + hipGetErrorString(g_timing_err));
  float sum = 0.f;
  for (size_t i = 0; i + 1 < g_ev_used; i += 2) {
    hipError_t e = hipEventSynchronize(g_ev[i + 1]);
    if (e != hipSuccess) return fail(RS_ERR_HIP, std::string("hipEventSynchronize: ") + hipGetErrorString(e));
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_ev[i], g_ev[i + 1]);
    if (e != hipSuccess) return fail(RS_ERR_HIP, std::string("hipEventElapsedTime: ") + hipGetErrorString(e));
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = (int)(g_ev_used / 2);
  if (work) *work = g_work;
  return RS_OK;
}

}  // extern "C"
