// Tile GEMM Y = A W^T on the gfx950 matrix cores with the block's fused epilogues:
// QKV (LayerNorm 1 folded in), attention projection (bias,
// x' = x + p, LayerNorm 2 statistics), fc1 (LayerNorm 2 folded in, GELU) and fc2 (bias,
// residual re-formed in fp32, the per-token partial sums of squares of the MLP-sublayer
// representation shift, and the next block's LayerNorm 1 statistics).
//
// LayerNorm (Sec. 3.3, Eqs. (5) and (6)) is applied without a pass of its own.  With row
// mean mu and 1/std rstd, LN(z) W^T + b = rstd ((z * gamma) W^T - mu c) + d, c = W gamma,
// d = W beta + b.  LayerNorm 1: the GEMM consumes the raw block input z = x against
// W' = W diag(gamma) (c = W' 1), prepared per call with c and d (rs_rowops.hip,
// fold_kernel).  LayerNorm 2: the projection epilogue, which forms x' in fp32, stores
// (x' - a) * gamma for fc1, a = the row mean of the block input (one rounding of a value
// near zero mean, as a LayerNorm output would have, even for rows far from zero mean;
// the shift does not change LN(x')), and fc1 uses its own weights.  Row statistics arrive
// as per-64-column slice partials from the kernel that produced the rows.
//
// The score is Eq. (4) of "Representation Shift: Unifying Token Compression with
// FlashAttention" (arXiv HTML), Sec. 3.2, for the MLP sublayer of Sec. 3.3 (case ii)
// and the L2 distance: || MLP(LN(x')) - x' ||_2.  The fc2 accumulators hold
// MLP(LN(x')) - b2 in fp32; the squared difference to x' is summed in registers while
// the output is written, so the MLP output is never re-read from HBM.
//
// Layout: A [M][K] (activations), W [N][K] (Linear weight, [out][in]); both are
// K-contiguous.  A workgroup of WM x WN waves computes a (WM*TM*16) x (WN*TN*16) tile,
// each wave TM x TN MFMA 16x16x32 tiles.  K advances 64 (bf16) or 32 (fp32) elements
// per LDS stage through two LDS buffers.  bf16 operands go from global memory straight
// into LDS (16 bytes per lane, no register round trip) one stage ahead of the matrix
// work; fp32 operands are staged through registers.  LDS rows hold 128 bytes in chunks
// of 8 elements; chunk c of row r sits at slot c ^ (r % chunks) so 8 consecutive rows
// of a fragment read fall on distinct banks.
//
// Orientation: the weight fragment is the MFMA A operand and the activation fragment
// the B operand, so a lane ends up holding 4 consecutive output columns of one row.
// The epilogue stages the fp32 tile in LDS, row-major, so every global access is a
// row-contiguous line of 8 elements per lane.
#include "rs_device.hpp"
#include "rs_launch.hpp"

namespace rs {
namespace {

// GELU for bf16 outputs.  With Q(t) = 1 - Phi(t) the upper normal tail, Phi(x) = 1 - Q(x)
// for x >= 0 and Q(-x) otherwise, so x Phi(x) = max(x, 0) - |x| Q(|x|) for every x.  Q is
// evaluated as 2^R(t), R a degree-4 polynomial in t = min(|x|, 13) fitted (weighted minimax)
// to log2 Q on [0, 5.5] (beyond, R keeps falling below -25, so the tail term is < 3e-8 |x|):
// one hardware exp2 and no reciprocal.  Max |error| against the exact erf form for finite
// inputs: 6.2e-6 (|x| < 1e4; relative error < 1e-24 beyond).  +-Inf inputs give NaN.
__device__ __forceinline__ float gelu_fitted(float x) {
  const float ax = fabsf(x);
  const float t = fminf(ax, 13.0f);
  float p = fmaf(t, 3.865753533318639e-03f, -4.4075679033994675e-02f);
  p = fmaf(p, t, -4.6802330017089844e-01f);
  p = fmaf(p, t, -1.1473647356033325f);
  p = fmaf(p, t, -1.0004818439483643f);
  const float q = __builtin_amdgcn_exp2f(p);
  return fmaf(-ax, q, fmaxf(x, 0.0f));
}
template <typename T> __device__ __forceinline__ float gelu_t(float x);
template <> __device__ __forceinline__ float gelu_t<bf16>(float x) { return gelu_fitted(x); }
template <> __device__ __forceinline__ float gelu_t<float>(float x) { return gelu_erf(x); }

constexpr int kCS = kGemmTile + 4;  // fp32 row stride of the staged output tile

template <typename T, int WM_, int WN_, int TM_, int TN_, int PF_, int KC_, int HALVES_, int NBUF_>
struct Tile {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_, PF = PF_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int BM = WM * TM * 16, BN = WN * TN * 16;
  static constexpr int KC = KC_;                       // 8-element chunks per row per stage
  static constexpr int CB = Chunk<T>::bytes;
  static constexpr int ROWB = KC * CB;                 // bytes per tile row of a stage
  // chunk c of row r sits at slot c ^ swz(r): any 8 consecutive rows' reads of one
  // chunk then fall on distinct banks
  static __device__ __forceinline__ int swz(int r) { return r % KC; }
  // the epilogue stages the output tile in HALVES pieces of BM / HALVES rows
  static constexpr int HALVES = HALVES_;
  // LDS stage buffers of the direct (bf16) mainloop: 2 = the next stage loads while this
  // one computes; 1 = load, wait, compute (other workgroups on the CU hide the wait)
  static constexpr int NBUF = NBUF_;
  static constexpr int ABYTES = BM * ROWB;
  static constexpr int STAGE = (BM + BN) * ROWB;
  static constexpr int NA = BM * KC / NT, NW = BN * KC / NT;
  static constexpr int RSTEP = NT / KC;
  static_assert((BM * KC) % NT == 0 && (BN * KC) % NT == 0, "loader must divide evenly");
  static_assert(ROWB == 128, "stage rows of 128 bytes");
};

// Representation-shift partials of 8 columns, distance `dist` between a and b (Sec. 3.3
// "Distance metrics"): 0 L2 -> s0 += sum (a-b)^2; 1 L1 -> s0 += sum |a-b|; 2 cosine ->
// s0 += a.b, s1 += a.a, s2 += b.b (finished per token after the slices are summed).
__device__ __forceinline__ void shift_partials(int dist, const float* a, const float* b,
                                               float& s0, float& s1, float& s2) {
  if (dist == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = a[e] - b[e];
      s0 += d * d;
    }
  } else if (dist == 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s0 += fabsf(a[e] - b[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s0 += a[e] * b[e];
      s1 += a[e] * a[e];
      s2 += b[e] * b[e];
    }
  }
}

// The epilogue of one 128 x 128 output tile, shared by the direct path and the split-K
// reduction.  `stage(Cs, h)` writes rows [h BM/HALVES, (h+1) BM/HALVES) of the tile's fp32
// accumulators to LDS as Cs[m - h BM/HALVES][n]; every LDS byte is free when it is first
// called.  Staging in two halves halves the epilogue's LDS, so that more workgroups fit
// on a CU.
template <typename T, int EPI, class G, class Stage>
__device__ __forceinline__ void tile_epilogue(char* smem, const GemmEpiArgs& ep, int M, int N,
                                              int m0, int n0, int nt, Stage&& stage) {
  static_assert(G::BM == 128 && G::BN == 128 && G::NT == 256, "epilogue assumes 128x128, 256 threads");
  constexpr int NPASS = G::BM / 16, HALVES = G::HALVES, HP = NPASS / HALVES;
  constexpr int HROWS = G::BM / HALVES;
  constexpr bool kFold = EPI == kEpiQKV || EPI == kEpiGelu;   // LayerNorm folded into A
  constexpr bool kResid = EPI == kEpiProj || EPI == kEpiFc2;
  constexpr bool kPatch = EPI == kEpiPatch;
  const int tid = threadIdx.x;
  const int er = tid >> 4, sub = tid & 15, ec = sub * 8;       // row pass: 16 threads per row
  const int n = n0 + ec;
  const bool col_ok = n < N;
  const int nsl = stat_slices(ep.C), sstride = stat_stride(ep.C);

  // Epilogue inputs from global memory (row statistics, x, p) for all of this thread's
  // rows are requested before the tile is staged, so their latency overlaps the staging
  // instead of being paid once per row pass.
  // kFold: thread t < 128 fetches all slice partials of tile row t (at most 16)
  float2 rpart[16];
  if (kFold && tid < G::BM) {
    const int m = m0 + tid;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      rpart[q] = make_float2(0.f, 0.f);
      if (q < nsl && m < M)
        rpart[q] = *reinterpret_cast<const float2*>(ep.stats_in + ((size_t)m * sstride + q) * 2);
    }
  }
  // kEpiProj: thread t < 128 fetches the slice means of the block input's row t (x's
  // statistics, when given): its row mean, subtracted from x' before x' * gamma2 is stored
  float rmean[16];
  const bool kShift = EPI == kEpiProj && ep.stats_in != nullptr;
  if (kShift && tid < G::BM) {
    const int m = m0 + tid;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      rmean[q] = 0.f;
      if (q < nsl && m < M) rmean[q] = ep.stats_in[((size_t)m * sstride + q) * 2];
    }
  }
  Frag8<T> px[NPASS], pp[NPASS];           // kResid: x (and p) of each row; kPatch: pos
  if (kResid || kPatch) {
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      const int m = m0 + pass * 16 + er;
      if (m < M && col_ok) {
        if (kPatch) {
          const int prow = m % ep.sample_patches + ep.cls_rows;   // row within the sample
          load_frag(px[pass], static_cast<const T*>(ep.pos) + (size_t)prow * N + n);
        } else {
          load_frag(px[pass], static_cast<const T*>(ep.x) + (size_t)m * N + n);
        }
        if (EPI == kEpiFc2) load_frag(pp[pass], static_cast<const T*>(ep.p) + (size_t)m * N + n);
      }
    }
  }
  // per-column constants of this thread's 8 columns
  float b8[8], g8[8], c8[8], d8[8];
  if (col_ok) {
    if (kFold) {
#pragma unroll
      for (int e = 0; e < 8; ++e) { c8[e] = ep.fold_c[n + e]; d8[e] = ep.fold_d[n + e]; }
    } else {
      load8f(static_cast<const T*>(ep.bias) + n, b8);
      // gamma2 only scales fc1's operand, which is not stored when out2 is null
      if (EPI == kEpiProj && ep.out2) load8f(static_cast<const T*>(ep.gamma) + n, g8);
    }
  }

  float* Cs = reinterpret_cast<float*>(smem);

  // folded LayerNorm: each tile row's (mean * rstd, rstd), merged once from its slice
  // partials (equal-count merge) and shared through LDS
  float2* Rs = reinterpret_cast<float2*>(smem + HROWS * kCS * 4);
  if (kFold && tid < G::BM) {
    float mean = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) mean += rpart[q].x;  // absent slices hold 0
    mean *= __builtin_amdgcn_rcpf((float)nsl);
    float m2 = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (q < nsl) {
        const float dm = rpart[q].x - mean;
        m2 += rpart[q].y + 64.f * dm * dm;
      }
    // hardware reciprocal and reciprocal square root (about 1 ulp each)
    const float rstd = __builtin_amdgcn_rsqf(fmaf(m2, __builtin_amdgcn_rcpf((float)ep.C), ep.eps));
    Rs[tid] = make_float2(mean * rstd, rstd);
  }
  if (kShift && tid < G::BM) {
    float mean = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) mean += rmean[q];  // absent slices hold 0
    Rs[tid] = make_float2(mean * __builtin_amdgcn_rcpf((float)nsl), 0.f);
  }

  // row pass: 8 consecutive columns per thread; lanes 0-7 / 8-15 of a row cover its two
  // 64-column slices of this tile
  const int slice = nt * 2 + (sub >> 3);          // 64-column slice of the row
  T* out = static_cast<T*>(ep.out);
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    if (pass % HP == 0) {
      if (pass > 0) __syncthreads();   // the previous half's row passes are done with Cs
      stage(Cs, pass / HP);
      __syncthreads();
    }
    const int mm = pass * 16 + er, m = m0 + mm, ms = mm - (pass / HP) * HROWS;
    const bool row_ok = m < M;
    const bool ok = col_ok && row_ok;
    float v[8];
    {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(Cs + ms * kCS + ec);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(Cs + ms * kCS + ec + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = lo[e]; v[4 + e] = hi[e]; }
    }
    if (kFold) {
      const float mr = Rs[mm].x, rstd = Rs[mm].y;
      if (ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[e] = fmaf(rstd, v[e], fmaf(-mr, c8[e], d8[e]));   // rstd (acc - mean c) + d
          if (EPI == kEpiGelu) v[e] = gelu_t<T>(v[e]);
        }
        store8f(out + (size_t)m * ep.ldo + n, v);
      }
      continue;
    }
    if (EPI == kEpiBias) {
      if (ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += b8[e];
        store8f(out + (size_t)m * ep.ldo + n, v);
      }
      continue;
    }
    // output row: the patch embedding leaves room for each sample's class-token row
    const size_t orow = kPatch ? (size_t)m + (ep.cls_rows ? m / ep.sample_patches + 1 : 0)
                               : (size_t)m;
    // kEpiProj / kEpiFc2: the output row in fp32 plus its slice partials, and when scoring
    // the representation-shift partials of this thread's columns: s0 (L2: sum of squared
    // differences, L1: sum of |differences|, cosine: sum a.b), s1 and s2 (cosine: a.a, b.b)
    float s0 = 0.f, s1 = 0.f, s2 = 0.f;
    float w[8];            // stored values whose slice partials are emitted
    if (ok) {
      float xv[8], pv[8];
      frag_to_f32(px[pass], xv);
      if (kPatch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = round_t<T>(v[e] + b8[e] + xv[e]);   // + pos
        store8f(out + orow * ep.ldo + n, w);
      } else if (EPI == kEpiProj) {
        // LayerNorm is invariant to a shift of its row, so fc1's operand and LayerNorm 2's
        // statistics are taken of x' - a, a = the row mean of the block input x (0 when its
        // statistics are not given).  x' - a is near zero mean even for rows far from
        // zero mean, so storing (x' - a) * gamma2 in the storage type keeps its precision
        // relative to the row's spread, as storing the normalised row would.
        const float a = kShift ? Rs[mm].x : 0.f;
        float pf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pf[e] = v[e] + b8[e];               // attention branch SA(LN(x)) in fp32
          pv[e] = round_t<T>(pf[e]);          // ... as stored
          w[e] = (xv[e] - a) + pv[e];         // x' (Eq. 5) - a in fp32: LayerNorm 2 statistics
        }
        store8f(out + (size_t)m * ep.ldo + n, pv);
        if (ep.out2) {
          float u[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) u[e] = w[e] * g8[e];   // (x' - a) * gamma2: fc1's A operand
          store8f(static_cast<T*>(ep.out2) + (size_t)m * N + n, u);
        }
        if (ep.part) shift_partials(ep.dist, pf, xv, s0, s1, s2);   // D(SA(LN(x)), x)
      } else if (ep.dist == 0 && !ep.shift_block) {
        // the method: || MLP(LN(x')) - x' ||_2
        frag_to_f32(pp[pass], pv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = v[e] + b8[e];   // MLP(LN(x'))
          const float xp = xv[e] + pv[e]; // x' (Eq. 5), re-formed in fp32
          const float d = y - xp;
          s0 += d * d;
          w[e] = round_t<T>(xp + y);      // x_hat (Eq. 6), as stored
        }
        store8f(out + (size_t)m * ep.ldo + n, w);
      } else {
        frag_to_f32(pp[pass], pv);
        float fa[8], fb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = v[e] + b8[e];
          const float xp = xv[e] + pv[e];
          fa[e] = ep.shift_block ? xp + y : y;       // x_hat | MLP(LN(x'))
          fb[e] = ep.shift_block ? xv[e] : xp;       // x     | x'
          w[e] = round_t<T>(xp + y);
        }
        store8f(out + (size_t)m * ep.ldo + n, w);
        if (ep.part) shift_partials(ep.dist, fa, fb, s0, s1, s2);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = 0.f;
    }
    // slice partials of the stored row values (8 lanes = one 64-column slice)
    float ssum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ssum += w[e];
    const float smean = sum8(ssum) * (1.0f / 64.0f);
    float sm2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dd = w[e] - smean;
      sm2 = fmaf(dd, dd, sm2);   // explicit: every statistics producer rounds alike
    }
    sm2 = sum8(sm2);
    if ((sub & 7) == 0 && row_ok && slice < nsl && ep.stats_out) {
      float* so = ep.stats_out + (orow * sstride + slice) * 2;
      so[0] = smean;
      so[1] = sm2;
    }
    if (!kPatch && ep.part) {
      s0 = sum8(s0);
      if (ep.dist == 2) {
        s1 = sum8(s1);
        s2 = sum8(s2);
      }
      if ((sub & 7) == 0 && row_ok) {
        float* pr = ep.part + (size_t)m * ep.pstride + slice;
        pr[0] = s0;
        if (ep.dist == 2) {
          pr[ep.nparts] = s1;
          pr[2 * ep.nparts] = s2;
        }
      }
    }
  }
}

// SPLIT == false: one workgroup per output tile over all of K, then the tile epilogue.
// SPLIT == true: `splits` workgroups per tile, each over one contiguous range of K stages,
// writing its fp32 partial tile to ep.split_ws [split][M][N]; splitk_reduce_kernel finishes.
// Launch ids are spread XCD-contiguously, and in split mode the splits of one tile are
// neighbours, so a tile's partials and its reduction share an XCD's L2.
template <typename T, int EPI, class G, bool SPLIT>
__global__ __launch_bounds__(G::NT) void gemm_kernel(const T* __restrict__ A,
                                                     const T* __restrict__ W, int M, int N,
                                                     int K, int splits, GemmEpiArgs ep) {
  constexpr int KC = G::KC, CB = G::CB, ROWB = G::ROWB, STAGE = G::STAGE, ABYTES = G::ABYTES;
  constexpr int NA = G::NA, NW = G::NW, RSTEP = G::RSTEP, TM = G::TM, TN = G::TN, PF = G::PF;
  // pipeline stages, or the staged fp32 tile plus one float2 per tile row
  constexpr int EBYTES = SPLIT ? 0 : (G::BM / G::HALVES) * kCS * 4 + G::BM * 8;
  constexpr int NBUF = sizeof(T) == 2 ? G::NBUF : 2;
  constexpr int SMEM = NBUF * STAGE > EBYTES ? NBUF * STAGE : EBYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int nM = (M + G::BM - 1) / G::BM, nN = (N + G::BN - 1) / G::BN;
  const int KTall = K / (8 * KC);
  int t, split = 0, kt0 = 0, KT = KTall;
  if (SPLIT) {
    const int u = xcd_contiguous(blockIdx.x, nM * nN * splits);
    t = u / splits;
    split = u - t * splits;
    kt0 = split * KTall / splits;
    KT = (split + 1) * KTall / splits - kt0;
  } else {
    t = xcd_contiguous(blockIdx.x, nM * nN);
  }
  const int mt = t / nN, nt = t - mt * nN;
  const int m0 = mt * G::BM, n0 = nt * G::BN;
  const int wm = wave % G::WM, wn = wave / G::WM;

  // ---- loader: this thread's chunks of A and W, and their swizzled LDS slots.  Thread t
  // moves chunk lc = t % KC of rows lr + i * RSTEP (lr = t / KC).  bf16: each row is 8
  // chunks of 16 bytes and a wave covers 8 whole rows = 1 KiB of LDS, which is the unit
  // of the direct global -> LDS load; lane lc then fetches global chunk lc ^ (r % 8) so
  // that slot lc holds it (the swizzle is an involution).  fp32 (32-byte chunks) goes
  // through registers.
  constexpr bool kDirect = sizeof(T) == 2;
  // kEpiPatch: A rows are image patches (im2col in the loader).  A chunk is 8 consecutive
  // pixels of one patch row (the patch width is a multiple of 8), so it is contiguous in
  // the image; its address is the patch origin plus an offset that depends on k only.
  constexpr bool kPatchA = EPI == kEpiPatch;
  const int lc = tid % KC, lr = tid / KC;
  const char* ag[NA];
  const char* wg[NW];
  int sa[NA], sw[NW], ak[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = lr + i * RSTEP;
    const int c = kDirect ? (lc ^ G::swz(r)) : lc;
    if constexpr (kPatchA) {
      const int m = min(m0 + r, M - 1), lp = ep.patch_log2;
      const int f = m / ep.frame_patches, q = m - f * ep.frame_patches;
      const int pr = q / ep.grid_w, pc = q - pr * ep.grid_w;
      const size_t cin = (size_t)(K >> (2 * lp));
      ag[i] = reinterpret_cast<const char*>(
          A + ((f * cin * ep.img_h + ((size_t)pr << lp)) * ep.img_w + ((size_t)pc << lp)));
      ak[i] = kt0 * KC * 8 + c * 8;    // k of this chunk at stage 0
    } else {
      ag[i] = reinterpret_cast<const char*>(A + (size_t)min(m0 + r, M - 1) * K) + (size_t)kt0 * ROWB + c * CB;
    }
    sa[i] = r * ROWB + ((lc ^ G::swz(r)) * CB);
  }
  // byte offset of A chunk i at stage kt (from ag[i])
  auto aoff = [&](int i, int kt) -> size_t {
    if constexpr (kPatchA) {
      const int k = ak[i] + kt * KC * 8, lp = ep.patch_log2, pm = (1 << lp) - 1;
      const int ch = k >> (2 * lp), py = (k >> lp) & pm, pxl = k & pm;
      return (((size_t)ch * ep.img_h + py) * ep.img_w + pxl) * sizeof(T);
    } else {
      return (size_t)kt * ROWB;
    }
  };
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int r = lr + i * RSTEP;
    const int c = kDirect ? (lc ^ G::swz(r)) : lc;
    wg[i] = reinterpret_cast<const char*>(W + (size_t)min(n0 + r, N - 1) * K) + (size_t)kt0 * ROWB + c * CB;
    sw[i] = ABYTES + r * ROWB + ((lc ^ G::swz(r)) * CB);
  }
  Frag8<T> ra[PF][NA], rw[PF][NW];
  auto gload = [&](int kt, int slot) {
    const size_t off = (size_t)kt * ROWB;
#pragma unroll
    for (int i = 0; i < NA; ++i) load_frag(ra[slot][i], ag[i] + aoff(i, kt));
#pragma unroll
    for (int i = 0; i < NW; ++i) load_frag(rw[slot][i], wg[i] + off);
  };
  auto sstore = [&](int slot, int buf) {
    char* s = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < NA; ++i) store_frag(s + sa[i], ra[slot][i]);
#pragma unroll
    for (int i = 0; i < NW; ++i) store_frag(s + sw[i], rw[slot][i]);
  };
  // direct: this wave's 1 KiB blocks of stage kt, rows wave * 8 + i * RSTEP ..
  auto dload = [&](int kt, int buf) {
    char* s = smem + buf * STAGE;
    const size_t off = (size_t)kt * ROWB;
#pragma unroll
    for (int i = 0; i < NA; ++i) load_lds16(ag[i] + aoff(i, kt), s + (wave * (64 / KC) + i * RSTEP) * ROWB);
#pragma unroll
    for (int i = 0; i < NW; ++i) load_lds16(wg[i] + off, s + ABYTES + (wave * (64 / KC) + i * RSTEP) * ROWB);
  };

  f32x4 acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const char* As = smem + buf * STAGE;
    const char* Ws = As + ABYTES;
#pragma unroll
    for (int ks = 0; ks < KC / 4; ++ks) {
      const int c = ks * 4 + g;
      Frag8<T> fa[TM], fw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * TM * 16 + i * 16 + l16;
        load_frag(fa[i], As + r * ROWB + ((c ^ G::swz(r)) * CB));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * TN * 16 + j * 16 + l16;
        load_frag(fw[j], Ws + r * ROWB + ((c ^ G::swz(r)) * CB));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[j][i] = mma16(acc[j][i], fw[j], fa[i]);
    }
  };

  if constexpr (kDirect) {
    // Two LDS buffers; the loads of stage kt + 1 are issued right after the barrier that
    // ends stage kt - 1 (whose buffer they overwrite) and land during stage kt's matrix work.
    static_assert(NA + NW > 0 && 64 % KC == 0, "direct loads: whole rows per wave");
    if constexpr (NBUF == 1) {
      for (int kt = 0; kt < KT; ++kt) {
        if (kt > 0) barrier_nofence();   // every wave's reads of stage kt - 1 are done
        dload(kt, 0);
        wait_vmem<0>();                  // this wave's part of stage kt is in LDS
        barrier_nofence();               // ... and every wave's
        compute(0);
      }
    } else {
      dload(0, 0);
      for (int kt = 0; kt < KT; ++kt) {
        wait_vmem<0>();          // this wave's part of stage kt is in LDS
        barrier_nofence();       // ... and every wave's; stage kt - 1's reads are done
        if (kt + 1 < KT) dload(kt + 1, (kt + 1) & 1);
        compute(kt & 1);
      }
    }
    __syncthreads();           // LDS is reused by the epilogue
  } else {
    gload(0, 0);
    sstore(0, 0);
    if (PF > 1 && KT > 1) gload(1, 1 % PF);
    __syncthreads();
    // One stage.  PF == 2: the next stage's registers arrived during the previous stage,
    // so they are written to the free LDS buffer first and those writes overlap this
    // stage's matrix work; then loads two stages ahead are issued.  PF == 1: loads one
    // stage ahead, written to LDS after the matrix work.
    auto step = [&](int kt, auto ls, auto ss) {
      if (PF > 1 && kt + 1 < KT) sstore(decltype(ss)::value, (kt + 1) & 1);
      if (kt + PF < KT) gload(kt + PF, decltype(ls)::value);
      compute(kt & 1);
      if (PF == 1 && kt + 1 < KT) sstore(decltype(ss)::value, (kt + 1) & 1);
      __syncthreads();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1 % PF>;
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      // PF == 2: stage kt -> slot 0 (loaded into for kt + 2), stored from slot 1;
      // PF == 1: single slot
      step(kt, I0{}, I1{});
      step(kt + 1, I1{}, I0{});
    }
    if (kt < KT) step(kt, I0{}, I1{});
  }

  // acc[j][i] = D[n][m]: lane holds row m, columns n..n+3
  if (SPLIT) {
    // partial tile straight from registers: 16-byte stores, 64 contiguous bytes per row
    float* ps = ep.split_ws + (size_t)split * M * N;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm * TM * 16 + i * 16 + l16, n = n0 + wn * TN * 16 + j * 16 + 4 * g;
        if (m < M && n < N) *reinterpret_cast<f32x4*>(ps + (size_t)m * N + n) = acc[j][i];
      }
    return;
  }
  tile_epilogue<T, EPI, G>(smem, ep, M, N, m0, n0, nt, [&](float* Cs, int h) {
    constexpr int HROWS = G::BM / G::HALVES;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = wm * TM * 16 + i * 16 + l16, n = wn * TN * 16 + j * 16 + 4 * g;
        if (m / HROWS == h) *reinterpret_cast<f32x4*>(Cs + (m - h * HROWS) * kCS + n) = acc[j][i];
      }
  });
}

// Split-K reduction: one workgroup per output tile sums the `splits` partial tiles in
// split order (a fixed order, so the result is deterministic) into LDS and runs the same
// tile epilogue as the direct path.
template <typename T, int EPI, class G>
__global__ __launch_bounds__(G::NT) void splitk_reduce_kernel(int M, int N, int splits, GemmEpiArgs ep) {
  __shared__ __attribute__((aligned(16))) char smem[(G::BM / G::HALVES) * kCS * 4 + G::BM * 8];
  constexpr int NPASS = G::BM / 16;
  const int nM = (M + G::BM - 1) / G::BM, nN = (N + G::BN - 1) / G::BN;
  const int t = xcd_contiguous(blockIdx.x, nM * nN);
  const int mt = t / nN, nt = t - mt * nN;
  const int m0 = mt * G::BM, n0 = nt * G::BN;
  f32x4 a[NPASS][2];
  const int tid = threadIdx.x, er = tid >> 4, ec = (tid & 15) * 8;
  tile_epilogue<T, EPI, G>(smem, ep, M, N, m0, n0, nt, [&](float* Cs, int h) {
    constexpr int HP = NPASS / G::HALVES;
    if (h > 0) {
#pragma unroll
      for (int pass = h * HP; pass < (h + 1) * HP; ++pass) {
        const int mm = (pass - h * HP) * 16 + er;
        *reinterpret_cast<f32x4*>(Cs + mm * kCS + ec) = a[pass][0];
        *reinterpret_cast<f32x4*>(Cs + mm * kCS + ec + 4) = a[pass][1];
      }
      return;
    }
    // Rows and columns past the matrix edge read a clamped, written element instead of
    // branching, so a split's 16 loads per thread are all in flight together; the
    // epilogue never uses those LDS entries.
    const size_t ncl = (size_t)min(n0 + ec, N - 8);
    size_t off[NPASS];
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass)
      off[pass] = (size_t)min(m0 + pass * 16 + er, M - 1) * N + ncl;
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) a[pass][0] = a[pass][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const size_t sstep = (size_t)M * N;
    const float* ps = ep.split_ws;
    for (int s = 0; s < splits; ++s, ps += sstep) {
      f32x4 r[NPASS][2];
#pragma unroll
      for (int pass = 0; pass < NPASS; ++pass) {
        r[pass][0] = *reinterpret_cast<const f32x4*>(ps + off[pass]);
        r[pass][1] = *reinterpret_cast<const f32x4*>(ps + off[pass] + 4);
      }
#pragma unroll
      for (int pass = 0; pass < NPASS; ++pass) {
        a[pass][0] += r[pass][0];
        a[pass][1] += r[pass][1];
      }
    }
#pragma unroll
    for (int pass = 0; pass < HP; ++pass) {
      const int mm = pass * 16 + er;
      *reinterpret_cast<f32x4*>(Cs + mm * kCS + ec) = a[pass][0];
      *reinterpret_cast<f32x4*>(Cs + mm * kCS + ec + 4) = a[pass][1];
    }
  });
}

template <typename T, class G, int EPI>
hipError_t launch_epi(Dtype dt, const T* a, const T* w, int M, int N, int K, const GemmEpiArgs& ep,
                      hipStream_t st) {
  const int tiles = ((M + G::BM - 1) / G::BM) * ((N + G::BN - 1) / G::BN);
  const int S = ep.split_ws ? gemm_splits(dt, M, N, K) : 1;
  if (S == 1) {
    gemm_kernel<T, EPI, G, false><<<tiles, G::NT, 0, st>>>(a, w, M, N, K, 1, ep);
    return hipGetLastError();
  }
  gemm_kernel<T, EPI, G, true><<<tiles * S, G::NT, 0, st>>>(a, w, M, N, K, S, ep);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  splitk_reduce_kernel<T, EPI, G><<<tiles, G::NT, 0, st>>>(M, N, S, ep);
  return hipGetLastError();
}

// 64-element stages (128-byte rows), two stage buffers and one-piece epilogue staging:
// 68 KiB of LDS, two workgroups per CU (proj and fc2, whose residual epilogues hold more
// registers).  fp32 stages 32 elements (128-byte rows of 32-byte chunks) through registers.
template <typename T> struct TileMainSel;
template <> struct TileMainSel<bf16> { using type = Tile<bf16, 2, 2, 4, 4, 1, 8, 1, 2>; };
template <> struct TileMainSel<float> { using type = Tile<float, 2, 2, 4, 4, 1, 4, 1, 2>; };
template <typename T> using TileMain = typename TileMainSel<T>::type;
// QKV, fc1 and the patch embedding (bf16): one stage buffer and the epilogue staged in
// two halves: about 35 KiB of LDS and under 128 registers, so four workgroups share a CU
// and the others' matrix work covers one's loads and its (VALU-heavy) folded-LayerNorm /
// GELU epilogue.  Measured against two buffers at DeiT-S: QKV 8 %, fc1 10-13 % faster;
// fc2 25 % slower (its registers allow only two workgroups, which then wait on every
// load).  32-element stages with two buffers (also four workgroups) lost to the doubled
// barrier count.
template <typename T> struct TileWideSel { using type = typename TileMainSel<T>::type; };
template <> struct TileWideSel<bf16> { using type = Tile<bf16, 2, 2, 4, 4, 1, 8, 2, 1>; };
// ... when the launch has enough tiles for the extra workgroups per CU to matter (smaller
// launches wait on their single buffer with too few neighbours to cover it; the
// threshold was swept over 0 / 768 / 1536 on DeiT-S, UMT-B and UMT-L)
#ifndef RS_WIDE_MIN_TILES
#define RS_WIDE_MIN_TILES 768
#endif
inline bool wide_tiles(int M, int N) {
  return ((M + 127) / 128) * ((N + 127) / 128) >= RS_WIDE_MIN_TILES;
}

template <typename T, class G>
hipError_t launch_cfg(Dtype dt, GemmEpilogue epi, const void* A, const void* W, int M, int N, int K,
                      const GemmEpiArgs& ep, hipStream_t st) {
  const T* a = static_cast<const T*>(A);
  const T* w = static_cast<const T*>(W);
  switch (epi) {
    case kEpiQKV:
      return wide_tiles(M, N) ? launch_epi<T, typename TileWideSel<T>::type, kEpiQKV>(dt, a, w, M, N, K, ep, st)
                              : launch_epi<T, G, kEpiQKV>(dt, a, w, M, N, K, ep, st);
    case kEpiProj: return launch_epi<T, G, kEpiProj>(dt, a, w, M, N, K, ep, st);
    case kEpiGelu:
      return wide_tiles(M, N) ? launch_epi<T, typename TileWideSel<T>::type, kEpiGelu>(dt, a, w, M, N, K, ep, st)
                              : launch_epi<T, G, kEpiGelu>(dt, a, w, M, N, K, ep, st);
    case kEpiFc2: return launch_epi<T, G, kEpiFc2>(dt, a, w, M, N, K, ep, st);
    case kEpiPatch:
      return wide_tiles(M, N) ? launch_epi<T, typename TileWideSel<T>::type, kEpiPatch>(dt, a, w, M, N, K, ep, st)
                              : launch_epi<T, G, kEpiPatch>(dt, a, w, M, N, K, ep, st);
    case kEpiBias: return launch_epi<T, G, kEpiBias>(dt, a, w, M, N, K, ep, st);
  }
  return hipErrorInvalidValue;
}

// fc2 always runs with 2 waves of 64 columns across a 128-column tile, so the score
// partial count per row is 2 * ceil(C / 128) (see score_parts()).

}  // namespace

hipError_t launch_gemm(Dtype dt, GemmEpilogue epi, const void* A, const void* W, int M, int N,
                       int K, const GemmEpiArgs& ep, hipStream_t stream) {
  if (dt == kBF16) return launch_cfg<bf16, TileMain<bf16>>(dt, epi, A, W, M, N, K, ep, stream);
  return launch_cfg<float, TileMain<float>>(dt, epi, A, W, M, N, K, ep, stream);
}

}  // namespace rs
