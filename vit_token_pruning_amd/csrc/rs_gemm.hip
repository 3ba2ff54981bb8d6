// Tile GEMM Y = A W^T on the gfx950 matrix cores with the block's fused epilogues:
// QKV (bias, per-head transposed V), attention projection (bias), fc1 (bias + exact
// GELU) and fc2 (bias, residual re-formed in fp32, and the per-token partial sums of
// squares of the MLP-sublayer representation shift).
//
// The score is Eq. (4) of "Representation Shift: Unifying Token Compression with
// FlashAttention" (arXiv HTML), Sec. 3.2, for the MLP sublayer of Sec. 3.3 (case ii)
// and the L2 distance: || MLP(LN(x')) - x' ||_2.  The fc2 accumulators already hold
// MLP(LN(x')) - b2 in fp32, so the squared difference is summed while the tile is in
// registers/LDS and the MLP output is never re-read from HBM.
//
// Layout: A [M][K] (activations), W [N][K] (Linear weight, [out][in]); both are
// K-contiguous.  Workgroup tile 128 (M) x 128 (N), 4 waves in 2 x 2, each 64 x 64 as
// 4 x 4 MFMA 16x16x32 tiles.  K advances 64 (bf16) or 32 (fp32) per LDS stage, double
// buffered: the next stage's global loads are in flight while the current one is
// multiplied.  LDS rows hold 8 chunks of 8 elements; chunk c of row r sits at slot
// c ^ (r % chunks) so the 16 rows a fragment read touches land on distinct banks.
#include "rs_device.hpp"
#include "rs_launch.hpp"

namespace rs {
namespace {

constexpr int BM = kGemmTile, BN = kGemmTile;
constexpr int CS = BN + 4;  // fp32 row stride of the staged output tile

template <typename T> struct GemmShape {
  static constexpr int KC = sizeof(T) == 2 ? 8 : 4;  // chunks per row per stage
  static constexpr int CB = Chunk<T>::bytes;           // chunk bytes
  static constexpr int ROWB = KC * CB;                 // 128 bytes per tile row
  static constexpr int OPB = BM * ROWB;                // one operand tile: 16 KB
  static constexpr int SMEM = (4 * OPB > BM * CS * 4) ? 4 * OPB : BM * CS * 4;
};

template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const T* __restrict__ A,
                                                      const T* __restrict__ W, int M, int N,
                                                      int K, GemmEpiArgs ep) {
  using S = GemmShape<T>;
  constexpr int KC = S::KC, CB = S::CB, ROWB = S::ROWB, OPB = S::OPB;
  __shared__ __attribute__((aligned(16))) char smem[S::SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN;
  const int t = xcd_contiguous(blockIdx.x, nM * nN);
  const int mt = t / nN, nt = t - mt * nN;
  const int m0 = mt * BM, n0 = nt * BN;
  const int wm = wave & 1, wn = wave >> 1;

  // ---- global -> LDS staging: each thread moves NL chunks of A and of W per stage
  constexpr int NL = KC / 2;
  constexpr int RSTEP = 256 / KC;
  const int lc = tid % KC, lr = tid / KC;
  const char* ag[NL];
  const char* wg[NL];
  int so[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int r = lr + i * RSTEP;
    const int am = min(m0 + r, M - 1), wn_ = min(n0 + r, N - 1);
    ag[i] = reinterpret_cast<const char*>(A + (size_t)am * K) + lc * CB;
    wg[i] = reinterpret_cast<const char*>(W + (size_t)wn_ * K) + lc * CB;
    so[i] = r * ROWB + ((lc ^ (r % KC)) * CB);
  }
  Frag8<T> ra[NL], rw[NL];
  const int KT = K / (8 * KC);

  f32x4 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < NL; ++i) {
    load_frag(ra[i], ag[i]);
    load_frag(rw[i], wg[i]);
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    store_frag(smem + so[i], ra[i]);
    store_frag(smem + OPB + so[i], rw[i]);
  }
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) {
      const size_t off = (size_t)(kt + 1) * ROWB;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        load_frag(ra[i], ag[i] + off);
        load_frag(rw[i], wg[i] + off);
      }
    }
    const char* As = smem + (kt & 1) * 2 * OPB;
    const char* Ws = As + OPB;
#pragma unroll
    for (int ks = 0; ks < KC / 4; ++ks) {
      const int c = ks * 4 + g;
      Frag8<T> fa[4], fw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + l16;
        load_frag(fa[i], As + r * ROWB + ((c ^ (r % KC)) * CB));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + l16;
        load_frag(fw[j], Ws + r * ROWB + ((c ^ (r % KC)) * CB));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = mma16(acc[j][i], fw[j], fa[i]);
    }
    if (more) {
      char* Ad = smem + ((kt + 1) & 1) * 2 * OPB;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        store_frag(Ad + so[i], ra[i]);
        store_frag(Ad + OPB + so[i], rw[i]);
      }
    }
    __syncthreads();
  }

  // ---- stage the fp32 tile in LDS as Cs[m][n] (acc[j][i] holds rows n, column m)
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 64 + i * 16 + l16, n = wn * 64 + j * 16 + 4 * g;
      *reinterpret_cast<f32x4*>(Cs + m * CS + n) = acc[j][i];
    }
  __syncthreads();

  const T* bias = static_cast<const T*>(ep.bias);
  if (EPI == kEpiQKV && n0 >= ep.vcol0) {
    // V columns: write V^T per head, [b][h][d][token]; lanes run along tokens so
    // each store instruction covers consecutive tokens of one (head, d) row.
    T* vt = static_cast<T*>(ep.vt);
    const int m = tid & 127, half = tid >> 7;
    const int gm = m0 + m;
    if (gm < M) {
      const int bb = gm / ep.L, tk = gm - bb * ep.L;
      for (int jj = 0; jj < 64; ++jj) {
        const int n = half * 64 + jj, gn = n0 + n;
        if (gn < N) {
          const int vc = gn - ep.vcol0, h = vc >> 6, d = vc & 63;
          const float v = Cs[m * CS + n] + to_f32(bias[gn]);
          vt[((size_t)(bb * ep.heads + h) * 64 + d) * ep.Lp + tk] = from_f32<T>(v);
        }
      }
    }
    return;
  }

  // ---- row pass: 16 threads per row, 8 consecutive columns each
  const int er = tid >> 4, ec = (tid & 15) * 8;
  const int gn = n0 + ec;
  const bool col_ok = gn < N;
  float b8[8];
  if (col_ok) load8f(bias + gn, b8);
  T* out = static_cast<T*>(ep.out);
#pragma unroll 1
  for (int pass = 0; pass < BM / 16; ++pass) {
    const int m = pass * 16 + er, gm = m0 + m;
    const bool ok = col_ok && gm < M;
    float v[8];
    {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(Cs + m * CS + ec);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(Cs + m * CS + ec + 4);
      v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
      v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
    }
    if (EPI == kEpiFc2) {
      float ss = 0.f;
      if (ok) {
        float xv[8], pv[8];
        load8f(static_cast<const T*>(ep.x) + (size_t)gm * N + gn, xv);
        load8f(static_cast<const T*>(ep.p) + (size_t)gm * N + gn, pv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = v[e] + b8[e];        // MLP(LN(x'))
          const float xp = xv[e] + pv[e];      // x' (Eq. 5), fp32
          const float d = y - xp;
          ss += d * d;
          v[e] = xp + y;                       // x_hat (Eq. 6)
        }
        store8f(out + (size_t)gm * ep.ldo + gn, v);
      }
      if (ep.part) {
        ss = sum16(ss);
        if ((tid & 15) == 0 && gm < M) ep.part[(size_t)gm * ep.nparts + nt] = ss;
      }
    } else if (ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] += b8[e];
        if (EPI == kEpiGelu) v[e] = gelu_erf(v[e]);
      }
      store8f(out + (size_t)gm * ep.ldo + gn, v);
    }
  }
}

template <typename T>
hipError_t launch_t(GemmEpilogue epi, const void* A, const void* W, int M, int N, int K,
                    const GemmEpiArgs& ep, hipStream_t st) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const T* a = static_cast<const T*>(A);
  const T* w = static_cast<const T*>(W);
  switch (epi) {
    case kEpiQKV: gemm_nt_kernel<T, kEpiQKV><<<tiles, 256, 0, st>>>(a, w, M, N, K, ep); break;
    case kEpiBias: gemm_nt_kernel<T, kEpiBias><<<tiles, 256, 0, st>>>(a, w, M, N, K, ep); break;
    case kEpiGelu: gemm_nt_kernel<T, kEpiGelu><<<tiles, 256, 0, st>>>(a, w, M, N, K, ep); break;
    case kEpiFc2: gemm_nt_kernel<T, kEpiFc2><<<tiles, 256, 0, st>>>(a, w, M, N, K, ep); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(Dtype dt, GemmEpilogue epi, const void* A, const void* W, int M, int N,
                       int K, const GemmEpiArgs& ep, hipStream_t stream) {
  return dt == kBF16 ? launch_t<bf16>(epi, A, W, M, N, K, ep, stream)
                     : launch_t<float>(epi, A, W, M, N, K, ep, stream);
}

}  // namespace rs
