// Fused multi-head attention that never stores the attention map: Eq. (1) of
// "Representation Shift: Unifying Token Compression with FlashAttention" (arXiv HTML,
// Sec. 3.1), Softmax(Q K^T / sqrt(d)) V per head with d = 64, computed one 64-key
// block at a time with a running maximum and running denominator (the softmax
// rescaling identity; Sec. 1 explains why fused kernels such as FlashAttention are the
// setting the method targets: no L x L map is written to HBM).
//
// gfx950 mapping
//  - one workgroup = (sample, head, 64 queries); 4 waves, 16 queries each.
//  - the scores are computed transposed, S^T = K Q^T (keys on MFMA rows, queries on
//    columns), so each lane owns one query: its row max / row sum need no cross-lane
//    work inside a tile beyond the 4 lane groups, the rescale factor applies to the
//    lane's own output registers, and the probabilities are already in the register
//    layout the P V product wants as its B operand (no LDS round trip for P).
//  - K and V tiles [64 keys][64 d] are staged in LDS row-major, straight from the QKV
//    output rows, double buffered.  bf16: global -> LDS directly (16 bytes per lane, a
//    wave fills 8 whole 128-byte rows), one tile ahead of the math, with 16-byte chunk c
//    of row r at slot c ^ (r % 8) so the K fragment reads (16 rows, one chunk) and the
//    V transpose reads (8 rows x 32 bytes per half-wave) fall on distinct banks.  fp32
//    is staged through registers into padded rows.  Keys past the sequence end are
//    clamped to the last row: finite values that meet probability 0.
//  - the V^T fragments of the P V product come from the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16): within each 16-lane group, lane j names 4 consecutive d of
//    key row base + j/4 and receives d0 + j of the 4 keys base .. base + 3.  fp32 reads
//    the 8 keys of a fragment one element at a time.
//  - exp2 with log2(e)/sqrt(d) folded into one FMA per score; the hardware exp2 is used
//    directly (results below 2^-126 flush to zero, which a softmax over at least one
//    term equal to 1 cannot notice).  The running maximum is only moved when it grows
//    by more than 2^8 (probabilities stay below 2^8 meanwhile), which skips most
//    rescales of the output registers; row maxima and sums across the four lane rows
//    use the gfx950 row-swap instructions.
#include "rs_attn_frag.hpp"
#include "rs_device.hpp"
#include "rs_launch.hpp"

namespace rs {
namespace {

using namespace attn;

__device__ __forceinline__ void store_o4(bf16* p, const f32x4& o, float s) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(o[0] * s, o[1] * s), pack_bf16x2(o[2] * s, o[3] * s)};
}
__device__ __forceinline__ void store_o4(float* p, const f32x4& o, float s) {
  *reinterpret_cast<f32x4*>(p) = o * s;
}

template <typename T>
__global__ __launch_bounds__(256) void attention_kernel(const T* __restrict__ qkv,
                                                        T* __restrict__ out, int L, int H,
                                                        float scale_log2) {
  constexpr bool kDirect = sizeof(T) == 2;
  constexpr int CB = Chunk<T>::bytes;                  // 8 elements
  constexpr int ROWB = kDirect ? 128 : 8 * CB + 16;    // K rows (fp32: 16 bytes of padding)
  constexpr int ROWBV = kDirect ? 128 : 8 * CB + 32;   // V rows (fp32: 32 bytes of padding)
  // K and V tiles of the two buffers live in separate LDS arrays: each access below names
  // a fixed one, which lets the compiler see that the math on one buffer does not touch
  // the direct loads in flight into the other (it would otherwise wait for them)
  __shared__ __attribute__((aligned(1024))) char k0[64 * ROWB], k1[64 * ROWB];
  __shared__ __attribute__((aligned(1024))) char v0[64 * ROWBV], v1[64 * ROWBV];

  const int C = H * 64, ldqkv = 3 * C;
  // the wave index is uniform: keep it (and the LDS addresses derived from it) scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  // launch index -> (query block, head, sample), query blocks fastest; each XCD gets a
  // contiguous range so the query blocks of one head re-read its K/V from one L2
  const int nq = (L + 63) >> 6;
  const int t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int qb = t % nq, h = (t / nq) % H, b = t / (nq * H);
  const int q0 = qb * 64 + wave * 16;
  const size_t row0 = (size_t)b * L;

  // Q as the B operand: lane (g, l16) holds query q0+l16, d = 32ks + 8g .. +7
  Frag8<T> qf[2];
  {
    const int q = min(q0 + l16, L - 1);
    const T* qp = qkv + (row0 + q) * ldqkv + h * 64 + g * 8;
    load_frag(qf[0], qp);
    load_frag(qf[1], qp + 32);
  }

  // staging: thread (lr = tid / 8, lc = tid % 8) moves 16-byte chunks of K and V rows
  // lr and lr + 32.  bf16 direct: lane lc of a wave fills LDS slot lc of its row, so it
  // fetches global chunk lc ^ (row % 8); the wave's 1 KiB is rows 8 wave .. + 7 (+ 32).
  const int lc = tid & 7, lr = tid >> 3;
  const int gc = kDirect ? (lc ^ (lr & 7)) : lc;       // (lr + 32) % 8 == lr % 8
  const T* kbase = qkv + row0 * ldqkv + C + h * 64 + gc * 8;
  const T* vbase = kbase + C;
  Frag8<T> rk[2], rv[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(kt * 64 + lr + 32 * i, L - 1);
      load_frag(rk[i], kbase + (size_t)key * ldqkv);
      load_frag(rv[i], vbase + (size_t)key * ldqkv);
    }
  };
  auto sstore = [&](char* Ks, char* Vs) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = lr + 32 * i;
      store_frag(Ks + r * ROWB + lc * CB, rk[i]);
      store_frag(Vs + r * ROWBV + lc * CB, rv[i]);
    }
  };
  // this lane's K row of tile kt is kt * 64 rows past its row of tile 0, except that the
  // last tile of a ragged L clamps rows past the end
  const T* krow0[2] = {kbase + (size_t)lr * ldqkv, kbase + (size_t)(lr + 32) * ldqkv};
  auto dload = [&](int kt, char* Ks, char* Vs) {
    const size_t tstep = (size_t)kt * 64 * ldqkv;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const T* kp = krow0[i] + tstep;
      if (kt * 64 + 64 > L) kp = kbase + (size_t)min(kt * 64 + lr + 32 * i, L - 1) * ldqkv;
      load_lds16(kp, Ks + (wave * 8 + 32 * i) * 128);
      load_lds16(kp + C, Vs + (wave * 8 + 32 * i) * 128);
    }
  };
  auto kaddr = [&](const char* Ks, int r, int c) {
    return kDirect ? Ks + r * 128 + ((c ^ (r & 7)) << 4) : Ks + r * ROWB + c * CB;
  };

  f32x4 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int nk = (L + 63) / 64;

  // A wave whose 16 queries all lie past the sequence end (in the last query block of a
  // ragged L) only helps stage K/V and meets the barriers.
  const bool active = q0 < L;

  // The math of one key tile from LDS buffers Ks, Vs.
  auto tile = [&](int kt, const char* Ks, const char* Vs) {
    // S^T tile: s[j] lane (g, l16) = keys 16j + 4g + v of query l16
    f32x4 s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = j * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Frag8<T> kf;
        load_frag(kf, kaddr(Ks, r, ks * 4 + g));
        s[j] = mma16(s[j], kf, qf[ks]);
      }
    }
    if (kt * 64 + 64 > L) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (kt * 64 + j * 16 + 4 * g + v >= L) s[j][v] = -INFINITY;
    }
    float mx = s[0][0];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[j][v]);
    mx = max_rows(mx);
    // The running maximum moves (and the output and denominator are rescaled) only when
    // some lane's maximum grew by more than 8 in the exp2 domain: until then the stale
    // maximum keeps every probability below 2^8, and numerator and denominator share it.
    const float m_new = fmaxf(m_run, mx);
    if (__builtin_amdgcn_ballot_w64((m_new - m_run) * scale_log2 > 8.0f)) {
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] *= alpha;
      m_run = m_new;
    }
    const float mb = m_run * scale_log2;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[j][v], scale_log2, -mb));
        s[j][v] = p;
        psum += p;
      }
    l_run += psum;

    Frag8<T> pf[2];
    pack_p(pf[0], s[0], s[1]);
    pack_p(pf[1], s[2], s[3]);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        Frag8<T> vf;
        if constexpr (kDirect) load_vt(vf, Vs, 32 * kc + 4 * g, d * 16, l16);
        else load_vt_f32<ROWBV>(vf, Vs, 32 * kc + 4 * g, d * 16, l16);
        o[d] = mma16(o[d], vf, pf[kc]);
      }
    }
  };

  if constexpr (kDirect) {
    // the loads of tile kt + 1 go out right after the barrier that frees their buffer;
    // two tiles per trip so that every access names its buffer statically
    auto step = [&](int kt, char* kc, char* vc, char* kn, char* vn) {
      wait_vmem<0>();          // this wave's part of tile kt (and Q) has landed
      barrier_nofence();       // ... and every wave's; tile kt - 1's reads are done
      if (kt + 1 < nk) dload(kt + 1, kn, vn);
      if (active) tile(kt, kc, vc);
    };
    dload(0, k0, v0);
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, k0, v0, k1, v1);
      step(kt + 1, k1, v1, k0, v0);
    }
    if (kt < nk) step(kt, k0, v0, k1, v1);
  } else {
    gload(0);
    sstore(k0, v0);
    __syncthreads();
    int kt = 0;
    auto step = [&](int kt, const char* kc, const char* vc, char* kn, char* vn) {
      const bool more = kt + 1 < nk;
      if (more) gload(kt + 1);
      if (active) tile(kt, kc, vc);
      if (more) sstore(kn, vn);
      __syncthreads();
    };
    for (; kt + 1 < nk; kt += 2) {
      step(kt, k0, v0, k1, v1);
      step(kt + 1, k1, v1, k0, v0);
    }
    if (kt < nk) step(kt, k0, v0, k1, v1);
  }

  const float inv = 1.0f / sum_rows(l_run);
  const int q = q0 + l16;
  if (q < L) {
    T* op = out + (row0 + q) * C + h * 64 + 4 * g;
#pragma unroll
    for (int d = 0; d < 4; ++d) store_o4(op + d * 16, o[d], inv);
  }
}

}  // namespace

hipError_t launch_attention(Dtype dt, const void* qkv, void* out, int B, int L, int H,
                            hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
  const int grid = ((L + 63) / 64) * H * B;
  if (dt == kBF16)
    attention_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(qkv),
                                                     static_cast<bf16*>(out), L, H, scale_log2);
  else
    attention_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(qkv),
                                                      static_cast<float*>(out), L, H, scale_log2);
  return hipGetLastError();
}

}  // namespace rs
