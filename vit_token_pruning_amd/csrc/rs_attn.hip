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
//    output rows, double buffered; K rows padded by 16 bytes so the 16 rows of a K
//    fragment read fall on distinct banks, V rows by 32 bytes so the 8 rows x 32 bytes of
//    one half-wave transpose read do.  Keys past the sequence end are clamped to the
//    last row: finite values that meet probability 0.
//  - the V^T fragments of the P V product come from the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16): within each 16-lane group, lane j names 4 consecutive d of
//    key row base + j/4 and receives d0 + j of the 4 keys base .. base + 3.  fp32 reads
//    the 8 keys of a fragment one element at a time.
//  - exp2 with log2(e)/sqrt(d) folded into one FMA per score; the hardware exp2 is used
//    directly (results below 2^-126 flush to zero, which a softmax over at least one
//    term equal to 1 cannot notice).
#include "rs_device.hpp"
#include "rs_launch.hpp"

namespace rs {
namespace {

// The 8 k-slots of P^T for lane group g and 32-key chunk kc hold keys
// {32kc + 4g + v} (slots 0..3, from score tile 2kc) and {32kc + 16 + 4g + v} (slots 4..7,
// from score tile 2kc+1).  The V^T fragment below uses the same assignment.
__device__ __forceinline__ void pack_p(Frag8<bf16>& f, const f32x4& a, const f32x4& b) {
  f.v[0] = pack_bf16x2(a[0], a[1]);
  f.v[1] = pack_bf16x2(a[2], a[3]);
  f.v[2] = pack_bf16x2(b[0], b[1]);
  f.v[3] = pack_bf16x2(b[2], b[3]);
}
__device__ __forceinline__ void pack_p(Frag8<float>& f, const f32x4& a, const f32x4& b) {
  f.v[0] = __builtin_bit_cast(u32x4, a);
  f.v[1] = __builtin_bit_cast(u32x4, b);
}
// V^T fragment for d = d0 + l16 and the keys of lane group g in 32-key chunk kc (the
// slot assignment of pack_p): keys kb + 0..3 (slots 0-3) and kb + 16 .. kb + 19 (slots
// 4-7), kb = 32 kc + 4 g.  Vs rows are keys, ROWBV bytes apart.
template <int ROWBV>
__device__ __forceinline__ void load_vt(Frag8<bf16>& f, const char* Vs, int kb, int d0, int l16) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const char* pa = Vs + (kb + (l16 >> 2)) * ROWBV + (d0 + 4 * (l16 & 3)) * 2;
#if __HIP_DEVICE_COMPILE__
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pa));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pa + 16 * ROWBV));
#else
  const v4i16 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
#endif
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  f.v = u32x4{ua[0], ua[1], ub[0], ub[1]};
}
template <int ROWBV>
__device__ __forceinline__ void load_vt(Frag8<float>& f, const char* Vs, int kb, int d0, int l16) {
  float* e = reinterpret_cast<float*>(&f);
  const char* col = Vs + (d0 + l16) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = *reinterpret_cast<const float*>(col + (kb + i) * ROWBV);
    e[4 + i] = *reinterpret_cast<const float*>(col + (kb + 16 + i) * ROWBV);
  }
}
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
  constexpr int CB = Chunk<T>::bytes;  // 8 elements
  constexpr int ROWB = 8 * CB + 16;    // K rows: 64 elements + 16 bytes of padding
  constexpr int ROWBV = 8 * CB + 32;   // V rows: 64 elements + 32 bytes of padding
  constexpr int TBK = 64 * ROWB, TB = TBK + 64 * ROWBV;  // one K tile + one V tile
  __shared__ __attribute__((aligned(16))) char smem[2 * TB];

  const int C = H * 64, ldqkv = 3 * C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  // staging: 2 chunks of K rows and 2 chunks of V rows per thread per tile
  const int lc = tid & 7, lr = tid >> 3;
  const T* kbase = qkv + row0 * ldqkv + C + h * 64 + lc * 8;
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
  auto sstore = [&](int buf) {
    char* Ks = smem + buf * TB;
    char* Vs = Ks + TBK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = lr + 32 * i;
      store_frag(Ks + r * ROWB + lc * CB, rk[i]);
      store_frag(Vs + r * ROWBV + lc * CB, rv[i]);
    }
  };

  f32x4 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int nk = (L + 63) / 64;

  // A wave whose 16 queries all lie past the sequence end (in the last query block of a
  // ragged L) only helps stage K/V and meets the barriers.
  const bool active = q0 < L;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    const char* Ks = smem + (kt & 1) * TB;
    const char* Vs = Ks + TBK;
    if (active) {
      // S^T tile: s[j] lane (g, l16) = keys 16j + 4g + v of query l16
      f32x4 s[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int r = j * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int c = ks * 4 + g;
          Frag8<T> kf;
          load_frag(kf, Ks + r * ROWB + c * CB);
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
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      const float mb = m_new * scale_log2;
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[j][v], scale_log2, -mb));
          s[j][v] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] *= alpha;

      Frag8<T> pf[2];
      pack_p(pf[0], s[0], s[1]);
      pack_p(pf[1], s[2], s[3]);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          Frag8<T> vf;
          load_vt<ROWBV>(vf, Vs, 32 * kc + 4 * g, d * 16, l16);
          o[d] = mma16(o[d], vf, pf[kc]);
        }
      }
    }
    if (more) sstore((kt + 1) & 1);
    __syncthreads();
  }

  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  const float inv = 1.0f / lt;
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
