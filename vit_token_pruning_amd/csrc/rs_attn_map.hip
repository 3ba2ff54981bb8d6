// Attention that forms the attention map, for the attention-map importance scores the
// method is compared against: Eq. (2) (the class token's attention row) and Eq. (3) (the
// mean of the attention rows over all queries) of "Representation Shift: Unifying Token
// Compression with FlashAttention" (arXiv HTML, Sec. 3.1).  Those scores need the
// normalised map A = Softmax(Q K^T / sqrt(d)), which a fused kernel never has; this
// kernel produces it, and optionally stores it to HBM as a non-fused attention does.
//
// One workgroup = (sample, head, 64 queries), 4 waves of 16 queries, the layout of the
// fused kernel (S^T = K Q^T, one query per lane).  Two passes over the keys: the first
// finds each query's row maximum and denominator; the second recomputes the scores, forms
// the final probabilities P = exp(s - m) / l, accumulates O = P V (no rescaling), and
//  - stores P to the map [B][H][L][Lpad] (bf16 or fp32 like the activations; rows padded
//    to a multiple of 8 keys, padding keys hold 0), if requested;
//  - writes query 0's row (fp32) to cls [B][H][L], if requested (Eq. (2));
//  - writes the workgroup's column sums of P over its queries to colsum [B][H][nq][L]
//    (fp32, nq = ceil(L / 64)), if requested (Eq. (3)): per key tile each wave sums its
//    16 queries across lanes, and the four waves' sums are added in a fixed order through
//    LDS one tile later.
// K and V tiles are staged as in the fused kernel (bf16: direct global -> LDS loads into
// swizzled 128-byte rows, V read with LDS transpose reads; fp32: registers and padded
// rows).
#include "rs_attn_frag.hpp"
#include "rs_device.hpp"
#include "rs_launch.hpp"

namespace rs {
namespace {

using namespace attn;

__device__ __forceinline__ void store_p4(bf16* p, const f32x4& v) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void store_p4(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ void store_o4(bf16* p, const f32x4& o) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
}
__device__ __forceinline__ void store_o4(float* p, const f32x4& o) {
  *reinterpret_cast<f32x4*>(p) = o;
}

template <typename T>
__global__ __launch_bounds__(256) void attention_map_kernel(
    const T* __restrict__ qkv, T* __restrict__ out, int L, int H, float scale_log2,
    T* __restrict__ map, int Lpad, float* __restrict__ cls, float* __restrict__ colsum) {
  constexpr bool kDirect = sizeof(T) == 2;
  constexpr int CB = Chunk<T>::bytes;
  constexpr int ROWB = kDirect ? 128 : 8 * CB + 16;
  constexpr int ROWBV = kDirect ? 128 : 8 * CB + 32;
  __shared__ __attribute__((aligned(1024))) char k0[64 * ROWB], k1[64 * ROWB];
  __shared__ __attribute__((aligned(1024))) char v0[64 * ROWBV], v1[64 * ROWBV];
  __shared__ float cacc[2][4][64];     // per-wave column sums of the last two key tiles

  const int C = H * 64, ldqkv = 3 * C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int nq = (L + 63) >> 6;
  const int t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int qb = t % nq, h = (t / nq) % H, b = t / (nq * H);
  const int q0 = qb * 64 + wave * 16;
  const int q = q0 + l16;
  const size_t row0 = (size_t)b * L, bh = (size_t)b * H + h;

  Frag8<T> qf[2];
  {
    const T* qp = qkv + (row0 + min(q, L - 1)) * ldqkv + h * 64 + g * 8;
    load_frag(qf[0], qp);
    load_frag(qf[1], qp + 32);
  }

  const int lc = tid & 7, lr = tid >> 3;
  const int gc = kDirect ? (lc ^ (lr & 7)) : lc;
  const T* kbase = qkv + row0 * ldqkv + C + h * 64 + gc * 8;
  const T* vbase = kbase + C;
  Frag8<T> rk[2], rv[2];
  auto gload = [&](int kt, bool with_v) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(kt * 64 + lr + 32 * i, L - 1);
      load_frag(rk[i], kbase + (size_t)key * ldqkv);
      if (with_v) load_frag(rv[i], vbase + (size_t)key * ldqkv);
    }
  };
  auto sstore = [&](char* Ks, char* Vs, bool with_v) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = lr + 32 * i;
      store_frag(Ks + r * ROWB + lc * CB, rk[i]);
      if (with_v) store_frag(Vs + r * ROWBV + lc * CB, rv[i]);
    }
  };
  auto dload = [&](int kt, char* Ks, char* Vs, bool with_v) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(kt * 64 + lr + 32 * i, L - 1);
      load_lds16(kbase + (size_t)key * ldqkv, Ks + (wave * 8 + 32 * i) * 128);
      if (with_v) load_lds16(vbase + (size_t)key * ldqkv, Vs + (wave * 8 + 32 * i) * 128);
    }
  };
  auto kaddr = [&](const char* Ks, int r, int c) {
    return kDirect ? Ks + r * 128 + ((c ^ (r & 7)) << 4) : Ks + r * ROWB + c * CB;
  };
  // S^T tile: s[j] lane (g, l16) = keys kt*64 + 16j + 4g + v of query l16; keys past the
  // end get -inf
  auto scores = [&](int kt, const char* Ks, f32x4 (&s)[4]) {
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
  };

  const int nk = (L + 63) / 64;
  const bool active = q0 < L;
  // Runs body(kt, Ks, Vs) over all key tiles with the tiles staged in the two LDS buffers
  // (K only when with_v is false); `flush(kt)` runs after the barrier that opens tile kt.
  auto sweep = [&](bool with_v, auto&& body, auto&& flush) {
    if constexpr (kDirect) {
      auto step = [&](int kt, char* kc, char* vc, char* kn, char* vn) {
        // this wave's loads of tile kt, its stores, and its LDS writes of cacc are done
        __builtin_amdgcn_s_waitcnt(0);
        barrier_nofence();
        flush(kt);
        if (kt + 1 < nk) dload(kt + 1, kn, vn, with_v);
        if (active) body(kt, kc, vc);
      };
      dload(0, k0, v0, with_v);
      int kt = 0;
      for (; kt + 1 < nk; kt += 2) {
        step(kt, k0, v0, k1, v1);
        step(kt + 1, k1, v1, k0, v0);
      }
      if (kt < nk) step(kt, k0, v0, k1, v1);
    } else {
      gload(0, with_v);
      sstore(k0, v0, with_v);
      __syncthreads();
      auto step = [&](int kt, const char* kc, const char* vc, char* kn, char* vn) {
        flush(kt);
        const bool more = kt + 1 < nk;
        if (more) gload(kt + 1, with_v);
        if (active) body(kt, kc, vc);
        if (more) sstore(kn, vn, with_v);
        __syncthreads();
      };
      int kt = 0;
      for (; kt + 1 < nk; kt += 2) {
        step(kt, k0, v0, k1, v1);
        step(kt + 1, k1, v1, k0, v0);
      }
      if (kt < nk) step(kt, k0, v0, k1, v1);
    }
    __syncthreads();   // every wave is done with both buffers (and with cacc's writes)
  };

  // ---- pass 1: row maximum and denominator
  float m_run = -INFINITY, l_run = 0.f;
  sweep(false, [&](int kt, const char* Ks, const char*) {
    f32x4 s[4];
    scores(kt, Ks, s);
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
      for (int v = 0; v < 4; ++v) psum += __builtin_amdgcn_exp2f(fmaf(s[j][v], scale_log2, -mb));
    l_run = l_run * alpha + psum;
    m_run = m_new;
  }, [](int) {});
  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  const float inv = 1.0f / lt, mb = m_run * scale_log2;
  const float qmask = q < L ? 1.0f : 0.0f;    // queries past the end add nothing

  // ---- pass 2: probabilities, the map, the scores' partial sums, O = P V
  f32x4 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  T* mrow = map ? map + (bh * L + min(q, L - 1)) * (size_t)Lpad : nullptr;
  float* csum = colsum ? colsum + (bh * nq + qb) * (size_t)L : nullptr;
  // column sums of tile kt - 1 (written to cacc[(kt - 1) & 1] by every active wave) are
  // added over the waves in wave order by threads 0..63 after the barrier opening tile kt
  auto flush = [&](int kt) {
    if (!csum || kt == 0 || tid >= 64) return;
    const int key = (kt - 1) * 64 + tid;
    if (key >= L) return;
    const float* c = &cacc[(kt - 1) & 1][0][0];
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (qb * 64 + w * 16 < L) sum += c[w * 64 + tid];
    csum[key] = sum;
  };
  sweep(true, [&](int kt, const char* Ks, const char* Vs) {
    f32x4 s[4];
    scores(kt, Ks, s);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        s[j][v] = __builtin_amdgcn_exp2f(fmaf(s[j][v], scale_log2, -mb)) * inv;
    if (mrow && q < L) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kg = kt * 64 + j * 16 + 4 * g;
        if (kg < Lpad) store_p4(mrow + kg, s[j]);
      }
    }
    if (cls && q == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = kt * 64 + j * 16 + 4 * g + v;
          if (key < L) cls[bh * L + key] = s[j][v];
        }
    }
    if (csum) {
      // sum over this wave's 16 queries (the 16 lanes of each lane group)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float c = s[j][v] * qmask;
          c += __shfl_xor(c, 1, 64);
          c += __shfl_xor(c, 2, 64);
          c += __shfl_xor(c, 4, 64);
          c += __shfl_xor(c, 8, 64);
          if (l16 == 0) cacc[kt & 1][wave][j * 16 + 4 * g + v] = c;
        }
    }
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
  }, flush);
  flush(nk);   // the last tile's column sums (sweep ended with a barrier)

  if (q < L) {
    T* op = out + (row0 + q) * C + h * 64 + 4 * g;
#pragma unroll
    for (int d = 0; d < 4; ++d) store_o4(op + d * 16, o[d]);
  }
}

// Eq. (2) / Eq. (3) averaged over heads: one thread per (sample, key).
//   mode 0: s = (1/H) sum_h cls[b][h][key]
//   mode 1: s = (1/(H L)) sum_h sum_qb colsum[b][h][qb][key]
__global__ __launch_bounds__(256) void map_score_kernel(const float* __restrict__ cls,
                                                        const float* __restrict__ colsum,
                                                        int B, int L, int H, int mode,
                                                        float* __restrict__ scores) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)B * L) return;
  const int b = (int)(i / L), key = (int)(i - (long long)b * L);
  const int nq = (L + 63) >> 6;
  float s = 0.f;
  if (mode == 0) {
    for (int h = 0; h < H; ++h) s += cls[((size_t)b * H + h) * L + key];
    s *= 1.0f / (float)H;
  } else {
    for (int h = 0; h < H; ++h) {
      float sh = 0.f;
      for (int qb = 0; qb < nq; ++qb) sh += colsum[(((size_t)b * H + h) * nq + qb) * L + key];
      s += sh;
    }
    s *= 1.0f / ((float)H * (float)L);
  }
  scores[i] = s;
}

}  // namespace

hipError_t launch_attention_map(Dtype dt, const void* qkv, void* out, int B, int L, int H,
                                void* map, int Lpad, float* cls, float* colsum,
                                hipStream_t stream) {
  const float scale_log2 = 1.4426950408889634f / 8.0f;  // log2(e) / sqrt(64)
  const int grid = ((L + 63) / 64) * H * B;
  if (dt == kBF16)
    attention_map_kernel<bf16><<<grid, 256, 0, stream>>>(
        static_cast<const bf16*>(qkv), static_cast<bf16*>(out), L, H, scale_log2,
        static_cast<bf16*>(map), Lpad, cls, colsum);
  else
    attention_map_kernel<float><<<grid, 256, 0, stream>>>(
        static_cast<const float*>(qkv), static_cast<float*>(out), L, H, scale_log2,
        static_cast<float*>(map), Lpad, cls, colsum);
  return hipGetLastError();
}

hipError_t launch_map_scores(const float* cls, const float* colsum, int B, int L, int H, int mode,
                             float* scores, hipStream_t stream) {
  const long long n = (long long)B * L;
  map_score_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(cls, colsum, B, L, H, mode,
                                                                   scores);
  return hipGetLastError();
}

}  // namespace rs
