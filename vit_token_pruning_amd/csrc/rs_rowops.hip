// Row-wise and selection kernels: LayerNorm, the standalone representation-shift score,
// the per-sample exact top-k, and the compaction of kept rows.
//
// Method: "Representation Shift: Unifying Token Compression with FlashAttention" (arXiv
// HTML).  LayerNorm is the LN of Sec. 3.3, Eqs. (5) and (6); the score is Eq. (4) with
// the L2 distance (Sec. 3.2); selection drops the lowest-scoring tokens, the same
// count in every sample, yielding the reduced set x~ of Sec. 3.1.
#include "rs_device.hpp"
#include "rs_launch.hpp"
#include "../../include/rs.h"

namespace rs {
namespace {

// ---------------------------------------------------------------- LayerNorm
// One wave per row; each lane holds up to two 8-element chunks (C <= 1024).
// Statistics in fp32: mean, then the biased variance around it.
template <typename T>
__global__ __launch_bounds__(256) void layernorm_kernel(const T* __restrict__ x,
                                                        const T* __restrict__ p,
                                                        const T* __restrict__ gam,
                                                        const T* __restrict__ bet, float eps,
                                                        T* __restrict__ out, int M, int C) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;  // whole wave
  const int nch = C >> 3;
  const size_t base = (size_t)row * C;
  float v[2][8];
  float s = 0.f;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int ch = lane + it * 64;
    if (ch < nch) {
      load8f(x + base + ch * 8, v[it]);
      if (p) {
        float q[8];
        load8f(p + base + ch * 8, q);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[it][e] += q[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[it][e];
    }
  }
  const float mean = wave_sum(s) / (float)C;
  float s2 = 0.f;
#pragma unroll
  for (int it = 0; it < 2; ++it)
    if (lane + it * 64 < nch)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[it][e] - mean;
        s2 += d * d;
      }
  const float rstd = 1.0f / sqrtf(wave_sum(s2) / (float)C + eps);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int ch = lane + it * 64;
    if (ch < nch) {
      float gg[8], bb[8], o[8];
      load8f(gam + ch * 8, gg);
      load8f(bet + ch * 8, bb);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[it][e] - mean) * rstd * gg[e] + bb[e];
      store8f(out + base + ch * 8, o);
    }
  }
}

// ---------------------------------------------------------------- standalone score
// 16 lanes per row: || fx - x ||_2 accumulated in fp32.
template <typename T>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ fx,
                                                    const T* __restrict__ x,
                                                    float* __restrict__ s, int M, int C) {
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4), sub = threadIdx.x & 15;
  float acc = 0.f;
  if (row < M) {
    const size_t base = (size_t)row * C;
    for (int ch = sub; ch < (C >> 3); ch += 16) {
      float a[8], b[8];
      load8f(fx + base + ch * 8, a);
      load8f(x + base + ch * 8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = a[e] - b[e];
        acc += d * d;
      }
    }
  }
  acc = sum16(acc);
  if (sub == 0 && row < M) s[row] = sqrtf(acc);
}

// ---------------------------------------------------------------- top-k
// Keys: fp32 scores mapped to uint32 so that unsigned order is score order; -0 and +0
// share a key; every NaN maps to 0 (below every number); the class token gets the
// all-ones key (above +Inf).
__device__ __forceinline__ uint32_t order_key(float s) {
  if (s != s) return 0u;
  uint32_t u = __float_as_uint(s);
  if (s == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;

// exclusive prefix sum over the 1024 threads of the workgroup
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();
  return before + incl - v;
}

// One workgroup per sample.  Exact k-th largest key by a 4-pass 8-bit radix select
// (MSB first) over an LDS histogram, then every key above it plus the lowest-index keys
// equal to it, emitted in ascending index order.  Integer work only: deterministic.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float* __restrict__ scores, const float* __restrict__ part, int P, int L, int k,
    int has_cls, float* __restrict__ scores_out, int32_t* __restrict__ kept,
    const int32_t* __restrict__ ids_in, int32_t* __restrict__ ids_out) {
  __shared__ uint32_t keys[RS_MAX_TOKENS];
  __shared__ uint32_t hist[256];
  __shared__ int wsum[kTopkThreads / 64];
  __shared__ uint32_t sel[2];
  const int b = blockIdx.x, tid = threadIdx.x;
  const size_t rb = (size_t)b * L;

  for (int i = tid; i < L; i += kTopkThreads) {
    float s;
    if (part) {
      const float* pp = part + (rb + i) * P;
      float a = 0.f;
      for (int q = 0; q < P; ++q) a += pp[q];
      s = sqrtf(a);
    } else {
      s = scores[rb + i];
    }
    if (scores_out) scores_out[rb + i] = s;
    keys[i] = (has_cls && i == 0) ? 0xFFFFFFFFu : order_key(s);
  }
  __syncthreads();

  uint32_t prefix = 0u, pmask = 0u;
  uint32_t krem = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < L; i += kTopkThreads) {
      const uint32_t key = keys[i];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane covers bins 255-4*tid down to 252-4*tid; counts above run high -> low
      uint32_t c[4], loc = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * tid - q];
        loc += c[q];
      }
      uint32_t incl = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, 64);
        if (tid >= o) incl += t;
      }
      uint32_t above = incl - loc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < krem && above + c[q] >= krem) {
          sel[0] = (uint32_t)(255 - 4 * tid - q);
          sel[1] = above;
        }
        above += c[q];
      }
    }
    __syncthreads();
    prefix |= sel[0] << shift;
    pmask |= 0xFFu << shift;
    krem -= sel[1];
    __syncthreads();
  }
  const uint32_t T = prefix;  // the k-th largest key; krem of its copies are kept

  const int seg = (L + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(tid * seg, L), i1 = min(i0 + seg, L);
  int eq = 0;
  for (int i = i0; i < i1; ++i) eq += keys[i] == T;
  const int eq_before = block_exclusive_scan(eq, wsum);
  int cnt = 0, e = eq_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    const bool keep = key > T || (key == T && (uint32_t)e < krem);
    e += key == T;
    cnt += keep;
  }
  int pos = block_exclusive_scan(cnt, wsum);
  e = eq_before;
  int32_t* kb = kept + (size_t)b * k;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = keys[i];
    const bool keep = key > T || (key == T && (uint32_t)e < krem);
    e += key == T;
    if (keep && pos < k) {
      kb[pos] = i;
      if (ids_out) ids_out[(size_t)b * k + pos] = ids_in ? ids_in[rb + i] : i;
      ++pos;
    }
  }
}

// ---------------------------------------------------------------- gather
// One 16-byte unit per thread, grid-stride; consecutive threads copy consecutive
// units of one kept row.
__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ x,
                                                     const int32_t* __restrict__ kept,
                                                     char* __restrict__ out, int L, int k,
                                                     int units_per_row, long long total) {
  for (long long u = (long long)blockIdx.x * 256 + threadIdx.x; u < total;
       u += (long long)gridDim.x * 256) {
    const long long row = u / units_per_row;
    const int c = (int)(u - row * units_per_row);
    const long long b = row / k;
    const long long src = b * L + kept[row];
    reinterpret_cast<u32x4*>(out)[u] =
        reinterpret_cast<const u32x4*>(x + src * (long long)units_per_row * 16)[c];
  }
}

__global__ void iota_kernel(int32_t* ids, int L, long long total) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (long long)gridDim.x * 256)
    ids[i] = (int32_t)(i % L);
}

int grid_for(long long units) {
  long long g = (units + 255) / 256;
  if (g > 16384) g = 16384;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

hipError_t launch_layernorm(Dtype dt, const void* x, const void* p, const void* g, const void* b,
                            float eps, void* out, int M, int C, hipStream_t stream) {
  const int grid = (M + 3) / 4;
  if (dt == kBF16)
    layernorm_kernel<bf16><<<grid, 256, 0, stream>>>(
        static_cast<const bf16*>(x), static_cast<const bf16*>(p), static_cast<const bf16*>(g),
        static_cast<const bf16*>(b), eps, static_cast<bf16*>(out), M, C);
  else
    layernorm_kernel<float><<<grid, 256, 0, stream>>>(
        static_cast<const float*>(x), static_cast<const float*>(p), static_cast<const float*>(g),
        static_cast<const float*>(b), eps, static_cast<float*>(out), M, C);
  return hipGetLastError();
}

hipError_t launch_score_rows(Dtype dt, const void* fx, const void* x, float* scores, int M, int C,
                             hipStream_t stream) {
  const int grid = (M + 15) / 16;
  if (dt == kBF16)
    score_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(fx),
                                                 static_cast<const bf16*>(x), scores, M, C);
  else
    score_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(fx),
                                                  static_cast<const float*>(x), scores, M, C);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, const float* part, int P, int B, int L, int k,
                       int has_cls, float* scores_out, int32_t* kept, const int32_t* ids_in,
                       int32_t* ids_out, hipStream_t stream) {
  topk_kernel<<<B, kTopkThreads, 0, stream>>>(scores, part, P, L, k, has_cls, scores_out, kept,
                                              ids_in, ids_out);
  return hipGetLastError();
}

hipError_t launch_gather(const void* x, const int32_t* kept, void* out, int B, int L, int k,
                         int row_bytes, hipStream_t stream) {
  const int upr = row_bytes / 16;
  const long long total = (long long)B * k * upr;
  gather_kernel<<<grid_for(total), 256, 0, stream>>>(static_cast<const char*>(x), kept,
                                                     static_cast<char*>(out), L, k, upr, total);
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* ids, int B, int L, hipStream_t stream) {
  const long long total = (long long)B * L;
  iota_kernel<<<grid_for(total), 256, 0, stream>>>(ids, L, total);
  return hipGetLastError();
}

}  // namespace rs
