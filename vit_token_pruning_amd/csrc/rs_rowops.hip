// Row-wise and selection kernels: LayerNorm preparation (row statistics, folded weights),
// the standalone representation-shift score, and the per-sample exact top-k with the
// compaction of the kept rows.
//
// Method: "Representation Shift: Unifying Token Compression with FlashAttention" (arXiv
// HTML).  LayerNorm is the LN of Sec. 3.3, Eqs. (5) and (6); the score is Eq. (4) with
// the L2 distance (Sec. 3.2) or the L1 / cosine distances of Sec. 3.3; selection drops the lowest-scoring tokens, the same
// count in every sample, yielding the reduced set x~ of Sec. 3.1.
#include "rs_device.hpp"
#include "rs_launch.hpp"
#include "../../include/rs.h"

namespace rs {
namespace {

// ---------------------------------------------------------------- LayerNorm preparation
// LayerNorm (Sec. 3.3) runs folded into the GEMM that consumes it (see rs_gemm.hip); these
// two kernels prepare it: the slice statistics of a block input that no GEMM epilogue
// produced (the encoder's first block), and the folded weights W' = W diag(gamma),
// c = W' 1, d = W beta + b.

// One wave per row; lane ch handles 8-element chunk ch (and ch + 64), so the 8 lanes
// 8s..8s+7 of an iteration hold slice s: its mean, then the sum of squared deviations.
template <typename T>
__global__ __launch_bounds__(256) void row_stats_kernel(const T* __restrict__ x,
                                                        float* __restrict__ stats, int M, int C) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;  // whole wave
  const int nch = C >> 3, stride = stat_stride(C);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int ch = lane + it * 64;
    if (it * 64 >= nch) break;  // uniform
    float v[8];
    if (ch < nch) {
      load8f(x + (size_t)row * C + ch * 8, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[e];
    const float mean = sum8(s) * (1.0f / 64.0f);
    float m2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = v[e] - mean;
      m2 += d * d;
    }
    m2 = sum8(m2);
    if ((ch & 7) == 0 && ch < nch) {
      float* so = stats + ((size_t)row * stride + (ch >> 3)) * 2;
      so[0] = mean;
      so[1] = m2;
    }
  }
}

struct FoldArgs {
  FoldJob job[kMaxFoldJobs];
  int rows_before[kMaxFoldJobs + 1];  // prefix sum of job rows
  int njobs;
  int C;
};

// 16 lanes per output row n of one job (four rows per wave): W'[n][k] = W[n][k] * gamma[k]
// (rounded to the storage type; only if the job has an output), c[n] = sum_k W'[n][k] (or
// the unrounded sum_k W[n][k] gamma[k]), d[n] = sum_k W[n][k] beta[k] + b[n].  Lane s of
// a row takes 8-element chunks s, s + 16, ... (at most 8 for C <= 1024) and requests all
// of them before using any, so a wave keeps up to 32 row chunks in flight.
constexpr int kFoldLanes = 16, kFoldRowsPerBlock = 256 / kFoldLanes;
template <typename T>
__global__ __launch_bounds__(256) void fold_kernel(FoldArgs fa) {
  constexpr int kMaxCh = 1024 / 8 / kFoldLanes;
  const int total = fa.rows_before[fa.njobs];
  const int r = blockIdx.x * kFoldRowsPerBlock + (threadIdx.x / kFoldLanes);
  const int sub = threadIdx.x % kFoldLanes;
  // a row past the end repeats the last row's reads (its 16 lanes still take part in the
  // row sums) and stores nothing
  const bool live = r < total;
  const int rr = live ? r : total - 1;
  int j = 0;
  while (j + 1 < fa.njobs && rr >= fa.rows_before[j + 1]) ++j;
  const FoldJob& jb = fa.job[j];
  const int n = rr - fa.rows_before[j], C = fa.C, nch = C >> 3;
  const T* w = static_cast<const T*>(jb.w) + (size_t)n * C;
  T* wo = jb.w_out && live ? static_cast<T*>(jb.w_out) + (size_t)n * C : nullptr;
  Frag8<T> raw[kMaxCh];
#pragma unroll
  for (int i = 0; i < kMaxCh; ++i) {
    const int ch = sub + i * kFoldLanes;
    if (ch < nch) load_frag(raw[i], w + ch * 8);
  }
  float c = 0.f, d = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxCh; ++i) {
    const int ch = sub + i * kFoldLanes;
    if (ch >= nch) break;
    float wv[8], g[8], b[8], o[8];
    frag_to_f32(raw[i], wv);
    load8f(static_cast<const T*>(jb.gamma) + ch * 8, g);
    load8f(static_cast<const T*>(jb.beta) + ch * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = jb.w_out ? round_t<T>(wv[e] * g[e]) : wv[e] * g[e];
      c += o[e];
      d = fmaf(wv[e], b[e], d);
    }
    if (wo) store8f(wo + ch * 8, o);
  }
  c = sum16(c);
  d = sum16(d);
  if (sub == 0 && live) {
    jb.c[n] = c;
    jb.d[n] = d + to_f32(static_cast<const T*>(jb.bias)[n]);
  }
}

// ---------------------------------------------------------------- around the encoder
// Class-token rows of the patch embedding (Sec. 3.1 tokens, class token first):
// out[b][0] = cls + pos[0] as stored, and that row's slice partials for the first
// block's LayerNorm.  One wave per sample, lanes as in row_stats_kernel.
template <typename T>
__global__ __launch_bounds__(256) void cls_rows_kernel(const T* __restrict__ cls,
                                                       const T* __restrict__ pos,
                                                       T* __restrict__ out,
                                                       float* __restrict__ stats, int B, int L,
                                                       int C) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= B) return;  // whole wave
  const size_t row = (size_t)b * L;
  const int nch = C >> 3, stride = stat_stride(C);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int ch = lane + it * 64;
    if (it * 64 >= nch) break;  // uniform
    float v[8];
    if (ch < nch) {
      float a[8], q[8];
      load8f(cls + ch * 8, a);
      load8f(pos + ch * 8, q);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = round_t<T>(a[e] + q[e]);
      store8f(out + row * C + ch * 8, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    float sm = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sm += v[e];
    const float mean = sum8(sm) * (1.0f / 64.0f);
    float m2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = v[e] - mean;
      m2 += d * d;
    }
    m2 = sum8(m2);
    if ((ch & 7) == 0 && ch < nch && stats) {
      float* so = stats + (row * stride + (ch >> 3)) * 2;
      so[0] = mean;
      so[1] = m2;
    }
  }
}

// Final LayerNorm and pooling before the head, in two launches.  pool_partial_kernel: one
// workgroup (4 waves) per (sample, block of kPoolRows rows); a wave normalises each of its
// rows (mean, then biased variance of the deviations, in fp32) and adds the normalised
// values to per-lane sums of the lane's 8-element chunks; the four waves' sums are added in
// a fixed order through LDS and written as the block's partial [C].  mode 0 (class token):
// row 0 alone, one block.  pool_finish_kernel sums a sample's blocks in order, divides by
// the row count (mode 1) and applies gamma, beta.
template <typename T>
__global__ __launch_bounds__(256) void pool_partial_kernel(const T* __restrict__ x, float eps,
                                                           int L, int C, int mode,
                                                           float* __restrict__ part) {
  __shared__ float wsum[4][RS_MAX_WIDTH];
  const int b = blockIdx.y, blk = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = C >> 3;
  const float invC = 1.0f / (float)C;
  float acc[2][8];
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[it][e] = 0.f;
  const int r0 = blk * kPoolRows, r1 = mode == 0 ? 1 : min(L, r0 + kPoolRows);
  for (int t = r0 + wave; t < r1; t += 4) {
    const T* xr = x + ((size_t)b * L + t) * C;
    float v[2][8];
    float sm = 0.f;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int ch = lane + it * 64;
      if (ch < nch) {
        load8f(xr + ch * 8, v[it]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[it][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm += v[it][e];
    }
    const float mean = wave_sum(sm) * invC;
    float q = 0.f;
#pragma unroll
    for (int it = 0; it < 2; ++it)
      if (lane + it * 64 < nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = v[it][e] - mean;
          q += d * d;
        }
      }
    const float rstd = 1.0f / sqrtf(wave_sum(q) * invC + eps);
#pragma unroll
    for (int it = 0; it < 2; ++it)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[it][e] += (v[it][e] - mean) * rstd;
  }
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int ch = lane + it * 64;
    if (ch < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wsum[wave][ch * 8 + e] = acc[it][e];
    }
  }
  __syncthreads();
  float* out = part + ((size_t)b * gridDim.x + blk) * C;
  for (int c = threadIdx.x; c < C; c += 256)
    out[c] = ((wsum[0][c] + wsum[1][c]) + wsum[2][c]) + wsum[3][c];
}

template <typename T>
__global__ __launch_bounds__(256) void pool_finish_kernel(const float* __restrict__ part,
                                                          const T* __restrict__ gamma,
                                                          const T* __restrict__ beta, int L,
                                                          int C, int mode, int nparts,
                                                          T* __restrict__ feat) {
  const int b = blockIdx.x;
  const float inv = mode == 0 ? 1.0f : 1.0f / (float)L;
  const float* pb = part + (size_t)b * nparts * C;
  for (int c = threadIdx.x; c < C; c += 256) {
    float z = 0.f;
    for (int q = 0; q < nparts; ++q) z += pb[(size_t)q * C + c];
    z *= inv;
    feat[(size_t)b * C + c] = from_f32<T>(fmaf(to_f32(gamma[c]), z, to_f32(beta[c])));
  }
}

// ---------------------------------------------------------------- standalone score
// Distance of one token's two rows from its accumulated sums: L2 sqrt(s0); L1 s0; cosine
// 1 - s0 / max(sqrt(s1) sqrt(s2), 1e-8) with s0 = a.b, s1 = a.a, s2 = b.b.
__device__ __forceinline__ float finish_dist(int dist, float s0, float s1, float s2) {
  if (dist == 0) return sqrtf(s0);
  if (dist == 1) return s0;
  return 1.0f - s0 / fmaxf(sqrtf(s1) * sqrtf(s2), 1e-8f);
}

// 16 lanes per row: D(fx, x) accumulated in fp32.
template <typename T>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ fx,
                                                    const T* __restrict__ x,
                                                    float* __restrict__ s, int M, int C,
                                                    int dist) {
  // 16 lanes per row; each lane takes every 16th 8-element chunk.  A row of up to 1024
  // elements is at most 8 chunks per lane, all requested before any is used, so a lane
  // waits for memory once per 8 chunks instead of once per chunk.
  constexpr int U = 8;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4), sub = threadIdx.x & 15;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f;
  if (row < M) {
    const size_t base = (size_t)row * C;
    const int nch = C >> 3;
    for (int c0 = 0; c0 < nch; c0 += 16 * U) {
      Frag8<T> fa[U], fb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ch = c0 + sub + 16 * u;
        if (ch < nch) {
          load_frag(fa[u], fx + base + ch * 8);
          load_frag(fb[u], x + base + ch * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ch = c0 + sub + 16 * u;
        if (ch < nch) {
          float a[8], b[8];
          frag_to_f32(fa[u], a);
          frag_to_f32(fb[u], b);
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
      }
    }
  }
  s0 = sum16(s0);
  if (dist == 2) {
    s1 = sum16(s1);
    s2 = sum16(s2);
  }
  if (sub == 0 && row < M) s[row] = finish_dist(dist, s0, s1, s2);
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
constexpr int kWaveMaxL = 256;

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

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

// One workgroup per sample, or G per sample when rows are copied (see below).  Selection
// of the k largest keys (ties to the lower index): the
// exact k-th largest key T by a 4-pass 8-bit radix select (MSB first) over an LDS
// histogram; kept = every key above T plus the lowest-index keys equal to it.
//  - L <= kWaveMaxL: wave 0 alone, 4 keys per lane, lane scans instead of workgroup
//    barriers (a short row's selection is otherwise all barrier latency).
//  - longer L: all threads, one histogram pass per 8 bits with workgroup barriers.
// Kept indices are emitted in ascending index order (block scans), composed with ids_in,
// and listed in LDS; then the workgroup copies up to two row sets of the kept rows
// (RowCopy: 16-byte units per row), so selection and compaction are one launch.  With G
// workgroups per sample every one of them makes the (deterministic, integer-only)
// selection, copies its contiguous share of the kept rows, and only the first writes the
// scores, indices and ids.
struct RowCopy {
  const char* src;  // [L] rows of `units` 16-byte units per sample, or null
  char* dst;        // [k] rows per sample
  int units;
};

// Copies kept rows j in [j0, j1) of sample b: dst row j = src row list[j].
__device__ __forceinline__ void copy_rows(const RowCopy& c, const uint32_t* list, int b, int L, int k,
                                          int j0, int j1) {
  if (!c.src) return;
  const int upr = c.units;
  const u32x4* src = reinterpret_cast<const u32x4*>(c.src) + (long long)b * L * upr;
  u32x4* dst = reinterpret_cast<u32x4*>(c.dst) + (long long)b * k * upr;
  constexpr int U = 8;  // rows in flight per thread
  const int tid = threadIdx.x;
  if (upr <= kTopkThreads) {
    // thread -> (row offset r, unit cu), fixed; rows j0 + r, j0 + r + rpi, ...
    const int rpi = kTopkThreads / upr, r = tid / upr, cu = tid - r * upr;
    if (r >= rpi) return;
    for (int jb = j0 + r; jb < j1; jb += rpi * U) {
      u32x4 v[U];
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int j = jb + q * rpi;
        if (j < j1) v[q] = src[(long long)list[j] * upr + cu];
      }
#pragma unroll
      for (int q = 0; q < U; ++q) {
        const int j = jb + q * rpi;
        if (j < j1) dst[(long long)j * upr + cu] = v[q];
      }
    }
  } else {
    for (int j = j0; j < j1; ++j) {
      const u32x4* s = src + (long long)list[j] * upr;
      u32x4* d = dst + (long long)j * upr;
      for (int cu = tid; cu < upr; cu += kTopkThreads) d[cu] = s[cu];
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float* __restrict__ scores, const float* __restrict__ part, int P, int dist, int L,
    int k, int has_cls, float* __restrict__ scores_out, int32_t* __restrict__ kept,
    const int32_t* __restrict__ ids_in, int32_t* __restrict__ ids_out, RowCopy c0, RowCopy c1,
    int G) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[RS_MAX_TOKENS];  // keys, then the kept list
  __shared__ uint32_t hist[256];
  __shared__ int wsum[kTopkThreads / 64];
  __shared__ uint32_t sel[2];
  // G workgroups per sample: each makes the same selection; workgroup g copies kept rows
  // [g k / G, (g + 1) k / G), and workgroup 0 alone writes scores, indices and ids
  const int b = blockIdx.x / G, g = blockIdx.x - b * G, tid = threadIdx.x;
  const bool lead = g == 0;
  const int cj0 = (int)((long long)g * k / G), cj1 = (int)((long long)(g + 1) * k / G);
  const size_t rb = (size_t)b * L;

  for (int i = tid; i < L; i += kTopkThreads) {
    float s;
    if (part) {
      // the token's slice partials: quantity q of slice p at q * P + p
      const float* pp = part + (rb + i) * (size_t)(dist == 2 ? 3 * P : P);
      float a = 0.f, aa = 0.f, bb = 0.f;
      for (int q = 0; q < P; ++q) a += pp[q];
      if (dist == 2)
        for (int q = 0; q < P; ++q) {
          aa += pp[P + q];
          bb += pp[2 * P + q];
        }
      s = finish_dist(dist, a, aa, bb);
    } else {
      s = scores[rb + i];
    }
    if (scores_out && lead) scores_out[rb + i] = s;
    keys[i] = (has_cls && i == 0) ? 0xFFFFFFFFu : order_key(s);
  }
  __syncthreads();

  // per-thread segment [i0, i1) and its keep flags (bit i - i0)
  const int seg = (L + kTopkThreads - 1) / kTopkThreads;  // <= 16
  const int i0 = min(tid * seg, L), i1 = min(i0 + seg, L);
  uint32_t keepbits = 0u;
  if (L <= kWaveMaxL) {
    // wave 0 alone: lane l holds keys 4l .. 4l + 3
    if (tid < 64) {
      const int lane = tid;
      uint32_t kk[4];
      bool valid[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        valid[q] = 4 * lane + q < L;
        kk[q] = valid[q] ? keys[4 * lane + q] : 0u;
      }
      uint32_t prefix = 0u, pmask = 0u, krem = (uint32_t)k;
      for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) hist[4 * lane + q] = 0u;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (valid[q] && (kk[q] & pmask) == prefix) atomicAdd(&hist[(kk[q] >> shift) & 255u], 1u);
        __builtin_amdgcn_wave_barrier();
        // lane covers bins 255-4*lane down to 252-4*lane; counts above run high -> low
        uint32_t c[4], loc = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[q] = hist[255 - 4 * lane - q];
          loc += c[q];
        }
        uint32_t above = wave_inclusive_scan(loc) - loc;
        uint32_t bin = 0u, ab = 0u;
        bool found = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (above < krem && above + c[q] >= krem) {
            found = true;
            bin = (uint32_t)(255 - 4 * lane - q);
            ab = above;
          }
          above += c[q];
        }
        const int src = __ffsll((unsigned long long)__ballot(found)) - 1;
        bin = __shfl(bin, src, 64);
        ab = __shfl(ab, src, 64);
        prefix |= bin << shift;
        pmask |= 0xFFu << shift;
        krem -= ab;
        __builtin_amdgcn_wave_barrier();
      }
      const uint32_t T = prefix;  // the k-th largest key; krem of its copies are kept
      uint32_t eq = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) eq += (valid[q] && kk[q] == T) ? 1u : 0u;
      uint32_t e = wave_inclusive_scan(eq) - eq;
      uint32_t keep = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (valid[q] && (kk[q] > T || (kk[q] == T && e < krem))) keep |= 1u << q;
        e += (valid[q] && kk[q] == T) ? 1u : 0u;
      }
      const uint32_t cnt = __builtin_popcount(keep);
      uint32_t pos = wave_inclusive_scan(cnt) - cnt;
      int32_t* kb = kept + (size_t)b * k;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (((keep >> q) & 1u) && pos < (uint32_t)k) {
          const int i = 4 * lane + q;
          if (lead) {
            kb[pos] = i;
            if (ids_out) ids_out[(size_t)b * k + pos] = ids_in ? ids_in[rb + i] : i;
          }
          keys[pos] = (uint32_t)i;  // kept list (the keys were read into registers above)
          ++pos;
        }
      }
    }
    if (!c0.src && !c1.src) return;
    __syncthreads();
    copy_rows(c0, keys, b, L, k, cj0, cj1);
    copy_rows(c1, keys, b, L, k, cj0, cj1);
    return;
  }
  {
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
    int eq = 0;
    for (int i = i0; i < i1; ++i) eq += keys[i] == T;
    int e = block_exclusive_scan(eq, wsum);
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = keys[i];
      if (key > T || (key == T && (uint32_t)e < krem)) keepbits |= 1u << (i - i0);
      e += key == T;
    }
  }
  int pos = block_exclusive_scan(__builtin_popcount(keepbits), wsum);  // also orders keys reads
  int32_t* kb = kept + (size_t)b * k;
  for (int i = i0; i < i1; ++i) {
    if (((keepbits >> (i - i0)) & 1u) && pos < k) {
      if (lead) {
        kb[pos] = i;
        if (ids_out) ids_out[(size_t)b * k + pos] = ids_in ? ids_in[rb + i] : i;
      }
      keys[pos] = (uint32_t)i;  // kept list (every key read above is done: scan barrier)
      ++pos;
    }
  }
  if (!c0.src && !c1.src) return;
  __syncthreads();
  copy_rows(c0, keys, b, L, k, cj0, cj1);
  copy_rows(c1, keys, b, L, k, cj0, cj1);
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

hipError_t launch_row_stats(Dtype dt, const void* x, float* stats, int M, int C, hipStream_t stream) {
  const int grid = (M + 3) / 4;
  if (dt == kBF16)
    row_stats_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(x), stats, M, C);
  else
    row_stats_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(x), stats, M, C);
  return hipGetLastError();
}

hipError_t launch_fold(Dtype dt, const FoldJob* jobs, int njobs, int C, hipStream_t stream) {
  FoldArgs fa;
  fa.njobs = njobs;
  fa.C = C;
  fa.rows_before[0] = 0;
  for (int j = 0; j < njobs; ++j) {
    fa.job[j] = jobs[j];
    fa.rows_before[j + 1] = fa.rows_before[j] + jobs[j].rows;
  }
  const int grid = (fa.rows_before[njobs] + kFoldRowsPerBlock - 1) / kFoldRowsPerBlock;
  if (dt == kBF16)
    fold_kernel<bf16><<<grid, 256, 0, stream>>>(fa);
  else
    fold_kernel<float><<<grid, 256, 0, stream>>>(fa);
  return hipGetLastError();
}

hipError_t launch_cls_rows(Dtype dt, const void* cls, const void* pos, void* out, float* stats,
                           int B, int L, int C, hipStream_t stream) {
  const int grid = (B + 3) / 4;
  if (dt == kBF16)
    cls_rows_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(cls),
                                                    static_cast<const bf16*>(pos),
                                                    static_cast<bf16*>(out), stats, B, L, C);
  else
    cls_rows_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(cls),
                                                     static_cast<const float*>(pos),
                                                     static_cast<float*>(out), stats, B, L, C);
  return hipGetLastError();
}

hipError_t launch_pool(Dtype dt, const void* x, const void* gamma, const void* beta, float eps,
                       int B, int L, int C, int mode, float* part, void* feat, hipStream_t stream) {
  const int np = pool_parts(L, mode);
  const dim3 grid(np, B);
  if (dt == kBF16) {
    pool_partial_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(x), eps, L, C,
                                                        mode, part);
    pool_finish_kernel<bf16><<<B, 256, 0, stream>>>(part, static_cast<const bf16*>(gamma),
                                                    static_cast<const bf16*>(beta), L, C, mode,
                                                    np, static_cast<bf16*>(feat));
  } else {
    pool_partial_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(x), eps, L, C,
                                                         mode, part);
    pool_finish_kernel<float><<<B, 256, 0, stream>>>(part, static_cast<const float*>(gamma),
                                                     static_cast<const float*>(beta), L, C, mode,
                                                     np, static_cast<float*>(feat));
  }
  return hipGetLastError();
}

hipError_t launch_score_rows(Dtype dt, const void* fx, const void* x, float* scores, int M, int C,
                             int dist, hipStream_t stream) {
  const int grid = (M + 15) / 16;
  if (dt == kBF16)
    score_kernel<bf16><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(fx),
                                                 static_cast<const bf16*>(x), scores, M, C, dist);
  else
    score_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(fx),
                                                  static_cast<const float*>(x), scores, M, C, dist);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, const float* part, int P, int dist, int B, int L,
                       int k, int has_cls, float* scores_out, int32_t* kept,
                       const int32_t* ids_in, int32_t* ids_out, const TopkCopy* copies,
                       int ncopies, hipStream_t stream) {
  RowCopy c[2] = {{nullptr, nullptr, 0}, {nullptr, nullptr, 0}};
  for (int i = 0; i < ncopies && i < 2; ++i)
    c[i] = {static_cast<const char*>(copies[i].src), static_cast<char*>(copies[i].dst),
            copies[i].row_bytes / 16};
  const int G = ncopies > 0 ? topk_copy_split(B) : 1;
  topk_kernel<<<B * G, kTopkThreads, 0, stream>>>(scores, part, P, dist, L, k, has_cls, scores_out,
                                                  kept, ids_in, ids_out, c[0], c[1], G);
  return hipGetLastError();
}

hipError_t launch_iota(int32_t* ids, int B, int L, hipStream_t stream) {
  const long long total = (long long)B * L;
  iota_kernel<<<grid_for(total), 256, 0, stream>>>(ids, L, total);
  return hipGetLastError();
}

}  // namespace rs
