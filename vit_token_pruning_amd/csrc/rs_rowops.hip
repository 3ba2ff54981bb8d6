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
      m2 = fmaf(d, d, m2);   // explicit: every statistics producer rounds alike
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
static_assert(sizeof(FoldArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// 16 lanes per output row n of one job (four rows per wave): W'[n][k] = W[n][k] * gamma[k]
// (rounded to the storage type; only if the job has an output), c[n] = sum_k W'[n][k] (or
// the unrounded sum_k W[n][k] gamma[k]), d[n] = sum_k W[n][k] beta[k] + b[n].  A job
// without gamma copies W unchanged (no c, d).  A packed job (bf16) writes W' in the
// weight-streaming linear kernel's layout instead of row-major: 8-element chunk ch of row n
// goes to slice n / 32, fragment block 2 (ch / 4) + t, lane 16 (ch % 4) + l16, where row
// n % 32 = 8 (l16 / 4) + 4 t + l16 % 4.  Lane s of a row takes 8-element chunks s, s + 16,
// ... (at most 8 for C <= 1024) and requests all of them before using any, so a wave keeps
// up to 32 row chunks in flight.
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
  const bool fold = jb.gamma != nullptr;
  const T* w = static_cast<const T*>(jb.w) + (size_t)n * C;
  char* wo = jb.w_out && live ? static_cast<char*>(jb.w_out) : nullptr;
  // packed layout: this row's place within its slice
  const int n32 = n & 31, pt = (n32 >> 2) & 1, pl16 = 4 * (n32 >> 3) + (n32 & 3);
  const size_t pslice = (size_t)(n >> 5) * (C >> 5) * 2 * 1024;
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
    if (fold) {
      load8f(static_cast<const T*>(jb.gamma) + ch * 8, g);
      load8f(static_cast<const T*>(jb.beta) + ch * 8, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = jb.w_out ? round_t<T>(wv[e] * g[e]) : wv[e] * g[e];
        c += o[e];
        d = fmaf(wv[e], b[e], d);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = wv[e];
    }
    if (wo) {
      if constexpr (sizeof(T) == 2) {
        if (jb.packed) {
          const size_t off = pslice + (size_t)(2 * (ch >> 2) + pt) * 1024 + ((ch & 3) * 16 + pl16) * 16;
          store8f(reinterpret_cast<T*>(wo + off), o);
          continue;
        }
      }
      store8f(reinterpret_cast<T*>(wo) + (size_t)n * C + ch * 8, o);
    }
  }
  c = sum16(c);   // (every row's 16 lanes take part; a copy job's sums are unused)
  d = sum16(d);
  if (fold && sub == 0 && live) {
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
      m2 = fmaf(d, d, m2);   // explicit: every statistics producer rounds alike
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
  // waits for memory once per 8 chunks instead of once per chunk.  Both rows are read
  // once: non-temporal loads (DeiT-S 256 x 197 x 384 bf16: 14.6 -> 13.2 us per call).
  // Measured against 8 lanes per row (more chunks in flight per lane): slower.
  constexpr int U = 8, LPR = 16;
  const int row = blockIdx.x * (256 / LPR) + (threadIdx.x / LPR), sub = threadIdx.x % LPR;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f;
  if (row < M) {
    const size_t base = (size_t)row * C;
    const int nch = C >> 3;
    for (int c0 = 0; c0 < nch; c0 += LPR * U) {
      Frag8<T> fa[U], fb[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ch = c0 + sub + LPR * u;
        if (ch < nch) {
          load_frag_nt(fa[u], fx + base + ch * 8);
          load_frag_nt(fb[u], x + base + ch * 8);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ch = c0 + sub + LPR * u;
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

constexpr int kTopkThreads = 512, kTopkWaves = kTopkThreads / 64;
// score partials per token: 2 per 128-column tile of a row of at most RS_MAX_WIDTH columns
constexpr int kMaxPartPairs = (RS_MAX_WIDTH + 127) / 128;
// Radix select: 11-bit digits (at most three passes over a 32-bit key), each pass with its
// own histogram of 2048 bins plus 64 buckets of 32 bins (the bucket counts let a wave find
// the selected bin with two 64-lane scans instead of reading all 2048 bins).
constexpr int kDigitBits = 11, kBins = 1 << kDigitBits, kBuckets = kBins / 32, kPasses = 3;
static_assert(32 * kTopkThreads >= RS_MAX_TOKENS, "top-k holds at most 32 keys per thread");
static_assert(RS_MAX_TOKENS < 65536, "the emission scan packs two 16-bit counts");

// Wave-wide inclusive scans with DPP: row shifts by 1, 2, 4, 8 within each row of 16
// lanes, then row 0's total broadcast into row 1 (and row 2's into row 3), then lane 31's
// into rows 2 and 3.  Lanes a shift leaves without a source take `id`.
template <class Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t id, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x111, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x112, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x114, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x118, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xa, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xc, 0xf, false));
  return v;
}
struct AddU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct MinU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};
struct MaxU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) { return wave_scan(v, 0u, AddU32()); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(v, ~0u, MinU32()), 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan(v, 0u, MaxU32()), 63);
}
// Workgroup barrier that waits only for this wave's LDS operations: the top-k's barriers
// order LDS traffic alone, and __syncthreads() would also wait for the global stores of
// scores, indices and ids still in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// exclusive prefix sum over the threads of the workgroup (kTopkWaves waves); wsum is
// written once, so a workgroup calls this once
__device__ __forceinline__ int block_exclusive_scan_once(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = (int)wave_inclusive_scan((uint32_t)v);
  if (lane == 63) wsum[wave] = incl;
  lds_barrier();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves - 1; ++w) before += w < wave ? wsum[w] : 0;
  return before + incl - v;
}

// Rows of kept tokens to copy (16-byte units per row).
struct RowCopy {
  const char* src;  // [L] rows of `units` 16-byte units per sample, or null
  char* dst;        // [k] rows per sample
  int units;
};

// Copies kept rows j in [j0, j1) of sample b: dst row j = src row list[j].  (Non-temporal
// loads of the source rows measured slower: DeiT-S 12.2 -> 13.0 us per call.)
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

// LDS of the top-k kernel: per radix pass the bin counts and the 32-bin bucket counts
// (cleared once, so a pass never waits for the previous pass's readers), per-wave partials.
struct __attribute__((aligned(16))) TopkShared {
  uint32_t fine[kPasses][kBins];
  uint32_t coarse[kPasses][kBuckets];
  uint32_t wlo[kTopkWaves], whi[kTopkWaves];
  int wsum[kTopkWaves];
};

// One workgroup per sample, or G per sample when rows are copied.  Thread t holds the
// keys of tokens t R .. t R + R - 1 in registers (R = keys per thread, L <= R kTopkThreads).
// The score of each token is finished from the GEMM epilogues' partials (or read) and
// mapped to an order key; the class token (index 0 when has_cls) is kept outside the
// selection.  Selection of the k largest (ties to the lower index): the competing keys'
// common high bits are skipped (their minimum and maximum share them), then MSB-first
// 11-bit digits: each pass counts the keys that match the prefix found so far into its
// histogram, one workgroup barrier, and every wave finds the same bin holding the
// krem-th largest (bucket scan, then bin scan).  T = the k-th largest key, krem = how
// many of its copies are kept (the lowest-index ones); a bin whose keys are all kept ends
// the passes early (T = the bin's lowest possible key, every copy kept).  One packed scan
// of (keys above T, keys equal to T) per thread places the kept tokens in ascending index
// order.  With G workgroups per sample every one of them makes the same (integer-only)
// selection and copies its contiguous share of the kept rows (listed in dynamic LDS);
// workgroup 0 of the sample alone writes the scores, indices and ids.
template <int R>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float* __restrict__ scores, const float* __restrict__ part, int P, int dist, int L,
    int k, int has_cls, float* __restrict__ scores_out, int32_t* __restrict__ kept,
    const int32_t* __restrict__ ids_in, int32_t* __restrict__ ids_out, RowCopy c0, RowCopy c1,
    int G) {
  __shared__ TopkShared sh;
  extern __shared__ __attribute__((aligned(16))) uint32_t list[];   // k words when copying
  const int b = blockIdx.x / G, g = blockIdx.x - b * G, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool lead = g == 0;
  const size_t rb = (size_t)b * L;
  {
    constexpr int n4 = kPasses * (kBins + kBuckets) / 4;   // fine and coarse are contiguous
    u32x4* h = reinterpret_cast<u32x4*>(&sh.fine[0][0]);
    for (int i = tid; i < n4; i += kTopkThreads) h[i] = u32x4{0u, 0u, 0u, 0u};
  }
  const int i0 = tid * R;
  float sv[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = i0 + j;
    sv[j] = 0.f;
    if (i < L) {
      if (part) {
        // the token's slice partials: quantity q of slice p at q * P + p (P even, <= 16,
        // so 8-byte aligned pairs); every pair is requested before any is summed, and the
        // sums run in slice order
        const float2* pp = reinterpret_cast<const float2*>(part + (rb + i) * (size_t)(dist == 2 ? 3 * P : P));
        const int P2 = P >> 1;
        float2 v[kMaxPartPairs];
#pragma unroll
        for (int h = 0; h < kMaxPartPairs; ++h) v[h] = h < P2 ? pp[h] : make_float2(0.f, 0.f);
        float a = 0.f, aa = 0.f, bb = 0.f;
#pragma unroll
        for (int h = 0; h < kMaxPartPairs; ++h)
          if (h < P2) {
            a += v[h].x;
            a += v[h].y;
          }
        if (dist == 2) {
#pragma unroll
          for (int h = 0; h < kMaxPartPairs; ++h) v[h] = h < P2 ? pp[P2 + h] : make_float2(0.f, 0.f);
          float2 w[kMaxPartPairs];
#pragma unroll
          for (int h = 0; h < kMaxPartPairs; ++h) w[h] = h < P2 ? pp[2 * P2 + h] : make_float2(0.f, 0.f);
#pragma unroll
          for (int h = 0; h < kMaxPartPairs; ++h)
            if (h < P2) {
              aa += v[h].x;
              aa += v[h].y;
              bb += w[h].x;
              bb += w[h].y;
            }
        }
        sv[j] = finish_dist(dist, a, aa, bb);
      } else {
        sv[j] = scores[rb + i];
      }
    }
  }
  uint32_t kk[R];
  uint32_t vmask = 0u, lo = ~0u, hi = 0u;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = i0 + j;
    kk[j] = order_key(sv[j]);
    if (i < L) {
      if (scores_out && lead) scores_out[rb + i] = sv[j];
      if (!(has_cls && i == 0)) {
        vmask |= 1u << j;
        lo = min(lo, kk[j]);
        hi = max(hi, kk[j]);
      }
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    sh.wlo[wave] = lo;
    sh.whi[wave] = hi;
  }
  lds_barrier();   // histograms cleared, per-wave extremes written
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    lo = min(lo, sh.wlo[w]);
    hi = max(hi, sh.whi[w]);
  }

  uint32_t krem = (uint32_t)(k - has_cls);
  uint32_t T = ~0u;
  if (krem > 0) {
    T = lo;
    if (lo != hi) {
      const int hb = 31 - __builtin_clz(lo ^ hi);          // highest bit where keys differ
      uint32_t pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);  // the common bits above it
      uint32_t prefix = hi & pmask;
      for (int top = hb, pass = 0; top >= 0; ++pass) {      // uniform; at most kPasses
        const int width = min(kDigitBits, top + 1), shift = top - width + 1;
        const int nb = 1 << width;
        const uint32_t dmask = (uint32_t)nb - 1u;
        uint32_t* const fine = sh.fine[pass];
        uint32_t* const coarse = sh.coarse[pass];
#pragma unroll
        for (int j = 0; j < R; ++j)
          if (((vmask >> j) & 1u) && (kk[j] & pmask) == prefix) {
            const uint32_t d = (kk[j] >> shift) & dmask;
            atomicAdd(&fine[d], 1u);
            atomicAdd(&coarse[d >> 5], 1u);
          }
        lds_barrier();
        // buckets high -> low on lanes 0, 1, ...: the bucket holding the krem-th largest
        const int nbk = nb >= 32 ? nb >> 5 : 1, bpb = nb >= 32 ? 32 : nb;
        const uint32_t cc = lane < nbk ? coarse[nbk - 1 - lane] : 0u;
        const uint32_t ci = wave_inclusive_scan(cc);
        const int cl = __ffsll((unsigned long long)__ballot(ci >= krem)) - 1;
        const int cb = nbk - 1 - cl;
        const uint32_t abk = (uint32_t)__builtin_amdgcn_readlane((int)(ci - cc), cl);
        // its bins high -> low: the bin
        const uint32_t fc = lane < bpb ? fine[cb * 32 + bpb - 1 - lane] : 0u;
        const uint32_t fi = wave_inclusive_scan(fc);
        const int fl = __ffsll((unsigned long long)__ballot(abk + fi >= krem)) - 1;
        const uint32_t bin = (uint32_t)(cb * 32 + bpb - 1 - fl);
        const uint32_t ab = abk + (uint32_t)__builtin_amdgcn_readlane((int)(fi - fc), fl);
        const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)fc, fl);
        prefix |= bin << shift;
        pmask |= dmask << shift;
        krem -= ab;
        if (cnt == krem) {   // every key of the bin is kept
          krem = (uint32_t)k;
          break;
        }
        top = shift - 1;
      }
      T = prefix;
    }
  }

  // kept = the class token, every key above T, the first krem copies of T in index order
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const bool v = (vmask >> j) & 1u;
    gt += (has_cls && i0 + j == 0) || (v && kk[j] > T) ? 1u : 0u;
    eq += v && kk[j] == T ? 1u : 0u;
  }
  // (counts <= L <= 16384 fit 16 bits each)
  const uint32_t before = (uint32_t)block_exclusive_scan_once((int)(gt | (eq << 16)), sh.wsum);
  uint32_t e = before >> 16;
  uint32_t pos = (before & 0xFFFFu) + min(e, krem);
  const bool copy = c0.src || c1.src;
  int32_t* kb = kept + (size_t)b * k;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = i0 + j;
    const bool v = (vmask >> j) & 1u;
    bool keep = (has_cls && i == 0) || (v && kk[j] > T);
    if (v && kk[j] == T) {
      keep = e < krem;
      ++e;
    }
    if (keep && pos < (uint32_t)k) {
      if (lead) {
        kb[pos] = i;
        if (ids_out) ids_out[(size_t)b * k + pos] = ids_in ? ids_in[rb + i] : i;
      }
      if (copy) list[pos] = (uint32_t)i;
      ++pos;
    }
  }
  if (!copy) return;
  lds_barrier();
  const int cj0 = (int)((long long)g * k / G), cj1 = (int)((long long)(g + 1) * k / G);
  copy_rows(c0, list, b, L, k, cj0, cj1);
  copy_rows(c1, list, b, L, k, cj0, cj1);
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

template <int R>
hipError_t launch_topk_r(int grid, size_t lds, const float* scores, const float* part, int P,
                         int dist, int L, int k, int has_cls, float* scores_out, int32_t* kept,
                         const int32_t* ids_in, int32_t* ids_out, const RowCopy& c0,
                         const RowCopy& c1, int G, hipStream_t stream) {
  // the kept list takes up to RS_MAX_TOKENS words of dynamic LDS beside the static part
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&topk_kernel<R>), hipFuncAttributeMaxDynamicSharedMemorySize,
      RS_MAX_TOKENS * 4);
  if (attr != hipSuccess) return attr;
  topk_kernel<R><<<grid, kTopkThreads, lds, stream>>>(scores, part, P, dist, L, k, has_cls,
                                                      scores_out, kept, ids_in, ids_out, c0, c1, G);
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
  const size_t lds = ncopies > 0 ? (size_t)k * 4 : 0;
  const int grid = B * G;
  if (L <= kTopkThreads)
    return launch_topk_r<1>(grid, lds, scores, part, P, dist, L, k, has_cls, scores_out, kept, ids_in, ids_out, c[0], c[1], G, stream);
  if (L <= 2 * kTopkThreads)
    return launch_topk_r<2>(grid, lds, scores, part, P, dist, L, k, has_cls, scores_out, kept, ids_in, ids_out, c[0], c[1], G, stream);
  if (L <= 4 * kTopkThreads)
    return launch_topk_r<4>(grid, lds, scores, part, P, dist, L, k, has_cls, scores_out, kept, ids_in, ids_out, c[0], c[1], G, stream);
  if (L <= 8 * kTopkThreads)
    return launch_topk_r<8>(grid, lds, scores, part, P, dist, L, k, has_cls, scores_out, kept, ids_in, ids_out, c[0], c[1], G, stream);
  return launch_topk_r<32>(grid, lds, scores, part, P, dist, L, k, has_cls, scores_out, kept, ids_in, ids_out, c[0], c[1], G, stream);
}

hipError_t launch_iota(int32_t* ids, int B, int L, hipStream_t stream) {
  const long long total = (long long)B * L;
  iota_kernel<<<grid_for(total), 256, 0, stream>>>(ids, L, total);
  return hipGetLastError();
}

}  // namespace rs
