// Device helpers shared by the gfx950 kernels: element types, 8-element register
// fragments, the 16x16x32 matrix-core step, packing and wavefront reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Eight consecutive elements of T held by one lane: the unit every kernel loads,
// stages through LDS and feeds to the matrix cores.
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { u32x4 v; };
template <> struct Frag8<float> { u32x4 v[2]; };

template <typename T> struct Chunk { static constexpr int bytes = 8 * (int)sizeof(T); };

__device__ __forceinline__ void load_frag(Frag8<bf16>& f, const void* p) { f.v = *(const u32x4*)p; }
__device__ __forceinline__ void load_frag(Frag8<float>& f, const void* p) {
  f.v[0] = ((const u32x4*)p)[0];
  f.v[1] = ((const u32x4*)p)[1];
}
// Streaming reads (data read once and not again by this kernel): non-temporal loads, which
// do not displace reused lines from the caches.
__device__ __forceinline__ void load_frag_nt(Frag8<bf16>& f, const void* p) {
  f.v = __builtin_nontemporal_load((const u32x4*)p);
}
__device__ __forceinline__ void load_frag_nt(Frag8<float>& f, const void* p) {
  f.v[0] = __builtin_nontemporal_load((const u32x4*)p);
  f.v[1] = __builtin_nontemporal_load((const u32x4*)p + 1);
}
__device__ __forceinline__ void store_frag(void* p, const Frag8<bf16>& f) { *(u32x4*)p = f.v; }
__device__ __forceinline__ void store_frag(void* p, const Frag8<float>& f) {
  ((u32x4*)p)[0] = f.v[0];
  ((u32x4*)p)[1] = f.v[1];
}
__device__ __forceinline__ void zero_frag(Frag8<bf16>& f) { f.v = u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ void zero_frag(Frag8<float>& f) {
  f.v[0] = u32x4{0u, 0u, 0u, 0u};
  f.v[1] = u32x4{0u, 0u, 0u, 0u};
}

// D(16x16) += A(16x32) * B(32x16).  Lane l holds row (l % 16) of A and column (l % 16)
// of B, each as the 8 k-values of group (l / 16); D lane l holds column (l % 16), rows
// 4*(l/16) .. 4*(l/16)+3.  The same k-slot assignment is used for A and B, so any
// consistent placement of k inside a group gives the same dot products.
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                 __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}
// fp32 operands: eight 16x16x4 steps, step j taking element j of every lane's group.
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const Frag8<float>& a, const Frag8<float>& b) {
  const float* pa = reinterpret_cast<const float*>(&a.v[0]);
  const float* pb = reinterpret_cast<const float*>(&b.v[0]);
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[j], pb[j], acc, 0, 0, 0);
  return acc;
}

// ---- direct global -> LDS loads ------------------------------------------------------
// 16 bytes per lane from global memory straight into LDS (no VGPR round trip): lane l's
// bytes land at lds + 16 l, so one wave writes 1 KiB of consecutive LDS; `lds` must be
// the same for every lane of the wave.  The builtin exists only for the device target.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
#endif
}
// Wait until at most N of this wave's vector-memory operations are outstanding (loads
// complete in issue order), leaving the LDS and export counters alone.
template <int N> __device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Workgroup barrier without the memory fence of __syncthreads(): that fence makes every
// wave drain all of its in-flight global -> LDS loads first, which would serialize a
// prefetch pipeline.  Callers wait for the loads they need with wait_vmem<> before
// arriving, and LDS reads issued before the barrier have been consumed by then.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// ---- element conversion ------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));  // RNE
}

// 8 consecutive elements <-> 8 floats
__device__ __forceinline__ void load8f(const bf16* p, float* f) {
  const u32x4 u = *(const u32x4*)p;
#pragma unroll
  for (int e = 0; e < 4; ++e) { f[2 * e] = bf16_lo(u[e]); f[2 * e + 1] = bf16_hi(u[e]); }
}
__device__ __forceinline__ void load8f(const float* p, float* f) {
  const f32x4 a = ((const f32x4*)p)[0], b = ((const f32x4*)p)[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) { f[e] = a[e]; f[4 + e] = b[e]; }
}
__device__ __forceinline__ void store8f(bf16* p, const float* f) {
  u32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(f[2 * e], f[2 * e + 1]);
  *(u32x4*)p = u;
}
__device__ __forceinline__ void store8f(float* p, const float* f) {
  ((f32x4*)p)[0] = f32x4{f[0], f[1], f[2], f[3]};
  ((f32x4*)p)[1] = f32x4{f[4], f[5], f[6], f[7]};
}
__device__ __forceinline__ void frag_to_f32(const Frag8<bf16>& f, float* o) {
#pragma unroll
  for (int e = 0; e < 4; ++e) { o[2 * e] = bf16_lo(f.v[e]); o[2 * e + 1] = bf16_hi(f.v[e]); }
}
__device__ __forceinline__ void frag_to_f32(const Frag8<float>& f, float* o) {
  const f32x4 a = __builtin_bit_cast(f32x4, f.v[0]);
  const f32x4 b = __builtin_bit_cast(f32x4, f.v[1]);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = a[e];
    o[4 + e] = b[e];
  }
}
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// the value a float takes once stored as T
template <typename T> __device__ __forceinline__ float round_t(float v) { return to_f32(from_f32<T>(v)); }


// Merge of equal-count slice partials (slice mean m_s, slice sum of squared deviations
// M2_s, 64 values each) into the row's mean and biased variance:
//   mean = avg(m_s),  M2 = sum(M2_s) + 64 * sum((m_s - mean)^2),  var = M2 / (64 * P).

// ---- wavefront reductions (64 lanes) -------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Lane exchanges inside a row of 16 lanes with DPP (plain VALU ops, no LDS routing):
// quad_perm [1,0,3,2] / [2,3,0,1], row_half_mirror (lane i <-> 7-i within 8),
// row_mirror (lane i <-> 15-i within 16).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// sum over the 8 consecutive lanes that share (lane / 8)
__device__ __forceinline__ float sum8(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: every lane holds its quad's sum
  v += dpp<0x141>(v);  // row_half_mirror: adds the other quad of the 8
  return v;
}
// sum over the 16 consecutive lanes that share (lane / 16)
__device__ __forceinline__ float sum16(float v) {
  v = sum8(v);
  v += dpp<0x140>(v);  // row_mirror: adds the other 8 of the 16
  return v;
}

// Combine the values of lanes i, i ^ 16, i ^ 32, i ^ 48 (the four 16-lane rows) with the
// gfx950 row swaps, plain VALU ops instead of LDS-routed shuffles.  permlane32_swap(v, v)
// gives every lane (v[i % 32], v[32 + i % 32]); permlane16_swap(v, v) gives (v of the
// even row, v of the odd row) of the lane's pair of rows (layout checked on the GPU with
// an in-bounds probe).  Every lane combines the two in the same order, so all four lanes
// end with the same bits.
// (The two results are read with __uint_as_float: a bit_cast of each vector element
// lets this compiler read the first result twice.)
__device__ __forceinline__ float max_rows(float v) {
#if __HIP_DEVICE_COMPILE__
  const unsigned u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const unsigned w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
#else
  return v;
#endif
}
__device__ __forceinline__ float sum_rows(float v) {
#if __HIP_DEVICE_COMPILE__
  const unsigned u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
#else
  return v;
#endif
}

// Exact GELU, z * Phi(z), with the device erf.
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// Workgroups are dealt round-robin over the 8 XCDs by launch index.  Map launch index
// `id` to a logical tile so that each XCD receives one contiguous range of logical
// tiles (neighbouring tiles then share operands in that XCD's L2).
__device__ __forceinline__ int xcd_contiguous(int id, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = id & 7, k = id >> 3;
  return x * q + (x < r ? x : r) + k;
}

}  // namespace rs
