// Throughput probes behind the attention roofline: how fast one CU issues the vector
// work of the fused attention's softmax (Eq. (1) of "Representation Shift: Unifying Token
// Compression with FlashAttention", arXiv HTML, Sec. 3.1, evaluated one key tile at a
// time), the matrix work of the same tile, and both together.  Every mode runs `iters`
// iterations of an unrolled body per wave on register data; empty asm statements mark the
// body's inputs as changed and its outputs as used, so the compiler neither hoists nor
// drops the work and adds no instructions for it.
//
//  mode 0  16 independent hardware exp2 (v_exp_f32), one per register chain
//  mode 1  16 independent fp32 FMAs
//  mode 2  the softmax of one 64-key x 16-query tile per lane's 16 scores, as the
//          attention kernel issues it: the max over 16 scores and across the lane rows,
//          the rescale test, 16 x (FMA + exp2 + add), the bf16 packing of P
//  mode 3  16 MFMA 16x16x32 bf16 (the tile's S = K Q^T and O += V^T P^T products)
//  mode 4  modes 2 and 3 interleaved in one wave on independent registers
//  mode 5  8 LDS reads of 16 bytes per lane (ds_read_b128; 1 KiB per wave, contiguous in
//          lane order, conflict free), the operand-fetch pattern of the MLP kernel
//  mode 6  8 such LDS reads and 8 MFMA 16x16x32 bf16, each product taking one fragment
//          read in the same iteration (one fragment per product, as the MLP kernel's
//          weight operands)
#include "rs_attn_frag.hpp"
#include "rs_device.hpp"
#include "rs_launch.hpp"

namespace rs {
namespace {

template <typename V> __device__ __forceinline__ void touch(V& v) { asm volatile("" : "+v"(v)); }
template <typename V> __device__ __forceinline__ void use(const V& v) { asm volatile("" ::"v"(v)); }

struct SoftmaxState {
  f32x4 s[4];
  float m_run, l_run;
};

// One tile's softmax work on the lane's 16 scores (keys 16j + 4g + v of its query).
__device__ __forceinline__ void softmax_tile(SoftmaxState& st, float scale_log2, Frag8<bf16>* pf) {
  float mx = st.s[0][0];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) mx = fmaxf(mx, st.s[j][v]);
  mx = max_rows(mx);
  const float m_new = fmaxf(st.m_run, mx);
  if (__builtin_amdgcn_ballot_w64((m_new - st.m_run) * scale_log2 > 8.0f)) {
    const float alpha = __builtin_amdgcn_exp2f((st.m_run - m_new) * scale_log2);
    st.l_run *= alpha;
    st.m_run = m_new;
  }
  const float mb = st.m_run * scale_log2;
  float psum = 0.f;
  f32x4 p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[j][v] = __builtin_amdgcn_exp2f(fmaf(st.s[j][v], scale_log2, -mb));
      psum += p[j][v];
    }
  st.l_run += psum;
  attn::pack_p(pf[0], p[0], p[1]);
  attn::pack_p(pf[1], p[2], p[3]);
}

// One body per mode, each in a loop of its own (so that no branch on the mode sits in
// the measured loop); returns a value that depends on all of the work.
template <int MODE>
__device__ __forceinline__ float probe_body(int iters, const char* lds) {
  const int tid = threadIdx.x;
  const float x0 = (float)(tid & 63) * (1.0f / 64.0f);
  float r = 0.f;
  if constexpr (MODE == 5 || MODE == 6) {
    // 16 KiB of LDS in 16 blocks of 1 KiB; iteration it reads blocks (it + i) % 16
    const char* lb = lds + (tid & 63) * 16;
    Frag8<bf16> qb;
    qb.v = u32x4{0x3c003c00u, 0x3c003c00u ^ (uint32_t)tid, 0x3c003c00u, 0x3c003c00u};
    f32x4 acc[8];
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    int off = 0;
    for (int it = 0; it < iters; ++it) {
      // the offset is opaque to the compiler (marked changed every iteration), so the
      // reads are neither hoisted out of the loop nor merged across iterations
      off ^= 8192;
      asm volatile("" : "+v"(off));
      const char* base = lb + off;
      Frag8<bf16> f[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i].v = *reinterpret_cast<const u32x4*>(base + i * 1024);
      if constexpr (MODE == 5) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x ^= f[i].v;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = mma16(acc[i], f[i], qb);
      }
    }
    r = __uint_as_float(x[0] ^ x[1] ^ x[2] ^ x[3]);
#pragma unroll
    for (int i = 0; i < 8; ++i) r += acc[i][0];
    return r;
  }
  if constexpr (MODE == 0 || MODE == 1) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = x0 + 0.01f * i;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        x[i] = MODE == 0 ? __builtin_amdgcn_exp2f(-x[i]) : fmaf(x[i], 0.999f, 0.001f);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) r += x[i];
  } else {
    Frag8<bf16> ka, qb;
    ka.v = u32x4{0x3f803f80u ^ (uint32_t)tid, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    qb.v = u32x4{0x3c003c00u, 0x3c003c00u ^ (uint32_t)tid, 0x3c003c00u, 0x3c003c00u};
    f32x4 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    SoftmaxState st;
#pragma unroll
    for (int j = 0; j < 4; ++j) st.s[j] = f32x4{x0, x0 + 1.f, x0 + 2.f, x0 + 3.f};
    st.m_run = 4.f;
    st.l_run = 0.f;
    for (int it = 0; it < iters; ++it) {
      if constexpr (MODE == 3 || MODE == 4) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = mma16(acc[i], ka, qb);
      }
      if constexpr (MODE == 2 || MODE == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) touch(st.s[j]);
        Frag8<bf16> pf[2];
        softmax_tile(st, 0.18033688f, pf);
        use(pf[0].v);
        use(pf[1].v);
      }
      if constexpr (MODE == 3 || MODE == 4) {
#pragma unroll
        for (int i = 8; i < 16; ++i) acc[i] = mma16(acc[i], ka, qb);
      }
    }
    r = st.l_run + st.m_run;
#pragma unroll
    for (int i = 0; i < 16; ++i) r += acc[i][0];
  }
  return r;
}

__global__ __launch_bounds__(256) void probe_kernel(int mode, int iters, float* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) char lds[16384];
  if (mode >= 5) {
    // every byte written before it is read
    for (int i = threadIdx.x; i < 1024; i += 256)
      reinterpret_cast<u32x4*>(lds)[i] = u32x4{0x3f803f80u ^ (uint32_t)i, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    __syncthreads();
  }
  float r;
  switch (mode) {
    case 0: r = probe_body<0>(iters, lds); break;
    case 1: r = probe_body<1>(iters, lds); break;
    case 2: r = probe_body<2>(iters, lds); break;
    case 3: r = probe_body<3>(iters, lds); break;
    case 4: r = probe_body<4>(iters, lds); break;
    case 5: r = probe_body<5>(iters, lds); break;
    default: r = probe_body<6>(iters, lds); break;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

hipError_t launch_probe(int mode, int workgroups, int iters, float* sink, hipStream_t stream) {
  probe_kernel<<<workgroups, 256, 0, stream>>>(mode, iters, sink);
  return hipGetLastError();
}

}  // namespace rs
