// The two linear layers of the attention sublayer for widths C <= 384 in bf16, weights
// streamed through LDS: the QKV projection with LayerNorm 1 applied in the kernel (Eq. (5)
// of "Representation Shift: Unifying Token Compression with FlashAttention", arXiv HTML,
// Sec. 3.3, feeds LN(x) to self-attention, whose queries, keys and values are linear maps
// of its input, Sec. 3.1 Eq. (1)), and the attention output projection (the term Eq. (5)
// adds to x).
//
// out[m][n] = A'[m] . W'[n] + b'[n].  QKV: A' = (x - mean) * rstd of the row, from the
// slice partials its producer wrote, rounded once to bf16; W' = W diag(gamma1) and
// b' = b + W beta1 (fp32) come from the LayerNorm fold pass, so LN(x) W^T + b is computed.
// Projection: A' = the row, W' = W, b' = b.  A workgroup of 4 waves owns 128 rows; each
// wave keeps its 32 rows (two 16-row groups) as MFMA B operands in registers (C / 4 VGPRs)
// and walks its range of the N outputs in slices of 32, whose W' rows the workgroup stages
// in LDS from the packed copy: staged row 16 t + 4 g' + r of a slice holds output
// 8 g' + 4 t + r, so lane group g ends with outputs 8 g .. 8 g + 7 and stores them as one
// 16-byte piece.  Each fragment read from LDS feeds the products of both row groups.
// Three 24 KiB units at C = 384 (slice c is read while c + 1 and c + 2 load) and a 6 KiB
// bias table leave room for two workgroups per CU.
#include "rs_device.hpp"
#include "rs_launch.hpp"

namespace rs {
namespace {

constexpr int kLinWaves = 4, kLinRG = 2, kLinRows = kLinWaves * 16 * kLinRG, kLinSlice = 32;
#ifndef RS_LIN_TARGET
#define RS_LIN_TARGET 192
#endif
#ifndef RS_LIN_XCD
#define RS_LIN_XCD 0
#endif
#ifndef RS_LIN_MIN_SLICES
#define RS_LIN_MIN_SLICES 4
#endif
// Measured (encoder step, three bf16 workloads): 192 beats 128, 256, 320 and 384 by
// 0.4-0.8 %; the encoder's other lane fills the CUs a launch leaves.
constexpr int kLinTargetGroups = RS_LIN_TARGET;
constexpr int kLinMinSlices = RS_LIN_MIN_SLICES;

__device__ __forceinline__ Frag8<bf16> lin_frag(const char* p) {
  Frag8<bf16> f;
  f.v = *reinterpret_cast<const u32x4*>(p);
  return f;
}

template <int NKS, bool LN>
__global__ __launch_bounds__(kLinWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void lin_kernel(LinArgs a, int M, int N, int NSW) {
  constexpr int C = NKS * 32;                  // K
  constexpr int UNITB = 2 * NKS * 1024;        // one slice's W rows: (k step, tile) blocks
  constexpr int NLOAD = 2 * NKS / kLinWaves;   // blocks each wave loads per unit
  constexpr int NT = (kLinMaxN / 4 + kLinWaves * 64 - 1) / (kLinWaves * 64);   // bias pieces
  static_assert((2 * NKS) % kLinWaves == 0, "unit staging layout");
  __shared__ __attribute__((aligned(16))) char smem[3 * UNITB + kLinMaxN * 4];   // + bias

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const bf16* A = static_cast<const bf16*>(a.a);
  // this workgroup's row block and output slices s0 .. s0 + NSW - 1 of the N / 32
#if RS_LIN_XCD
  const int nsplit = N / kLinSlice / NSW;
  const int lid = xcd_contiguous(blockIdx.x, gridDim.x);
  const int rb = lid / nsplit, s0 = (lid % nsplit) * NSW;
#else
  const int rb = blockIdx.x, s0 = blockIdx.y * NSW;
#endif
  int mrow[kLinRG];                            // this lane's rows (clamped for loads)
  bool ok[kLinRG];
#pragma unroll
  for (int r = 0; r < kLinRG; ++r) {
    const int m = rb * kLinRows + wave * 16 * kLinRG + 16 * r + l16;
    ok[r] = m < M;
    mrow[r] = min(m, M - 1);
  }

  // staging: unit c (buffer c % 3) = slice c's W rows, NLOAD 1 KiB blocks per wave;
  // slices past the end are clamped (loaded, never read) so every unit is NLOAD loads
  const char* gbase = static_cast<const char*>(a.wpack) + (size_t)s0 * UNITB +
                      (size_t)wave * NLOAD * 1024 + lane * 16;
  auto stage = [&](int sc) {
    const char* gs = gbase + (size_t)min(sc, NSW - 1) * UNITB;
    char* ls = smem + (sc % 3) * UNITB + wave * NLOAD * 1024;
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) load_lds16(gs + j * 1024, ls + j * 1024);
  };
  // Units 0 and 1 first: the row loads below are younger, so the compiler's wait for
  // them covers these too, and the two streams overlap.
  stage(0);
  stage(1);

  // rows of A as B operands: row group r, k step s, k group g
  Frag8<bf16> xb[kLinRG][NKS];
#pragma unroll
  for (int r = 0; r < kLinRG; ++r)
#pragma unroll
    for (int s = 0; s < NKS; ++s) load_frag(xb[r][s], A + (size_t)mrow[r] * C + 32 * s + 8 * g);
  // LN: the rows' slice partials (mean, M2 of each 64-column slice)
  constexpr int SST = stat_stride(C), NSL = stat_slices(C);
  f32x4 sp[kLinRG][SST / 2];
  if constexpr (LN) {
#pragma unroll
    for (int r = 0; r < kLinRG; ++r)
#pragma unroll
      for (int q = 0; q < SST / 2; ++q)
        sp[r][q] = *reinterpret_cast<const f32x4*>(a.stats + ((size_t)mrow[r] * SST + 2 * q) * 2);
  }
  // bias table in LDS, fp32 [N]: LN the folded bias (fp32), else the layer's bias (bf16)
  char* btab = smem + 3 * UNITB;
  {
    u32x4 tv[NT];
    const int ntab = LN ? N / 4 : N / 8;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = threadIdx.x + i * kLinWaves * 64;
      if (t < ntab)
        tv[i] = LN ? *reinterpret_cast<const u32x4*>(a.bias_f + t * 4)
                   : *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.bias) + t * 8);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = threadIdx.x + i * kLinWaves * 64;
      if (t < ntab) {
        if (LN) {
          *reinterpret_cast<u32x4*>(btab + t * 16) = tv[i];
        } else {
          Frag8<bf16> f;
          f.v = tv[i];
          float v[8];
          frag_to_f32(f, v);
          *reinterpret_cast<f32x4*>(btab + t * 32) = f32x4{v[0], v[1], v[2], v[3]};
          *reinterpret_cast<f32x4*>(btab + t * 32 + 16) = f32x4{v[4], v[5], v[6], v[7]};
        }
      }
    }
  }
  if constexpr (LN) {
    // LayerNorm 1 with gamma folded into W and beta into the bias: the operand is
    // (x - mean) * rstd, rounded once to bf16.  mean and the biased variance merged from
    // the slice partials (equal counts of 64).
#pragma unroll
    for (int r = 0; r < kLinRG; ++r) {
      float mp[SST], m2p[SST];
#pragma unroll
      for (int q = 0; q < SST / 2; ++q) {
        mp[2 * q] = sp[r][q][0]; m2p[2 * q] = sp[r][q][1];
        mp[2 * q + 1] = sp[r][q][2]; m2p[2 * q + 1] = sp[r][q][3];
      }
      float mean = 0.f;
#pragma unroll
      for (int q = 0; q < NSL; ++q) mean += mp[q];
      mean *= 1.0f / NSL;
      float m2 = 0.f;
#pragma unroll
      for (int q = 0; q < NSL; ++q) {
        const float dm = mp[q] - mean;
        m2 += m2p[q] + 64.f * dm * dm;
      }
      const float rstd = __builtin_amdgcn_rsqf(fmaf(m2, 1.0f / C, a.eps));
      const float mr = -mean * rstd;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        float u[8];
        frag_to_f32(xb[r][s], u);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          xb[r][s].v[e] = pack_bf16x2(fmaf(u[2 * e], rstd, mr), fmaf(u[2 * e + 1], rstd, mr));
      }
    }
  }
  const char* lb = smem + lane * 16;
  const char* bl = btab + 32 * g + 128 * s0;  // + 128 c: this lane's 8 bias values of slice c
  bf16* out = static_cast<bf16*>(a.out) + s0 * kLinSlice;

  // One slice as 2 NKS slots, each one fragment read and the products of both row groups
  // with it (k step q / 2, tile q % 2: four accumulation chains, each used every fourth
  // product).  Fragments are read kDepth slots ahead and scheduling barriers keep the
  // order: left alone, the compiler moves each read next to its product.  The previous
  // slice's outputs are stored in the second slot, after this slice's first reads.
  //
  // Waits: unit c's loads were issued before slice c - 1's stores and unit c + 1's loads,
  // so at most NLOAD outstanding vector-memory operations (loads complete in issue order)
  // means unit c has landed in this wave's share, whether or not the stores were issued;
  // the barrier then makes every wave's share visible.
  constexpr int NQ = 2 * NKS, kDepth = 6;
  u32x4 pk[kLinRG];                            // slice c - 1's outputs, stored in slice c
  int pc = -1;
  for (int c = 0; c < NSW; ++c) {
    wait_vmem<NLOAD>();
    if (c == 0)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // + the bias table
    else
      barrier_nofence();
    const char* us = lb + (c % 3) * UNITB;
    f32x4 acc[kLinRG][2];
#pragma unroll
    for (int r = 0; r < kLinRG; ++r) acc[r][0] = acc[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frag8<bf16> f[kDepth];
#pragma unroll
    for (int q = 0; q < kDepth; ++q) f[q] = lin_frag(us + q * 1024);
    const f32x4 bv0 = *reinterpret_cast<const f32x4*>(bl + c * 128);
    const f32x4 bv1 = *reinterpret_cast<const f32x4*>(bl + c * 128 + 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const Frag8<bf16> cur = f[q % kDepth];
      if (q + kDepth < NQ) f[q % kDepth] = lin_frag(us + (q + kDepth) * 1024);
#pragma unroll
      for (int r = 0; r < kLinRG; ++r) acc[r][q & 1] = mma16(acc[r][q & 1], cur, xb[r][q >> 1]);
      if (q == 1 && pc >= 0) {
#pragma unroll
        for (int r = 0; r < kLinRG; ++r)
          if (ok[r]) *reinterpret_cast<u32x4*>(out + (size_t)mrow[r] * a.ldo + pc * kLinSlice + 8 * g) = pk[r];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // outputs 32 c + 8 g + e (e = 4 t + j) of each row, + bias, packed for the next slice
    const float bv[8] = {bv0[0], bv0[1], bv0[2], bv0[3], bv1[0], bv1[1], bv1[2], bv1[3]};
#pragma unroll
    for (int r = 0; r < kLinRG; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pk[r][e] = pack_bf16x2(acc[r][e >> 1][(2 * e) & 3] + bv[2 * e],
                               acc[r][e >> 1][(2 * e + 1) & 3] + bv[2 * e + 1]);
    pc = c;
    stage(c + 2);
  }
#pragma unroll
  for (int r = 0; r < kLinRG; ++r)
    if (ok[r]) *reinterpret_cast<u32x4*>(out + (size_t)mrow[r] * a.ldo + pc * kLinSlice + 8 * g) = pk[r];
  wait_vmem<0>();   // the clamped units' direct-to-LDS loads have landed before the LDS is freed
}

template <int NKS>
hipError_t launch_lin_nks(const LinArgs& a, int M, int N, hipStream_t st) {
  // Rows alone give M / 128 workgroups, too few to fill the chip at most token counts;
  // the N outputs are split into contiguous slice ranges as well (each range re-reads and
  // re-normalises its rows), the fewest ranges that reach kLinTargetGroups workgroups,
  // keeping at least kLinMinSlices slices per range.
  const int rows = (M + kLinRows - 1) / kLinRows, ns = N / kLinSlice;
  int split = 1;
  for (int d = 1; d <= ns; ++d) {
    if (ns % d != 0 || ns / d < kLinMinSlices) continue;
    split = d;
    if ((long)rows * d >= kLinTargetGroups) break;
  }
#if RS_LIN_XCD
  const dim3 grid(rows * split);
#else
  const dim3 grid(rows, split);
#endif
  if (a.stats)
    lin_kernel<NKS, true><<<grid, kLinWaves * 64, 0, st>>>(a, M, N, ns / split);
  else
    lin_kernel<NKS, false><<<grid, kLinWaves * 64, 0, st>>>(a, M, N, ns / split);
  return hipGetLastError();
}

}  // namespace

bool lin_supported(Dtype dt, int K, int N) {
  return dt == kBF16 && K >= 64 && K <= kMlpMaxWidth && K % 64 == 0 && N % kLinSlice == 0 &&
         N >= kLinSlice && N <= kLinMaxN;
}

hipError_t launch_lin(Dtype dt, const LinArgs& a, int M, int K, int N, hipStream_t st) {
  if (!lin_supported(dt, K, N) || a.ldo < N) return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  switch (K / 64) {
    case 1: return launch_lin_nks<2>(a, M, N, st);
    case 2: return launch_lin_nks<4>(a, M, N, st);
    case 3: return launch_lin_nks<6>(a, M, N, st);
    case 4: return launch_lin_nks<8>(a, M, N, st);
    case 5: return launch_lin_nks<10>(a, M, N, st);
    case 6: return launch_lin_nks<12>(a, M, N, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace rs
