// The MLP sublayer of a block in one kernel, for widths C <= 384 in bf16: LayerNorm 2,
// fc1 + GELU, fc2, the residual x_hat = x' + MLP(LN(x')) (Eq. (6) of "Representation
// Shift: Unifying Token Compression with FlashAttention", arXiv HTML, Sec. 3.3) and the
// per-token partial sums of the representation shift of Eq. (4) (Sec. 3.2), by default
// || MLP(LN(x')) - x' ||_2.  The hidden activations never leave registers: a workgroup
// owns 128 token rows, and for each 32-unit slice of the hidden layer its waves compute
// that slice of GELU(LN(x') W1^T + b1) for their rows and multiply it into full-width fc2
// accumulators.  Neither the hidden activations nor a LayerNorm-2 operand are written to
// memory.
//
// Work split.  8 waves (two per SIMD), each owning 16 token rows.  A wave keeps
//   - LN(x') of its rows as the fc1 B operand, bf16, for the whole kernel (C / 8 VGPRs),
//   - the fc2 accumulators of its rows over all C outputs, fp32 (C / 4 registers),
// and per hidden slice reads the slice's W1 rows and W2 columns from LDS, where the
// workgroup stages them with direct global -> LDS loads.  The loop is software-pipelined
// over the slices: iteration c runs fc2 of slice c (its GELU output already in registers)
// and fc1 + GELU of slice c + 1, two independent streams of matrix and vector work, so
// one unit holds slice c + 1's W1 rows and slice c's W2 columns; unit c + 1 loads into
// the other of two LDS buffers while unit c is read.  One barrier per slice.
//
// Register layouts (mma16: lane l holds column l % 16 of B and of D, k-group l / 16):
//   fc1: D1[hidden][token] = W1s (A, 16 hidden x 32 k) * LN(x')^T (B, 32 k x 16 tokens).
//        Lane (token j = l % 16, g = l / 16) receives hidden rows 4g .. 4g + 3 of a
//        16-row tile.  The slice's W1 rows are staged permuted: staged row 16 t + 4 g' + r
//        holds hidden unit 8 g' + 4 t + r of the slice, so after tiles t = 0, 1 lane g
//        holds hidden units 8 g .. 8 g + 7 -- exactly the B-operand k-slots of group g of
//        a 32-k step of fc2.  The GELU output feeds fc2 straight from registers.
//   fc2: D2[out][token] = W2s (A, 16 outputs x 32 hidden) * h^T (B).  The W2 rows
//        (output columns) are staged permuted the same way, so lane g ends up with output
//        columns 32 J + 8 g .. 32 J + 8 g + 7 of every 32-column group J: the epilogue
//        reads x, p and writes x_hat in 16-byte pieces, and lanes g = 0..3 of a token
//        together cover 64-column slices for the slice partials.
// Every staged fragment block is 1 KiB in lane order (lane l's 16 bytes at 16 l), so the
// fragment reads are contiguous and bank-conflict free; each direct load fills one block.
#include "rs_device.hpp"
#include "rs_launch.hpp"

namespace rs {
namespace {

constexpr int kMlpWaves = 8, kMlpRows = 128, kMlpSlice = 32;
constexpr int kMlpMaxHidden = 4096;   // b1 is kept in LDS (8 KiB)

// The GELU of the bf16 path (same form and constants as the fc1 epilogue of rs_gemm.hip):
// x Phi(x) = max(x, 0) - |x| Q(|x|), Q = 1 - Phi evaluated as 2^R(t), R a fitted degree-4
// polynomial in t = min(|x|, 13).  Max |error| against the erf form 6.2e-6.
__device__ __forceinline__ float mlp_gelu(float x) {
  const float ax = fabsf(x);
  const float t = fminf(ax, 13.0f);
  float p = fmaf(t, 3.865753533318639e-03f, -4.4075679033994675e-02f);
  p = fmaf(p, t, -4.6802330017089844e-01f);
  p = fmaf(p, t, -1.1473647356033325f);
  p = fmaf(p, t, -1.0004818439483643f);
  const float q = __builtin_amdgcn_exp2f(p);
  return fmaf(-ax, q, fmaxf(x, 0.0f));
}

// Sum over the token's 4 lanes (lanes i, i ^ 16, i ^ 32, i ^ 48) as the tree
// (v0 + v1) + (v2 + v3), with v_g the value of lane group g: the order in which the row
// statistics kernel combines the 8-column chunk sums of a 64-column slice, so the slice
// partials written here equal the ones it computes from the stored rows bit for bit.
// permlane16_swap pairs groups g, g ^ 1; permlane32_swap then pairs g, g ^ 2.
__device__ __forceinline__ float sum_groups(float v) {
#if __HIP_DEVICE_COMPILE__
  const unsigned u = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const unsigned w = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
#else
  return v;
#endif
}

__device__ __forceinline__ Frag8<bf16> lds_frag(const char* p) {
  Frag8<bf16> f;
  f.v = *reinterpret_cast<const u32x4*>(p);
  return f;
}

// EPI: 0 = the method's score, sum (y - x')^2 of the MLP-sublayer shift; 1 = any of the
// distances and the whole-block shift (runtime choice).
template <int NKS, int EPI>
__global__ __launch_bounds__(kMlpWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mlp_kernel(MlpArgs a, int M, int Hd) {
  constexpr int C = NKS * 32;          // width; NKS = 32-element k steps of fc1
  constexpr int NT = C / 16;           // 16-column output tiles (W2 fragment blocks)
  constexpr int NJ = C / 32;           // 32-column output groups
  constexpr int W1B = 2 * NKS * 1024;  // staged W1 rows of a slice: (k step, tile) blocks
  constexpr int UNITB = W1B + NT * 1024;
  constexpr int NLOAD = 4 * NKS / kMlpWaves;   // fragment blocks each wave loads per unit
  static_assert(NT * 1024 == W1B && (4 * NKS) % kMlpWaves == 0, "unit staging layout");
  __shared__ __attribute__((aligned(16))) char smem[3 * UNITB + kMlpMaxHidden * 2 + C * 2];   // + b1, b2

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int m = blockIdx.x * kMlpRows + wave * 16 + l16;   // this lane's token row
  const bool ok = m < M;
  const size_t mc = (size_t)min(m, M - 1);
  const bf16* x = static_cast<const bf16*>(a.x);
  const bf16* p = static_cast<const bf16*>(a.p);
  const int NC = Hd / kMlpSlice;

  // ---- staging.  Unit c (LDS buffer c % 3): fragment blocks u < 2 NKS hold slice c + 2's
  // W1 rows (k step u / 2, row tile u % 2), blocks 2 NKS + j slice c's W2 columns for
  // output tile j.  Block u of a slice is 1 KiB of the packed weights (lane l's MFMA
  // operand at 16 l), so each direct load copies 1 KiB of consecutive bytes.  Waves 0-3
  // load the W1 blocks, waves 4-7 the W2 blocks.  The W1 blocks of the last two units name
  // slices past the end; they are clamped to the last slice (loaded, so every unit is the
  // same NLOAD loads per wave, and read by fc1 work whose results are not used).
  const bool w1side = wave < kMlpWaves / 2;
  const char* gbase = static_cast<const char*>(a.wpack) + (size_t)wave * NLOAD * 1024 + lane * 16;
  auto stage = [&](int sc, char* lds_base) {
    const char* gs = gbase + (size_t)min(sc, NC - 1) * UNITB;
    char* ls = lds_base + wave * NLOAD * 1024;
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) load_lds16(gs + j * 1024, ls + j * 1024);
  };
  auto bufp = [&](int c) { return (c % 3) * UNITB; };
  auto stage_unit = [&](int c) { stage(w1side ? c + 2 : c, smem + bufp(c)); };

  // Prologue loads, in the order they are needed: slices 0 and 1's W1 rows (W1 waves, into
  // buffer 2), this lane's x and p (LayerNorm 2), b1 / b2 for the LDS tables; units 0 and
  // 1 after the LayerNorm (the compiler waits for every earlier load before the first use
  // of x, so loads issued before it would all be waited for).
  if (w1side) {
    stage(0, smem + 2 * UNITB);
    stage(1, smem + 2 * UNITB + W1B);
  }
  Frag8<bf16> fx[NKS], fp[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    load_frag(fx[s], x + mc * C + 32 * s + 8 * g);
    load_frag(fp[s], p + mc * C + 32 * s + 8 * g);
  }
  char* btab = smem + 3 * UNITB;
  char* b2tab = btab + Hd * 2;
  const int ntab = Hd / 8 + C / 8;                       // 16-byte pieces of b1 then b2
  const int ti = threadIdx.x;                            // one piece per thread (ntab <= 560)
  u32x4 tv = u32x4{0u, 0u, 0u, 0u};
  if (ti < ntab)
    tv = ti < Hd / 8 ? *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.b1) + ti * 8)
                     : *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.b2) + (ti - Hd / 8) * 8);
  u32x4 tv2 = u32x4{0u, 0u, 0u, 0u};
  const int ti2 = ti + kMlpWaves * 64;
  if (ti2 < ntab)
    tv2 = ti2 < Hd / 8 ? *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.b1) + ti2 * 8)
                       : *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.b2) + (ti2 - Hd / 8) * 8);

  // ---- LayerNorm 2 of x' = x + p (Eq. (5)), exact two-pass statistics in fp32 over the
  // row (each token's row is spread over its 4 lanes g = 0..3), one rounding to bf16 of
  // the normalised, affine row: the fc1 B operand for k-step s, k-group g.
  Frag8<bf16> xb[NKS];
  {
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      float u[8], v[8];
      frag_to_f32(fx[s], u);
      frag_to_f32(fp[s], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += u[e] + v[e];
    }
    const float mean = sum_rows(sum) * (1.0f / C);
    float m2 = 0.f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      float u[8], v[8];
      frag_to_f32(fx[s], u);
      frag_to_f32(fp[s], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = (u[e] + v[e]) - mean;
        m2 = fmaf(d, d, m2);
      }
    }
    const float rstd = __builtin_amdgcn_rsqf(fmaf(sum_rows(m2), 1.0f / C, a.eps));
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      float u[8], v[8], gm[8], bt[8], o[8];
      frag_to_f32(fx[s], u);
      frag_to_f32(fp[s], v);
      load8f(static_cast<const bf16*>(a.ln_g) + 32 * s + 8 * g, gm);
      load8f(static_cast<const bf16*>(a.ln_b) + 32 * s + 8 * g, bt);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(((u[e] + v[e]) - mean) * rstd, gm[e], bt[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) xb[s].v[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
    }
  }
  if (ti < ntab) *reinterpret_cast<u32x4*>(btab + ti * 16) = tv;   // b1 then b2, contiguous
  if (ti2 < ntab) *reinterpret_cast<u32x4*>(btab + ti2 * 16) = tv2;
  stage_unit(0);
  stage_unit(1);
  __builtin_amdgcn_sched_barrier(0);

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const char* lb = smem + lane * 16;
  const char* bl = btab + 16 * g;         // + 64 sc: this lane's 8 b1 values of slice sc
  auto b1_of = [&](int sc, float* bv) { frag_to_f32(lds_frag(bl + min(sc, NC - 1) * kMlpSlice * 2), bv); };

  // fc1 of one slice alone, from the W1 blocks at `w1s` (prologue)
  auto fc1 = [&](const char* w1s, f32x4& h0, f32x4& h1) {
    h0 = h1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      h0 = mma16(h0, lds_frag(w1s + (2 * s) * 1024), xb[s]);
      h1 = mma16(h1, lds_frag(w1s + (2 * s + 1) * 1024), xb[s]);
    }
  };

  // Pipeline: iteration c runs fc2 of slice c, GELU of slice c + 1 and fc1 of slice
  // c + 2 -- three independent streams -- reading unit c (W1 of c + 2, W2 of c), while
  // units c + 1 and c + 2 load.  The last two iterations run on clamped slices whose fc1
  // and GELU results are not used, so every iteration is the same pinned sequence.
  Frag8<bf16> hbuf;                       // GELU output of slice c: the fc2 B operand
  f32x4 hp0, hp1;                         // fc1 of slice c + 1 (no bias)
  wait_vmem<2 * NLOAD>();                 // W1 waves: slices 0 and 1 staged (units 0, 1 may not be)
  // the b1 / b2 table writes done, then every wave (no fence: __syncthreads() would also
  // wait for units 0 and 1)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  {
    f32x4 t0, t1;
    fc1(lb + 2 * UNITB, t0, t1);
    float bv[8];
    b1_of(0, bv);
    hbuf.v[0] = pack_bf16x2(mlp_gelu(t0[0] + bv[0]), mlp_gelu(t0[1] + bv[1]));
    hbuf.v[1] = pack_bf16x2(mlp_gelu(t0[2] + bv[2]), mlp_gelu(t0[3] + bv[3]));
    hbuf.v[2] = pack_bf16x2(mlp_gelu(t1[0] + bv[4]), mlp_gelu(t1[1] + bv[5]));
    hbuf.v[3] = pack_bf16x2(mlp_gelu(t1[2] + bv[6]), mlp_gelu(t1[3] + bv[7]));
    fc1(lb + 2 * UNITB + W1B, hp0, hp1);  // slice 1's fc1
  }

  // One iteration's matrix work as one straight sequence of 4 NKS slots, each one fragment
  // read from LDS and one product with it: even slots are fc1 of slice c + 2 (step q / 4,
  // tile (q / 2) % 2), odd slots fc2 of slice c (output tile q / 2).  Each slot's fragment
  // is read kDepth slots ahead, and the GELU of slice c + 1 is spread over the slots.
  // Scheduling barriers between slots keep that order: left to itself the compiler moves
  // each fragment read next to its product, and the wave then waits on LDS at almost every
  // product.  The next unit's loads are issued after the slots (direct-to-LDS loads issued
  // among the fragment reads make the compiler wait for every outstanding LDS read at each
  // product).
  constexpr int NQ = 4 * NKS, kDepth = 6;
  for (int c = 0; c < NC; ++c) {
    // this wave's blocks of unit c have landed (unit c + 1, if there is one, may not)
    if (c + 1 < NC) wait_vmem<NLOAD>(); else wait_vmem<0>();
    barrier_nofence();   // ... and every wave's; unit c - 1's buffer is no longer read
    const char* us = lb + bufp(c);
    auto faddr = [&](int q) { return us + ((q & 1) ? W1B + (q >> 1) * 1024 : (q >> 1) * 1024); };
    f32x4 h0 = f32x4{0.f, 0.f, 0.f, 0.f}, h1 = h0;
    float gl[8], gv[8];
    {
      float bv[8];
      b1_of(c + 1, bv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gl[e] = hp0[e] + bv[e];
        gl[4 + e] = hp1[e] + bv[4 + e];
      }
    }
    Frag8<bf16> f[kDepth];
#pragma unroll
    for (int q = 0; q < kDepth; ++q) f[q] = lds_frag(faddr(q));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const Frag8<bf16> cur = f[q % kDepth];
      if (q + kDepth < NQ) f[q % kDepth] = lds_frag(faddr(q + kDepth));
      if (q & 1) {
        acc[q >> 1] = mma16(acc[q >> 1], cur, hbuf);
      } else if ((q >> 1) & 1) {
        h1 = mma16(h1, cur, xb[q >> 2]);
      } else {
        h0 = mma16(h0, cur, xb[q >> 2]);
      }
      // GELU element i at slots spread evenly over the iteration
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((i * NQ) / 8 == q) gv[i] = mlp_gelu(gl[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) hbuf.v[e] = pack_bf16x2(gv[2 * e], gv[2 * e + 1]);
    hp0 = h0;
    hp1 = h1;
    // into the buffer unit c - 1 used; units past the last are not loaded (the epilogue's
    // row loads would otherwise wait for them: loads complete in issue order)
    if (c + 2 < NC) stage_unit(c + 2);
  }

  // ---- epilogue: acc[2 J + t][r] = y - b2 of row m, output column 32 J + 8 g + 4 t + r.
  // y = MLP(LN(x')); x' = x + p re-formed in fp32; x_hat = x' + y stored; the shift
  // partials and the stored row's statistics per 64-column slice (J = 2 sl, 2 sl + 1),
  // summed over the token's 4 lanes.  x and p of slice sl + 2 are requested before slice sl
  // is computed.
  const int nsl = C / 64, sstride = stat_stride(C);
  bf16* out = static_cast<bf16*>(a.out);
  Frag8<bf16> ex[3][2], epp[3][2];        // [buffer][J within the slice]
  auto load_slice = [&](int sl, int b) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int n = 64 * sl + 32 * h2 + 8 * g;
      load_frag(ex[b][h2], x + mc * C + n);
      load_frag(epp[b][h2], p + mc * C + n);
    }
  };
  load_slice(0, 0);
  if (1 < nsl) load_slice(1, 1);
#pragma unroll
  for (int sl = 0; sl < nsl; ++sl) {
    if (sl + 2 < nsl) load_slice(sl + 2, (sl + 2) % 3);
    float w[16], s0 = 0.f, s1 = 0.f, s2 = 0.f, cs[2] = {0.f, 0.f};
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int J = 2 * sl + h2, n = 32 * J + 8 * g;
      float xv[8], pv[8], bb[8];
      frag_to_f32(ex[sl % 3][h2], xv);
      frag_to_f32(epp[sl % 3][h2], pv);
      frag_to_f32(lds_frag(b2tab + n * 2), bb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = acc[2 * J + (e >> 2)][e & 3] + bb[e];   // MLP(LN(x'))
        const float xp = xv[e] + pv[e];                          // x' (Eq. (5)) in fp32
        w[8 * h2 + e] = round_t<bf16>(xp + y);                   // x_hat (Eq. (6)), as stored
        cs[h2] += w[8 * h2 + e];                                 // this 8-column chunk's sum
        if (EPI == 0) {
          const float d = y - xp;
          s0 = fmaf(d, d, s0);
        } else {
          const float fa = a.shift_block ? xp + y : y;            // x_hat | MLP(LN(x'))
          const float fb = a.shift_block ? xv[e] : xp;            // x     | x'
          if (a.dist == 0) {
            s0 = fmaf(fa - fb, fa - fb, s0);
          } else if (a.dist == 1) {
            s0 += fabsf(fa - fb);
          } else {
            s0 = fmaf(fa, fb, s0);
            s1 = fmaf(fa, fa, s1);
            s2 = fmaf(fb, fb, s2);
          }
        }
      }
      if (ok) store8f(out + mc * C + n, w + 8 * h2);
    }
    if (a.stats_out) {
      // slice statistics of the stored row in the row statistics kernel's order:
      // sequential within each 8-column chunk (chunk g of J = 2 sl, chunk 4 + g of
      // J = 2 sl + 1), then ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7))
      const float smean = (sum_groups(cs[0]) + sum_groups(cs[1])) * (1.0f / 64.0f);
      float cm[2] = {0.f, 0.f};
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = w[8 * h2 + e] - smean;
          cm[h2] = fmaf(d, d, cm[h2]);
        }
      const float sm2 = sum_groups(cm[0]) + sum_groups(cm[1]);
      if (ok && g == 0) {
        float* so = a.stats_out + (mc * sstride + sl) * 2;
        so[0] = smean;
        so[1] = sm2;
      }
    }
    if (a.part) {
      s0 = sum_groups(s0);
      if (EPI == 1 && a.dist == 2) {
        s1 = sum_groups(s1);
        s2 = sum_groups(s2);
      }
      if (ok && g == 0) {
        float* pr = a.part + mc * a.pstride + sl;
        pr[0] = s0;
        if (EPI == 1 && a.dist == 2) {
          pr[a.nparts] = s1;
          pr[2 * a.nparts] = s2;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // two slices' loads ahead, not all of them
  }
  // partial slots past the last 64-column slice (the score reads nparts per quantity)
  if (a.part && ok && g == 0) {
    for (int q = 0; q < (a.dist == 2 ? 3 : 1); ++q)
      for (int sl = nsl; sl < a.nparts; ++sl) a.part[mc * a.pstride + q * a.nparts + sl] = 0.f;
  }
  wait_vmem<0>();
}

// Packing of W1 / W2 into the fused kernel's fragment order: 16-byte chunk i of a block's
// packed weights is lane (i % 64) of fragment block (i / 64) % (4 NKS) of slice
// i / (256 NKS) (the order the kernel stages, see above).
struct MlpPackArgs {
  MlpPackJob job[kMaxPackJobs];
  int njobs, C, Hd;
};
__global__ __launch_bounds__(256) void mlp_pack_kernel(MlpPackArgs pa) {
  const int C = pa.C, Hd = pa.Hd, nks = C / 32;
  const size_t per_job = (size_t)C * Hd / 4;   // 16-byte chunks per block
  const size_t id = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= per_job * pa.njobs) return;
  const MlpPackJob& jb = pa.job[id / per_job];
  const size_t i = id % per_job;
  const int per_slice = 256 * nks;                // chunks per slice: 4 NKS blocks of 64
  const int sc = (int)(i / per_slice), rem = (int)(i % per_slice);
  const int u = rem >> 6, lane = rem & 63, l16 = lane & 15, g = lane >> 4;
  const int prow = 8 * (l16 >> 2) + (l16 & 3);
  const bf16* src;
  if (u < 2 * nks) {
    const int s = u >> 1, t = u & 1;
    src = static_cast<const bf16*>(jb.w1) + (size_t)(sc * kMlpSlice + prow + 4 * t) * C + 32 * s + 8 * g;
  } else {
    const int v = u - 2 * nks;
    src = static_cast<const bf16*>(jb.w2) + (size_t)(32 * (v >> 1) + prow + 4 * (v & 1)) * Hd +
          sc * kMlpSlice + 8 * g;
  }
  *reinterpret_cast<u32x4*>(static_cast<char*>(jb.out) + i * 16) = *reinterpret_cast<const u32x4*>(src);
}

template <int NKS>
hipError_t launch_nks(const MlpArgs& a, int M, int hidden, hipStream_t st) {
  const int grid = (M + kMlpRows - 1) / kMlpRows;
  if (a.part && (a.dist != 0 || a.shift_block))
    mlp_kernel<NKS, 1><<<grid, kMlpWaves * 64, 0, st>>>(a, M, hidden);
  else
    mlp_kernel<NKS, 0><<<grid, kMlpWaves * 64, 0, st>>>(a, M, hidden);
  return hipGetLastError();
}

}  // namespace

bool mlp_fused_supported(Dtype dt, int C, int hidden) {
  return dt == kBF16 && C >= 64 && C <= kMlpMaxWidth && C % 64 == 0 && hidden >= 2 * kMlpSlice &&
         hidden <= kMlpMaxHidden && hidden % kMlpSlice == 0;
}

hipError_t launch_mlp_pack(const MlpPackJob* jobs, int njobs, int C, int hidden, hipStream_t st) {
  if (njobs < 1 || njobs > kMaxPackJobs || !mlp_fused_supported(kBF16, C, hidden)) return hipErrorInvalidValue;
  MlpPackArgs pa;
  for (int j = 0; j < njobs; ++j) pa.job[j] = jobs[j];
  pa.njobs = njobs;
  pa.C = C;
  pa.Hd = hidden;
  const size_t chunks = (size_t)C * hidden / 4 * njobs;
  mlp_pack_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, st>>>(pa);
  return hipGetLastError();
}

hipError_t launch_mlp(Dtype dt, const MlpArgs& a, int M, int C, int hidden, hipStream_t st) {
  if (!mlp_fused_supported(dt, C, hidden)) return hipErrorInvalidValue;
  if (M <= 0) return hipSuccess;
  switch (C / 64) {
    case 1: return launch_nks<2>(a, M, hidden, st);
    case 2: return launch_nks<4>(a, M, hidden, st);
    case 3: return launch_nks<6>(a, M, hidden, st);
    case 4: return launch_nks<8>(a, M, hidden, st);
    case 5: return launch_nks<10>(a, M, hidden, st);
    case 6: return launch_nks<12>(a, M, hidden, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace rs
