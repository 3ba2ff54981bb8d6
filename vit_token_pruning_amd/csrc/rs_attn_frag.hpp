// Register and LDS fragment helpers shared by the two attention kernels (the fused one
// and the map-forming one): both compute S^T = K Q^T with one query per lane and take the
// P V product as O^T = V^T P^T, V read column-wise from row-major LDS tiles.
#pragma once
#include "rs_device.hpp"

namespace rs {
namespace attn {

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
// 4-7), kb = 32 kc + 4 g.  bf16 V rows are 128 bytes with swizzled 16-byte chunks.
__device__ __forceinline__ const char* vt_addr(const char* Vs, int row, int d) {
  const int c = d >> 3;                          // 16-byte chunk of element d
  return Vs + row * 128 + ((c ^ (row & 7)) << 4) + ((d & 7) << 1);
}
__device__ __forceinline__ void load_vt(Frag8<bf16>& f, const char* Vs, int kb, int d0, int l16) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const int row = kb + (l16 >> 2), d = d0 + 4 * (l16 & 3);
  const char* pa = vt_addr(Vs, row, d);
  const char* pb = vt_addr(Vs, row + 16, d);
#if __HIP_DEVICE_COMPILE__
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pa));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(pb));
#else
  const v4i16 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
#endif
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  f.v = u32x4{ua[0], ua[1], ub[0], ub[1]};
}
// fp32: padded rows of ROWBV bytes, no swizzle
template <int ROWBV>
__device__ __forceinline__ void load_vt_f32(Frag8<float>& f, const char* Vs, int kb, int d0, int l16) {
  float* e = reinterpret_cast<float*>(&f);
  const char* col = Vs + (d0 + l16) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[i] = *reinterpret_cast<const float*>(col + (kb + i) * ROWBV);
    e[4 + i] = *reinterpret_cast<const float*>(col + (kb + 16 + i) * ROWBV);
  }
}

}  // namespace attn
}  // namespace rs
