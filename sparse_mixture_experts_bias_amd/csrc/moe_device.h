// moe_device.h - device-side types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV static __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// storage type tags
enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
// weight format tags
// WF_MXS: MXFP4 in the stream of the block-scaled FP4 x FP8 MFMA (moe_pack_weights_scaled)
enum { WF_DENSE = 0, WF_AFFINE4 = 1, WF_MXFP4 = 2, WF_MXS = 3 };

MOE_DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
MOE_DEV float f16_bits_to_f32(uint32_t b) {
  union { uint16_t u; _Float16 h; } c;
  c.u = (uint16_t)b;
  return (float)c.h;
}

// load one stored activation element as float
template <int DT>
MOE_DEV float load_act(const void *p, int64_t i) {
  if constexpr (DT == DT_F32) return ((const float *)p)[i];
  else if constexpr (DT == DT_BF16) return bf16_bits_to_f32(((const uint16_t *)p)[i]);
  else return f16_bits_to_f32(((const uint16_t *)p)[i]);
}

// store a float in a storage type (round to nearest even)
template <int DT>
MOE_DEV void store_act(void *p, int64_t i, float v) {
  if constexpr (DT == DT_F32) ((float *)p)[i] = v;
  else if constexpr (DT == DT_BF16) ((__bf16 *)p)[i] = (__bf16)v;
  else ((_Float16 *)p)[i] = (_Float16)v;
}

// 8 packed 16-bit elements (bf16 or f16) -> 8 floats
template <int DT>
MOE_DEV void unpack8(u32x4_t v, float *f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == DT_BF16) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    } else {
      f[2 * i] = f16_bits_to_f32(v[i] & 0xFFFFu);
      f[2 * i + 1] = f16_bits_to_f32(v[i] >> 16);
    }
  }
}

MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// silu(g) = g * sigmoid(g); the reciprocal is the hardware one (1 ulp), the result is stored in 16 bits
// the SwiGLU clamp of a pre-activation to [-lim, lim]; NaN stays NaN (fminf / fmaxf alone
// would return the bound)
MOE_DEV float clamp_act(float v, float lim) { return __builtin_isnan(v) ? v : fminf(fmaxf(v, -lim), lim); }
MOE_DEV float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
