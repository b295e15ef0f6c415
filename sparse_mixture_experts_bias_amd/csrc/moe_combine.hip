// moe_combine.hip - weighted combine of the per-slot expert outputs.
//
//   y_r[t] = sum_j w[t,j] * o[slot_pos[t*K+j]]   (j ascending, fp32; the combine
//            loop of ferrox-models kimi_latent_moe_forward)
//   mode 0: write y_r (f32)
//   mode 1: write rms_norm(y_r) * norm_w  (latent flow of latent_moe.rs, before up_proj)
//   mode 2: write y_r + shared            (shared expert added at weight 1)
//   mode 3: write c0*y_r + c1*shared      (mlxcel PR #1044 point 2: per-token blend)
// The shared expert's output sits in row TK + t of the same buffer.
#include "moe_kernels.h"

template <int DT>
MOE_DEV void load8(const void *base, int64_t i, float *f) {
  if constexpr (DT == DT_F32) {
    const f32x4_t a = *(const f32x4_t *)((const float *)base + i);
    const f32x4_t b = *(const f32x4_t *)((const float *)base + i + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[q] = a[q];
      f[q + 4] = b[q];
    }
  } else {
    unpack8<DT>(*(const u32x4_t *)((const uint16_t *)base + i), f);
  }
}

template <int DT>
MOE_DEV void store8(void *base, int64_t i, const float *f) {
  if constexpr (DT == DT_F32) {
    *(f32x4_t *)((float *)base + i) = f32x4_t{f[0], f[1], f[2], f[3]};
    *(f32x4_t *)((float *)base + i + 4) = f32x4_t{f[4], f[5], f[6], f[7]};
  } else {
    u32x4_t v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint16_t lo, hi;
      if constexpr (DT == DT_BF16) {
        lo = __builtin_bit_cast(uint16_t, (__bf16)f[2 * q]);
        hi = __builtin_bit_cast(uint16_t, (__bf16)f[2 * q + 1]);
      } else {
        lo = __builtin_bit_cast(uint16_t, (_Float16)f[2 * q]);
        hi = __builtin_bit_cast(uint16_t, (_Float16)f[2 * q + 1]);
      }
      v[q] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    *(u32x4_t *)((uint16_t *)base + i) = v;
  }
}

constexpr int CMB_T = 256;      // threads per block
constexpr int CMB_COLS = 8 * CMB_T;
constexpr int CMB_MAXIT = 4;    // rms-norm mode keeps up to 4*2048 columns in registers
constexpr int CMB_JB = 8;       // slot rows loaded together

template <int ODT, int YDT>
__global__ __launch_bounds__(CMB_T) void combine_kernel(const CombineArgs a) {
  __shared__ int pos[MOE_MAX_TOPK];
  __shared__ float wt[MOE_MAX_TOPK];
  __shared__ float red[CMB_T / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < a.K) {
    pos[tid] = a.slot_pos ? a.slot_pos[(int64_t)t * a.K + tid] : t * a.K + tid;
    wt[tid] = a.topk_w[(int64_t)t * a.K + tid];
  }
  __syncthreads();
  const int ncb = (a.D + CMB_COLS - 1) / CMB_COLS;
  float keep[CMB_MAXIT][8];
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < CMB_MAXIT; ++it) {
    const int cb = blockIdx.y + it * gridDim.y;
    if (cb >= ncb) break;
    const int c = cb * CMB_COLS + tid * 8;
    if (c >= a.D) continue;
    float s[8];
    if (a.mode >= 2) load8<ODT>(a.o, (int64_t)(a.TK + t) * a.ldo + c, s);  // in flight with the slot rows
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // slot rows in batches of CMB_JB, every load of a batch issued before the first FMA;
    // the sum still runs over j in ascending order
    for (int j0 = 0; j0 < a.K; j0 += CMB_JB) {
      float f[CMB_JB][8];
#pragma unroll
      for (int jj = 0; jj < CMB_JB; ++jj) load8<ODT>(a.o, (int64_t)pos[min(j0 + jj, a.K - 1)] * a.ldo + c, f[jj]);
#pragma unroll
      for (int jj = 0; jj < CMB_JB; ++jj) {
        if (j0 + jj < a.K) {
          const float w = wt[j0 + jj];
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = fmaf(w, f[jj][q], v[q]);
        }
      }
    }
    if (a.mode == 1) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        keep[it][q] = v[q];
        ss = fmaf(v[q], v[q], ss);
      }
      continue;
    }
    if (a.mode >= 2) {
      if (a.mode == 2) {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] += s[q];
      } else {
        const float c0 = a.coef[2 * t], c1 = a.coef[2 * t + 1];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = fmaf(c0, v[q], c1 * s[q]);
      }
    }
    store8<YDT>(a.y, (int64_t)t * a.ldy + c, v);
  }
  if (a.mode != 1) return;
  // rms norm over the whole row (gridDim.y == 1)
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < CMB_T / 64; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)a.D + a.eps);
#pragma unroll
  for (int it = 0; it < CMB_MAXIT; ++it) {
    const int c = it * CMB_COLS + tid * 8;
    if (it >= ncb || c >= a.D) break;
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = keep[it][q] * inv * (a.norm_w ? a.norm_w[c + q] : 1.0f);
    store8<YDT>(a.y, (int64_t)t * a.ldy + c, v);
  }
}

template <int ODT, int YDT>
static hipError_t launch_c(const CombineArgs &a, hipStream_t s) {
  const int ncb = (a.D + CMB_COLS - 1) / CMB_COLS;
  const int gy = (a.mode == 1) ? 1 : ncb;
  hipLaunchKernelGGL((combine_kernel<ODT, YDT>), dim3(a.T, gy), dim3(CMB_T), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(int odt, int ydt, const CombineArgs &a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
#define C(O, Y) \
  if (odt == O && ydt == Y) return launch_c<O, Y>(a, s);
  C(DT_F32, DT_F32)
  C(DT_F32, DT_BF16)
  C(DT_BF16, DT_F32)
  C(DT_BF16, DT_BF16)
  C(DT_BF16, DT_F16)
  C(DT_F16, DT_F32)
  C(DT_F16, DT_BF16)
  C(DT_F16, DT_F16)
#undef C
  return hipErrorInvalidValue;
}
