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

template <int ODT, int YDT, int NT>
__global__ __launch_bounds__(NT) void combine_kernel(const CombineArgs a) {
  constexpr int CMB_COLS = 8 * NT;  // columns per block pass
  __shared__ int pos[MOE_MAX_TOPK];
  __shared__ float wt[MOE_MAX_TOPK];
  __shared__ float red[NT / 64];
  const int t = blockIdx.x, tid = threadIdx.x;
  // token-ordered rows (no slot_pos: row t*K + j): the row loads need nothing from memory
  // first, and the weights come through the scalar cache beside them; otherwise the slot
  // positions and weights go through LDS before the row loads
  const bool direct = a.slot_pos == nullptr;
  if (!direct) {
    if (tid < a.K) {
      pos[tid] = a.slot_pos[(int64_t)t * a.K + tid];
      wt[tid] = a.topk_w[(int64_t)t * a.K + tid];
    }
    __syncthreads();
  }
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
      for (int jj = 0; jj < CMB_JB; ++jj) {
        const int j = min(j0 + jj, a.K - 1);
        load8<ODT>(a.o, (direct ? (int64_t)t * a.K + j : (int64_t)pos[j]) * a.ldo + c, f[jj]);
      }
#pragma unroll
      for (int jj = 0; jj < CMB_JB; ++jj) {
        if (j0 + jj < a.K) {
          const float w = direct ? a.topk_w[(int64_t)t * a.K + j0 + jj] : wt[j0 + jj];
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
  for (int w = 0; w < NT / 64; ++w) tot += red[w];
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

// a few tokens (decode): 64-thread blocks over 512 columns each, so that the rows spread over
// four times the CUs; otherwise (and for the rms norm, which needs a whole row per block) 256
template <int ODT, int YDT>
static hipError_t launch_c(const CombineArgs &a, hipStream_t s) {
  if (a.mode != 1 && a.T <= 64) {
    const int ncb = (a.D + 8 * 64 - 1) / (8 * 64);
    hipLaunchKernelGGL((combine_kernel<ODT, YDT, 64>), dim3(a.T, ncb), dim3(64), 0, s, a);
  } else {
    const int ncb = (a.D + CMB_COLS - 1) / CMB_COLS;
    const int gy = (a.mode == 1) ? 1 : ncb;
    hipLaunchKernelGGL((combine_kernel<ODT, YDT, CMB_T>), dim3(a.T, gy), dim3(CMB_T), 0, s, a);
  }
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

// ---------------------------------------------------------------------------
// split_fp8: f16 activations -> the FP8 operand pair of the block-scaled MFMA.
// Per row and block of 32 elements: hi = e4m3(v / 2^Eh) with the smallest Eh that keeps the
// block's largest magnitude within e4m3's 448, then the remainder r = v - hi * 2^Eh (exact in
// fp32) as lo = e4m3(r / 2^El) with El chosen the same way from r.  hi * 2^Eh + lo * 2^El keeps
// about 8 significant bits of every element (more than bf16's), and each of the two products
// with the weights carries its own E8M0 block scale, so the pair costs two MFMAs where the
// weights need no conversion at all.
// Output: hl [rows][cols / 128][256 bytes]: per 128 elements the 128 hi codes, then the 128 lo
// codes (the row stride is cols * 2 bytes, that of the f16 input rows); hs [rows][cols / 32]:
// Eh + 127 | (El + 127) << 8.  cols % 128 == 0.
// ---------------------------------------------------------------------------
static __device__ __forceinline__ int e8m0_for(float amax) {
  if (!(amax > 0.f)) return 127;  // an all-zero block (and NaN: out of contract)
  int x;
  const float m = frexpf(amax, &x);  // amax = m 2^x, m in [0.5, 1); 448 = 0.875 2^9
  const int E = m <= 0.875f ? x - 9 : x - 8;
  return min(max(E + 127, 1), 254);
}

// 2^(127 - e) for e in 1..254
static __device__ __forceinline__ float inv_pow2(int e) { return __uint_as_float((uint32_t)(254 - e) << 23); }
static __device__ __forceinline__ float pow2(int e) { return __uint_as_float((uint32_t)e << 23); }

// OCP E4M3 (bias 7, 3 mantissa bits, no infinities, largest finite 448), written out from the
// format: y with |y| <= 448 rounded to nearest even; returns the code and the rounded value.
// Below 2^-6 the codes are the subnormals q 2^-9 (q = 0..8, 8 being the smallest normal).
static __device__ __forceinline__ uint32_t e4m3_rne(float y, float &yr) {
  const uint32_t sgn = __float_as_uint(y) >> 31 << 7;
  const float a = fabsf(y);
  if (!(a <= 448.0f)) {  // NaN (nothing larger reaches here): the e4m3 NaN code, so it propagates
    yr = y;
    return 0x7Fu | sgn;
  }
  uint32_t code;
  float r;
  if (a < 0.015625f) {
    const float q = rintf(a * 512.0f);  // 0..8, ties to even
    code = (uint32_t)q;
    r = q * (1.0f / 512.0f);
  } else {
    uint32_t bits = __float_as_uint(a);
    bits += 0x7FFFFu + ((bits >> 20) & 1u);  // round the mantissa to 3 bits, ties to even
    bits &= 0xFFF00000u;
    r = __uint_as_float(bits);
    code = ((((bits >> 23) - 120u) << 3) | ((bits >> 20) & 7u));
  }
  yr = sgn ? -r : r;
  return code | sgn;
}

__global__ __launch_bounds__(256) void split_fp8_kernel(const uint16_t *in, int64_t ldi, int rows, int cols,
                                                        uint8_t *hl, uint16_t *hs) {
  const int nb = cols / 32;
  const int64_t total = (int64_t)rows * nb;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(i / nb), b = (int)(i % nb);
    const f16x8_t *src = (const f16x8_t *)(in + (int64_t)r * ldi + 32 * b);
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f16x8_t h = src[q];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[8 * q + j] = (float)h[j];
    }
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(v[k]));
    const int eh = e8m0_for(amax);
    const float ih = inv_pow2(eh), ph = pow2(eh);
    uint32_t hw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u}, lw[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    float ramax = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      float yr;
      hw[k / 4] |= e4m3_rne(v[k] * ih, yr) << (8 * (k % 4));
      v[k] -= yr * ph;  // exact: both terms carry at most 11 significant bits at nearby scales
      ramax = fmaxf(ramax, fabsf(v[k]));
    }
    const int el = e8m0_for(ramax);
    const float il = inv_pow2(el);
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      float yr;
      lw[k / 4] |= e4m3_rne(v[k] * il, yr) << (8 * (k % 4));
    }
    uint8_t *dst = hl + (int64_t)r * cols * 2 + (b >> 2) * 256 + (b & 3) * 32;
    *(u32x4_t *)dst = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
    *(u32x4_t *)(dst + 16) = u32x4_t{hw[4], hw[5], hw[6], hw[7]};
    *(u32x4_t *)(dst + 128) = u32x4_t{lw[0], lw[1], lw[2], lw[3]};
    *(u32x4_t *)(dst + 144) = u32x4_t{lw[4], lw[5], lw[6], lw[7]};
    hs[(int64_t)r * nb + b] = (uint16_t)(eh | (el << 8));
  }
}

hipError_t launch_split_fp8(const void *in, int64_t ldi, int rows, int cols, void *hl, uint16_t *hs, hipStream_t s) {
  const int64_t total = (int64_t)rows * (cols / 32);
  if (total <= 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 16384 ? want : 16384);
  hipLaunchKernelGGL(split_fp8_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t *)in, ldi, rows, cols,
                     (uint8_t *)hl, hs);
  return hipGetLastError();
}

// bf16 -> f16, 8 elements per thread (n a multiple of 8; both 16-byte aligned): the f16 copy of
// the block input that the prefill GEMMs read when the intermediates are f16.  Exact for
// magnitudes in f16's normal range (a bf16 mantissa fits in f16's); below it the f16
// subnormals round, above 65504 the result is inf.
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint32_t *in, uint32_t *out, int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const bf16x8_t v = *(const bf16x8_t *)(in + 4 * i);
    f16x8_t r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (_Float16)(float)v[j];
    *(f16x8_t *)(out + 4 * i) = r;
  }
}

hipError_t launch_bf16_to_f16(const void *in, void *out, int64_t n, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  const int64_t want = (n8 + 255) / 256;
  const int grid = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(bf16_to_f16_kernel, dim3(grid), dim3(256), 0, s, (const uint32_t *)in, (uint32_t *)out, n8);
  return hipGetLastError();
}
