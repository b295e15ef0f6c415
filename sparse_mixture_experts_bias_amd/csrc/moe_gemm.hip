// moe_gemm.hip - grouped expert GEMM for gfx950 (the gather_qmm pattern).
//
// One launch applies a stack of expert weight matrices to activation rows that
// are grouped by expert (the sorted slots of the permutation), plus optionally
// one more segment for the shared expert.  Two epilogues:
//   GATEUP: h = silu(clamp(gate z + b_g)) * clamp(up z + b_u)  (SwiGLU, w1 = gate,
//           w3 = up of ferrox-models latent_moe.rs; the swiglu_limit clamp of
//           libmir-metal's gate/up kernel, read as a clamp of both to [-L, L])
//   LINEAR: o = W a + b (+ an f32 residual)      (down projections, latent maps)
//
// Work unit = (m-chunk of up to 64 rows of one segment, block of output columns).
// A 256-thread workgroup (4 waves) stages the chunk's activation rows in LDS,
// 256 reduction elements at a time; every wave streams its own weight rows
// straight from HBM into registers, dequantises them there, and feeds
// v_mfma_f32_16x16x32_{bf16,f16} (tokens = A operand, weight rows = B operand).
//
// Weight formats (see moe_linear in include/moe.h):
//   AFFINE4 (mlxcel issue #974's affine gather_qmm plane): a nibble q becomes the
//     16-bit value MAGIC+q by OR-ing it into the mantissa of MAGIC (128 in bf16,
//     1024 in f16); that is exact, so each MFMA over one quantisation group sums
//     (MAGIC+q)*a exactly-rounded in fp32, and the group is folded in fp32 as
//       acc += scale * S_g + (qbias - MAGIC*scale) * sum_g(a)
//     which equals sum (scale*q + qbias)*a without rounding the weights.
//     The nibble pairs come out as (q_i, q_{i+4}), so the activation rows are
//     staged with the matching element order inside every 8-element block.
//   MXFP4 (libmir-metal ExpertLayout blocks/scales): gfx950's scaled FP4
//     conversion turns E2M1 codes times the block's 2^(e-127) into bf16/f16
//     exactly; the block scale is applied in that conversion.
//   DENSE bf16: used as is (converted to f16 when the activations are f16).
#include "moe_kernels.h"

namespace {

template <int AT>
MOE_DEV f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (AT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// 8 nibbles (element i in bits 4i..4i+3) -> 4 words holding (MAGIC+q_i, MAGIC+q_{i+4}), i = 0..3
template <int AT>
MOE_DEV u32x4_t cvt_affine(uint32_t w) {
  constexpr uint32_t M = (AT == DT_BF16) ? 0x43004300u : 0x64006400u;
  u32x4_t r;
  r[0] = (w & 0x000F000Fu) | M;
  r[1] = ((w >> 4) & 0x000F000Fu) | M;
  r[2] = ((w >> 8) & 0x000F000Fu) | M;
  r[3] = ((w >> 12) & 0x000F000Fu) | M;
  return r;
}

// activation block (e0..e7) -> (e0,e4),(e1,e5),(e2,e6),(e3,e7): the order of cvt_affine
MOE_DEV u32x4_t pair_i_i4(u32x4_t v) {
  u32x4_t o;
  o[0] = (v[0] & 0xFFFFu) | (v[2] << 16);
  o[1] = (v[0] >> 16) | (v[2] & 0xFFFF0000u);
  o[2] = (v[1] & 0xFFFFu) | (v[3] << 16);
  o[3] = (v[1] >> 16) | (v[3] & 0xFFFF0000u);
  return o;
}

// 8 E2M1 codes (two per byte, low nibble first) times a power-of-two scale
template <int AT>
MOE_DEV u32x4_t cvt_mxfp4(uint32_t w, float scale) {
  u32x4_t r;
  if constexpr (AT == DT_BF16) {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  } else {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, scale, 3));
  }
  return r;
}

MOE_DEV float e8m0_to_f32(uint32_t e) {
  return e == 0u ? __uint_as_float(0x00400000u) : (e == 255u ? __uint_as_float(0x7FC00000u) : __uint_as_float(e << 23));
}

template <int AT>
MOE_DEV u32x4_t cvt_dense(u32x4_t w) {
  if constexpr (AT == DT_BF16) {
    return w;
  } else {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 lo = (_Float16)__uint_as_float(w[i] << 16);
      const _Float16 hi = (_Float16)__uint_as_float(w[i] & 0xFFFF0000u);
      r[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    return r;
  }
}

}  // namespace

template <int AT, int WF, int GS, bool GATEUP, int OT>
__global__ __launch_bounds__(MOE_GEMM_THREADS, 2) void expert_gemm(const GemmParams p) {
  constexpr bool AFF = (WF == WF_AFFINE4);
  constexpr bool MX = (WF == WF_MXFP4);
  constexpr bool DENSE = (WF == WF_DENSE);
  constexpr int KC = DENSE ? 128 : MOE_KC;       // reduction elements per staged chunk
  constexpr int STEPS = KC / 32;                 // MFMA k-steps per chunk
  constexpr int NU = STEPS / GS;                 // units (GS steps each) per chunk
  constexpr int WPS = DENSE ? 4 : 1;             // weight words per lane per step
  constexpr int NW = STEPS * WPS;                // weight words per lane per subtile per chunk
  constexpr int BPR = KC / 8;                    // 8-element blocks per chunk row
  constexpr int RPI = MOE_GEMM_THREADS / BPR;    // rows staged per iteration
  constexpr int SIT = MOE_MC / RPI;              // staging iterations per chunk
  constexpr int LDA = KC + 8;                    // padded LDS row (16-bit elements)
  constexpr float MAGIC = (AT == DT_BF16) ? 128.0f : 1024.0f;
  __shared__ __attribute__((aligned(16))) uint16_t sA[MOE_MC * LDA];
  __shared__ __attribute__((aligned(16))) float sX[AFF ? NU : 1][MOE_MC];
  __shared__ int64_t sRow[MOE_MC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kb = lane >> 4;
  const int sblk = tid % BPR, srow0 = tid / BPR;  // this thread's staging block / first row

  int nr_routed, nr_shared;
  if (p.tiles) {
    nr_routed = p.tile_count[0];
    nr_shared = p.tile_count[1];
  } else {
    nr_routed = 0;
    nr_shared = (p.plain_rows + MOE_MC - 1) / MOE_MC;
  }
  const int units_r = nr_routed * p.seg[0].nblk;
  const int total = units_r + nr_shared * p.seg[1].nblk;

  for (int u = blockIdx.x; u < total; u += gridDim.x) {
    const bool sh = u >= units_r;
    int ti, nb;
    if (!sh) {
      ti = u / p.seg[0].nblk;
      nb = u - ti * p.seg[0].nblk;
    } else {
      const int v = u - units_r;
      const int q = v / p.seg[1].nblk;
      nb = v - q * p.seg[1].nblk;
      ti = nr_routed + q;
    }
    int4 tile;
    if (p.tiles)
      tile = p.tiles[ti];
    else
      tile = make_int4(p.E, ti * MOE_MC, min(MOE_MC, p.plain_rows - ti * MOE_MC), 0);
    const int e = sh ? 0 : tile.x;
    const int r0 = tile.y, nr = tile.z;

#define SF(f) (sh ? p.seg[1].f : p.seg[0].f)
    const uint16_t *Ab = (const uint16_t *)SF(A.a);
    const int64_t lda = SF(A.lda);
    const int32_t *gat = SF(A.gather);
    const int gdiv = SF(A.gdiv), rsub = SF(A.row_sub);
    const int Kd = SF(K);
    const float limit = SF(limit);
    const WMat W0 = sh ? p.seg[1].w0 : p.seg[0].w0;
    const WMat W1 = GATEUP ? (sh ? p.seg[1].w1 : p.seg[0].w1) : W0;
#undef SF

    int rowb[2];
    bool act[2];
    if constexpr (GATEUP) {
      const int c0 = nb * 64 + wave * 16;
      rowb[0] = rowb[1] = c0;
      act[0] = act[1] = c0 < W0.rows;
    } else {
      const int c0 = nb * 128 + wave * 32;
      rowb[0] = c0;
      rowb[1] = c0 + 16;
      act[0] = c0 < W0.rows;
      act[1] = c0 + 16 < W0.rows;
    }
    const uint32_t *wrow[2];
    const uint16_t *srow[2];
    const uint16_t *qrow[2];
    const uint8_t *erow[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const WMat &M = b ? W1 : W0;
      const int64_t row = act[b] ? rowb[b] + r16 : 0;
      wrow[b] = (const uint32_t *)((const char *)M.w + (int64_t)e * M.w_stride + row * M.ldw);
      srow[b] = AFF ? (const uint16_t *)M.scales + (int64_t)e * M.s_stride + row * M.lds : nullptr;
      qrow[b] = AFF ? (const uint16_t *)M.qbias + (int64_t)e * M.s_stride + row * M.lds : nullptr;
      erow[b] = MX ? (const uint8_t *)M.scales + (int64_t)e * M.s_stride + row * M.lds : nullptr;
    }
    const int n_mt = (nr + 15) >> 4;
    const int nchunks = (Kd + KC - 1) / KC;

    // where each of the unit's activation rows starts
    __syncthreads();  // the previous unit is done with sRow / sA
    if (tid < nr) {
      const int64_t arow = gat ? (int64_t)(gat[r0 + tid] / gdiv) : (int64_t)(r0 + tid - rsub);
      sRow[tid] = arow * lda;
    }
    __syncthreads();

    // ---- loaders (raw bits only: nothing here waits for the loads)
    u32x4_t areg[SIT];
    auto load_a = [&](int kc) {
      const int kn = min(KC, Kd - kc);
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int row = srow0 + RPI * it;
        areg[it] = u32x4_t{0u, 0u, 0u, 0u};
        if (row < nr && sblk * 8 < kn) areg[it] = *(const u32x4_t *)(Ab + sRow[row] + kc + sblk * 8);
      }
    };
    uint32_t wcur[2][NW], wnxt[2][NW];
    uint32_t scur[2][NU], snxt[2][NU];  // AFF: scale bits; MX: e8m0 byte
    uint32_t qcur[2][NU], qnxt[2][NU];  // AFF: qbias bits
    auto load_w = [&](int kc, uint32_t (&w)[2][NW], uint32_t (&sr)[2][NU], uint32_t (&qr)[2][NU]) {
      const int nsteps = min(KC, Kd - kc) >> 5;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (!act[b]) continue;
#pragma unroll
        for (int uu = 0; uu < NU; ++uu) {
          if (uu * GS < nsteps) {
            if constexpr (DENSE) {
              const u32x4_t v = *(const u32x4_t *)(wrow[b] + ((kc + 32 * uu + 8 * kb) >> 1));
#pragma unroll
              for (int i = 0; i < 4; ++i) w[b][4 * uu + i] = v[i];
            } else {
              const int wi = ((kc + 32 * GS * uu) >> 3) + kb * GS;
              if constexpr (GS == 1) {
                w[b][uu] = wrow[b][wi];
              } else if constexpr (GS == 2) {
                const u32x2_t v = *(const u32x2_t *)(wrow[b] + wi);
                w[b][2 * uu] = v[0];
                w[b][2 * uu + 1] = v[1];
              } else {
                const u32x4_t v = *(const u32x4_t *)(wrow[b] + wi);
#pragma unroll
                for (int i = 0; i < 4; ++i) w[b][4 * uu + i] = v[i];
              }
              if constexpr (AFF) {
                const int g = (kc >> 5) / GS + uu;
                sr[b][uu] = srow[b][g];
                qr[b][uu] = qrow[b][g];
              } else {
                sr[b][uu] = erow[b][((kc + 64 * uu) >> 5) + (kb >> 1)];
              }
            }
          }
        }
      }
    };
    // activation chunk: registers -> LDS (affine: group sums + pair order)
    auto store_a = [&](int kc) {
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int row = srow0 + RPI * it;
        if (row < nr) {
          u32x4_t v = areg[it];
          if constexpr (AFF) {
            float f[8];
            unpack8<AT>(v, f);
            float s = ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
#pragma unroll
            for (int o = 1; o < 4 * GS; o <<= 1) s += __shfl_xor(s, o, 64);
            if ((sblk & (4 * GS - 1)) == 0) sX[sblk / (4 * GS)][row] = s;
            v = pair_i_i4(v);
          }
          *(u32x4_t *)&sA[row * LDA + sblk * 8] = v;
        }
      }
    };

    f32x4_t acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[mt][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load_a(0);
    load_w(0, wcur, scur, qcur);
    for (int c = 0; c < nchunks; ++c) {
      const int kc = c * KC;
      const int nsteps = min(KC, Kd - kc) >> 5;
      __syncthreads();  // readers of the previous chunk are done
      store_a(kc);
      if (c + 1 < nchunks) {  // next chunk in flight while this one computes
        load_a(kc + KC);
        load_w(kc + KC, wnxt, snxt, qnxt);
      }
      __syncthreads();

      if (act[0] || act[1]) {
#pragma unroll
        for (int uu = 0; uu < NU; ++uu) {
          if (uu * GS >= nsteps) break;
          float sc[2], qb[2];
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            if constexpr (AFF) {
              sc[b] = bf16_bits_to_f32(scur[b][uu]);
              qb[b] = bf16_bits_to_f32(qcur[b][uu]);
            } else if constexpr (MX) {
              sc[b] = e8m0_to_f32(scur[b][uu]);
            }
          }
          f32x4_t accg[4][2];
#pragma unroll
          for (int s = 0; s < GS; ++s) {
            const int q = uu * GS + s;
            u32x4_t bf[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              if constexpr (AFF)
                bf[b] = cvt_affine<AT>(wcur[b][q]);
              else if constexpr (MX)
                bf[b] = cvt_mxfp4<AT>(wcur[b][q], sc[b]);
              else
                bf[b] = cvt_dense<AT>(u32x4_t{wcur[b][4 * q], wcur[b][4 * q + 1], wcur[b][4 * q + 2], wcur[b][4 * q + 3]});
            }
            const int blk8 = uu * 4 * GS + kb * GS + s;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
              if (mt < n_mt) {
                const u32x4_t av = *(const u32x4_t *)&sA[(mt * 16 + r16) * LDA + blk8 * 8];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                  if (act[b]) {
                    if constexpr (AFF)
                      accg[mt][b] = mfma16<AT>(av, bf[b], s == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : accg[mt][b]);
                    else
                      acc[mt][b] = mfma16<AT>(av, bf[b], acc[mt][b]);
                  }
                }
              }
            }
          }
          if constexpr (AFF) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
              if (mt < n_mt) {
                const f32x4_t xs = *(const f32x4_t *)&sX[uu][mt * 16 + 4 * kb];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                  if (act[b]) {
                    const float c_ = fmaf(-MAGIC, sc[b], qb[b]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                      acc[mt][b][i] = fmaf(sc[b], accg[mt][b][i], fmaf(c_, xs[i], acc[mt][b][i]));
                  }
                }
              }
            }
          }
        }
      }
      if (c + 1 < nchunks) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
          for (int i = 0; i < NW; ++i) wcur[b][i] = wnxt[b][i];
#pragma unroll
          for (int i = 0; i < NU; ++i) {
            scur[b][i] = snxt[b][i];
            qcur[b][i] = qnxt[b][i];
          }
        }
      }
    }

    // ---- epilogue: acc[mt][b][i] is row mt*16 + 4*kb + i, column rowb[b] + r16
    if constexpr (GATEUP) {
      if (act[0]) {
        const int col = rowb[0] + r16;
        const float bg = W0.bias ? bf16_bits_to_f32(((const uint16_t *)W0.bias)[(int64_t)e * W0.rows + col]) : 0.f;
        const float bu = W1.bias ? bf16_bits_to_f32(((const uint16_t *)W1.bias)[(int64_t)e * W1.rows + col]) : 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (mt < n_mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = mt * 16 + 4 * kb + i;
              if (m < nr) {
                float g = acc[mt][0][i] + bg, v = acc[mt][1][i] + bu;
                if (limit > 0.f) {
                  g = fminf(fmaxf(g, -limit), limit);
                  v = fminf(fmaxf(v, -limit), limit);
                }
                store_act<OT>(p.out, (int64_t)(r0 + m) * p.ldo + col, silu_f(g) * v);
              }
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (!act[b]) continue;
        const int col = rowb[b] + r16;
        const float bo = W0.bias ? bf16_bits_to_f32(((const uint16_t *)W0.bias)[(int64_t)e * W0.rows + col]) : 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (mt < n_mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = mt * 16 + 4 * kb + i;
              if (m < nr) {
                float v = acc[mt][b][i] + bo;
                if (p.resid) v += p.resid[(int64_t)(r0 + m) * p.ldr + col];
                store_act<OT>(p.out, (int64_t)(r0 + m) * p.ldo + col, v);
              }
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// f32 path (f32 activations, DENSE F32 weights): one thread per output element,
// sequential fp32 dot products.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void f32_gemm_kernel(const F32GemmParams p) {
  const int r = blockIdx.x;
  const int c = blockIdx.y * 64 + threadIdx.x;
  const bool sh = r >= p.TK;
  if (c >= (sh ? p.ncols_s : p.ncols_r)) return;
  int e;
  const float *a;
  if (!sh) {
    const int slot = p.sorted_slot[r];
    e = p.topk_idx[slot];
    a = p.gateup ? p.a_routed + (int64_t)(slot / p.K) * p.lda_r : p.a_routed + (int64_t)r * p.lda_r;
  } else {
    e = 0;
    a = p.gateup ? p.a_shared + (int64_t)(r - p.TK) * p.lda_s : p.a_shared + (int64_t)r * p.lda_s;
  }
  const WMat &M0 = sh ? p.s0 : p.r0;
  const WMat &M1 = sh ? p.s1 : p.r1;
  const float *w0 = (const float *)((const char *)M0.w + (int64_t)e * M0.w_stride + (int64_t)c * M0.ldw);
  float v0 = 0.f;
  for (int k = 0; k < M0.cols; ++k) v0 = fmaf(a[k], w0[k], v0);
  if (M0.bias) v0 += ((const float *)M0.bias)[(int64_t)e * M0.rows + c];
  float out;
  if (p.gateup) {
    const float *w1 = (const float *)((const char *)M1.w + (int64_t)e * M1.w_stride + (int64_t)c * M1.ldw);
    float v1 = 0.f;
    for (int k = 0; k < M1.cols; ++k) v1 = fmaf(a[k], w1[k], v1);
    if (M1.bias) v1 += ((const float *)M1.bias)[(int64_t)e * M1.rows + c];
    if (p.limit > 0.f) {
      v0 = fminf(fmaxf(v0, -p.limit), p.limit);
      v1 = fminf(fmaxf(v1, -p.limit), p.limit);
    }
    out = v0 / (1.0f + expf(-v0)) * v1;
  } else {
    out = v0;
  }
  p.out[(int64_t)r * p.ldo + c] = out;
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
template <int AT, int WF, int GS, bool GU, int OT>
static hipError_t launch_t(const GemmParams &p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((expert_gemm<AT, WF, GS, GU, OT>), dim3(grid), dim3(MOE_GEMM_THREADS), 0, s, p);
  return hipGetLastError();
}

template <int AT, int WF, int GS>
static hipError_t launch_o(bool gateup, int odt, const GemmParams &p, int grid, hipStream_t s) {
  if (gateup) {
    if (odt == DT_BF16) return launch_t<AT, WF, GS, true, DT_BF16>(p, grid, s);
    if (odt == DT_F16) return launch_t<AT, WF, GS, true, DT_F16>(p, grid, s);
  } else {
    if (odt == DT_F32) return launch_t<AT, WF, GS, false, DT_F32>(p, grid, s);
    if (odt == DT_BF16) return launch_t<AT, WF, GS, false, DT_BF16>(p, grid, s);
    if (odt == DT_F16) return launch_t<AT, WF, GS, false, DT_F16>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int AT>
static hipError_t launch_w(int wfmt, int group, bool gateup, int odt, const GemmParams &p, int grid, hipStream_t s) {
  if (wfmt == WF_DENSE) return launch_o<AT, WF_DENSE, 1>(gateup, odt, p, grid, s);
  if (wfmt == WF_MXFP4) return launch_o<AT, WF_MXFP4, 2>(gateup, odt, p, grid, s);
  if (wfmt == WF_AFFINE4) {
    if (group == 32) return launch_o<AT, WF_AFFINE4, 1>(gateup, odt, p, grid, s);
    if (group == 64) return launch_o<AT, WF_AFFINE4, 2>(gateup, odt, p, grid, s);
    if (group == 128) return launch_o<AT, WF_AFFINE4, 4>(gateup, odt, p, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_expert_gemm(int adt, int wfmt, int group, bool gateup, int odt, const GemmParams &p, int grid,
                              hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (adt == DT_BF16) return launch_w<DT_BF16>(wfmt, group, gateup, odt, p, grid, s);
  if (adt == DT_F16) return launch_w<DT_F16>(wfmt, group, gateup, odt, p, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_f32_gemm(const F32GemmParams &p, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int cols = p.ncols_r > p.ncols_s ? p.ncols_r : p.ncols_s;
  hipLaunchKernelGGL(f32_gemm_kernel, dim3(rows, (cols + 63) / 64), dim3(64), 0, s, p);
  return hipGetLastError();
}
