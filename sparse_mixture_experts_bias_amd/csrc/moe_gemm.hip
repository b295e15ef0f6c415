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

// 32x32x16 MFMA: lane l holds A[m = l%32][k = 8*(l/32) .. +8), B[k = 8*(l/32) .. +8][n = l%32]
// and D[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32], i = 0..15.
template <int AT>
MOE_DEV f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (AT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// Work unit: (m-chunk of up to 32 rows of one segment, block of output columns).
// Every wave owns one 32-row weight tile (GATEUP: 16 gate rows and the 16 up rows of
// the same columns; LINEAR: 32 output rows).  Tokens are the MFMA's A operand and
// weight rows its B operand, so every lane of a tile holds a single weight row.
//
// Weight stream: per chunk each tile row contributes one contiguous 128-byte
// segment; a wave fetches its 4 KB with 16-byte loads, 8 lanes per row (whole
// cache lines, no partial requests), two chunks ahead of the MFMAs, and writes them
// into its own LDS tile with the 16-byte blocks of each row XOR-swizzled so that
// the MFMA-layout reads (32 rows, same column) spread over the banks.
// Scales/qbias (AFFINE4) or E8M0 exponents (MXFP4) of the tile's rows are copied
// to LDS once per unit with contiguous loads.
//
// Reduction order inside a weight row: a "unit" of UE elements is split between
// the two half-waves (UE/2 contiguous elements each); MFMA step s of the unit uses
// elements [s*8, s*8+8) of each half.  For AFFINE4 a unit is one quantisation
// group, so each step stays inside one group and the exact fold applies per group.
template <int AT, int WF, int GQ, bool GATEUP, int OT>
__global__ __launch_bounds__(MOE_GEMM_THREADS, 3) void expert_gemm(const GemmParams p) {
  constexpr bool AFF = (WF == WF_AFFINE4);
  constexpr bool MX = (WF == WF_MXFP4);
  constexpr bool DENSE = (WF == WF_DENSE);
  constexpr int UE = AFF ? GQ : (MX ? 64 : 32);            // elements per unit (both halves)
  constexpr int SPU = UE / 16;                             // MFMA steps per unit
  constexpr int LB = DENSE ? UE : UE / 4;                  // bytes per lane per unit
  constexpr int KC = DENSE ? 64 : MOE_KC;                  // reduction elements per chunk (128 B per row)
  constexpr int NU = KC / UE;                              // units per chunk
  constexpr int BPR = KC / 8;                              // 8-element activation blocks per chunk row
  constexpr int RPI = MOE_GEMM_THREADS / BPR;              // activation rows staged per iteration
  constexpr int SIT = (MOE_MC + RPI - 1) / RPI;            // activation staging iterations
  constexpr int LDA = KC + 8;                              // padded LDS activation row (16-bit elements)
  constexpr float MAGIC = (AT == DT_BF16) ? 128.0f : 1024.0f;
  static_assert(MOE_MC == 32, "one 32-row m-tile per chunk");
  static_assert((DENSE ? KC * 2 : KC / 2) == 128, "128-byte row segments per chunk");
  __shared__ __attribute__((aligned(16))) uint16_t sA[MOE_MC * LDA];
  __shared__ int64_t sRow[MOE_MC];
  extern __shared__ __attribute__((aligned(16))) char dyn[];  // per wave: weight tile + scale strip

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, kb = lane >> 5;
  const int sblk = tid % BPR, srow0 = tid / BPR;
  char *wlds = dyn + wave * p.wave_lds;                    // 32 x 128 B weight tile
  char *slds = wlds + 4096;                                // scale strip(s)

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

    // tile row t (0..31) -> weight matrix row; GATEUP: rows 0-15 gate, 16-31 up
    const int col0 = GATEUP ? nb * 64 + wave * 16 : nb * 128 + wave * 32;
    const bool act = col0 < W0.rows;
    auto row_of = [&](int t) { return GATEUP ? col0 + (t & 15) : col0 + t; };
    auto row_ok = [&](int t) { return row_of(t) < W0.rows; };
    auto mat_of = [&](int t) -> const WMat & { return (GATEUP && t >= 16) ? W1 : W0; };
    const int nchunks = (Kd + KC - 1) / KC;
    const int nib = min(4, (nr + 7) >> 3);       // 8-row blocks of the m-tile that hold rows

    // this lane's loader rows (tile rows 8*i + lane/8) and their segment base pointers
    const char *lrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 8 * i + (lane >> 3);
      const WMat &M = mat_of(t);
      const int64_t rr = row_ok(t) ? row_of(t) : 0;
      lrow[i] = (const char *)M.w + (int64_t)e * M.w_stride + rr * M.ldw + 16 * (lane & 7);
    }

    u32x4_t gA[4], gB[4], gC[4];  // weight ring: chunk c, c+1 in flight, c+2 being loaded
    auto load_w = [&](int kc, u32x4_t (&g)[4]) {
      const int kcc = min(kc, (nchunks - 1) * KC);
      const int64_t off = DENSE ? (int64_t)kcc * 2 : kcc / 2;
      // the last chunk may be shorter than 128 B per row: clamp the piece into the row
      const int rowbytes = DENSE ? Kd * 2 : Kd / 2;
      const int64_t o2 = min((int64_t)rowbytes - 16, off + 16 * (lane & 7)) - 16 * (lane & 7);
#pragma unroll
      for (int i = 0; i < 4; ++i) g[i] = *(const u32x4_t *)(lrow[i] + o2);
    };
    load_w(0, gA);  // in flight during the setup below
    load_w(KC, gB);

    __syncthreads();  // the previous unit is done with sRow / sA / the LDS tiles
    if (tid < nr) {
      const int64_t arow = gat ? (int64_t)(gat[r0 + tid] / gdiv) : (int64_t)(r0 + tid - rsub);
      sRow[tid] = arow * lda;
    }

    // ---- scale strips -> LDS (once per unit): AFF: [32][G] bf16 scales then [32][G] qbias;
    //      MX: [32][NB] e8m0 bytes.  Row t of a strip belongs to tile row t.
    if constexpr (AFF || MX) {
      const int G = AFF ? Kd / UE : Kd / 32;         // entries per row
      const int esz = AFF ? 2 : 1;
      const int rowb = G * esz;                      // bytes per strip row in LDS (unpadded)
      const int nstrip = AFF ? 2 : 1;
      // lanes walk the strip rows with 2-byte loads: lane -> (row offset, entry pair)
      const int EPR = (rowb + 1) / 2;                // 2-byte words per row
      int epp = 1;
      while (epp < EPR) epp <<= 1;                   // <= 64 (checked on the host)
      const int rps = 64 / epp;                      // rows per pass
      for (int sidx = 0; sidx < nstrip; ++sidx) {
        for (int t0 = 0; t0 < 32; t0 += 8 * rps) {
          uint16_t v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int t = t0 + i * rps + lane / epp;
            const int w = lane % epp;
            v[i] = 0;
            if (t < 32 && w < EPR) {
              const WMat &M = mat_of(t);
              const int64_t rr = row_ok(t) ? row_of(t) : 0;
              const uint16_t *src = (const uint16_t *)((const char *)(sidx ? M.qbias : M.scales) +
                                                       ((int64_t)e * M.s_stride + rr * M.lds) * esz);
              v[i] = (esz == 2 || (rowb & 1) == 0 || w < EPR - 1)
                         ? src[w]
                         : (uint16_t)((const uint8_t *)src)[2 * w];
            }
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int t = t0 + i * rps + lane / epp;
            const int w = lane % epp;
            if (t < 32 && w < EPR) *(uint16_t *)(slds + sidx * 32 * p.strip_row + t * p.strip_row + 2 * w) = v[i];
          }
        }
      }
    }
    __syncthreads();

    // ---- loaders: raw bits only; every call issues the same loads (addresses clamped
    // into valid memory) so the compiler can count them; out-of-chunk data is masked
    // when consumed.
    u32x4_t areg[SIT];
    uint32_t amask = 0;
    auto load_a = [&](int kc) {
      const int kcc = min(kc, (nchunks - 1) * KC);
      const int kn = min(KC, Kd - kcc);
      amask = 0;
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int row = srow0 + RPI * it;
        const bool ok = row < nr && sblk * 8 < kn && kc < Kd;
        amask |= ok ? (1u << it) : 0u;
        const int rr = row < nr ? row : 0;
        const int cc = sblk * 8 < kn ? sblk * 8 : 0;
        areg[it] = *(const u32x4_t *)(Ab + sRow[rr] + kcc + cc);
      }
    };
    auto put_w = [&](const u32x4_t (&g)[4]) {  // registers -> swizzled LDS tile
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 8 * i + (lane >> 3);
        const int pos = (lane & 7) ^ ((t >> 1) & 7);
        *(u32x4_t *)(wlds + t * 128 + 16 * pos) = g[i];
      }
    };
    auto store_a = [&]() {
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int row = srow0 + RPI * it;
        if (row < nr) {
          u32x4_t v = areg[it];
          if (!((amask >> it) & 1u)) v = u32x4_t{0u, 0u, 0u, 0u};
          if constexpr (AFF) v = pair_i_i4(v);
          *(u32x4_t *)&sA[row * LDA + sblk * 8] = v;
        }
      }
    };

    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;

    const char *my_w = wlds + r32 * 128;
    const int my_sw = (r32 >> 1) & 7;
    auto compute = [&](int kc) {
      if (!act) return;
      const int nunits = min(KC, Kd - kc) / UE;
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) {
        if (uu >= nunits) break;
        // this lane's LB bytes of the unit: byte offset (UE*uu + UE/2*kb) * bytes-per-element
        const int boff = DENSE ? (UE * uu + (UE / 2) * kb) * 2 : (UE * uu + (UE / 2) * kb) / 2;
        uint32_t wv[LB / 4];
        if constexpr (LB == 8) {
          const int blk = boff >> 4;
          const u32x2_t a = *(const u32x2_t *)(my_w + 16 * (blk ^ my_sw) + (boff & 15));
          wv[0] = a[0];
          wv[1] = a[1];
        } else {
#pragma unroll
          for (int h = 0; h < LB / 16; ++h) {
            const int blk = (boff >> 4) + h;
            const u32x4_t a = *(const u32x4_t *)(my_w + 16 * (blk ^ my_sw));
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[4 * h + i] = a[i];
          }
        }
        float sc = 0.f, qb = 0.f;
        if constexpr (AFF) {
          const int g = kc / UE + uu;
          sc = bf16_bits_to_f32(*(const uint16_t *)(slds + r32 * p.strip_row + 2 * g));
          qb = bf16_bits_to_f32(*(const uint16_t *)(slds + 32 * p.strip_row + r32 * p.strip_row + 2 * g));
        } else if constexpr (MX) {
          sc = e8m0_to_f32(*(const uint8_t *)(slds + r32 * p.strip_row + (kc >> 5) + 2 * uu + kb));
        }
        f32x16_t accg, accx;  // AFF: sum of (MAGIC+q)*a and of a over the unit (one group)
#pragma unroll
        for (int s = 0; s < SPU; ++s) {
          u32x4_t bfr;
          if constexpr (AFF)
            bfr = cvt_affine<AT>(wv[s]);
          else if constexpr (MX)
            bfr = cvt_mxfp4<AT>(wv[s], sc);
          else
            bfr = cvt_dense<AT>(u32x4_t{wv[4 * s], wv[4 * s + 1], wv[4 * s + 2], wv[4 * s + 3]});
          const int blk8 = uu * (UE / 8) + kb * (UE / 16) + s;
          const u32x4_t av = *(const u32x4_t *)&sA[r32 * LDA + blk8 * 8];
          if constexpr (AFF) {
            constexpr uint32_t ONE2 = (AT == DT_BF16) ? 0x3F803F80u : 0x3C003C00u;  // (1.0, 1.0)
            const u32x4_t ones = {ONE2, ONE2, ONE2, ONE2};
            if (s == 0) {
              f32x16_t z;
#pragma unroll
              for (int i = 0; i < 16; ++i) z[i] = 0.f;
              accg = mfma32<AT>(av, bfr, z);
              accx = mfma32<AT>(av, ones, z);
            } else {
              accg = mfma32<AT>(av, bfr, accg);
              accx = mfma32<AT>(av, ones, accx);
            }
          } else {
            acc = mfma32<AT>(av, bfr, acc);
          }
        }
        if constexpr (AFF) {
          const float c_ = fmaf(-MAGIC, sc, qb);
#pragma unroll
          for (int ib = 0; ib < 4; ++ib) {
            if (ib < nib) {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc[4 * ib + j] = fmaf(sc, accg[4 * ib + j], fmaf(c_, accx[4 * ib + j], acc[4 * ib + j]));
            }
          }
        }
      }
    };
    // one chunk: stage its activations and weights, launch the loads two chunks ahead, compute
    auto chunk = [&](int c, const u32x4_t (&gcur)[4], u32x4_t (&gnext2)[4]) {
      const int kc = c * KC;
      __syncthreads();  // readers of the previous chunk's activations are done
      if (c < nchunks) {
        store_a();
        put_w(gcur);
      }
      load_a(kc + KC);
      load_w(kc + 2 * KC, gnext2);
      __syncthreads();
      if (c < nchunks) compute(kc);
    };

    load_a(0);
    for (int c = 0; c < nchunks; c += 3) {
      chunk(c, gA, gC);
      chunk(c + 1, gB, gA);
      chunk(c + 2, gC, gB);
    }

    // ---- epilogue: acc[4*ib + j] is row 8*ib + 4*kb + j of the m-chunk, tile row r32
    if (act) {
      const bool lane_ok = row_ok(r32);
      const int wrow_i = row_of(r32);
      const WMat &M = mat_of(r32);
      const float bo =
          (lane_ok && M.bias) ? bf16_bits_to_f32(((const uint16_t *)M.bias)[(int64_t)e * M.rows + wrow_i]) : 0.f;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        if (ib < nib) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int m = 8 * ib + 4 * kb + j;
            float v = acc[4 * ib + j] + bo;
            if constexpr (GATEUP) {
              if (limit > 0.f) v = fminf(fmaxf(v, -limit), limit);
              const float up = __shfl_xor(v, 16, 64);   // lanes r32 >= 16 hold the up rows
              if (r32 < 16 && m < nr)
                store_act<OT>(p.out, (int64_t)(r0 + m) * p.ldo + col0 + r32, silu_f(v) * up);
            } else {
              if (lane_ok && m < nr) {
                if (p.resid) v += p.resid[(int64_t)(r0 + m) * p.ldr + wrow_i];
                store_act<OT>(p.out, (int64_t)(r0 + m) * p.ldo + wrow_i, v);
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
template <int AT, int WF, int GQ, bool GU, int OT>
static hipError_t launch_t(const GemmParams &p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((expert_gemm<AT, WF, GQ, GU, OT>), dim3(grid), dim3(MOE_GEMM_THREADS),
                     (size_t)p.wave_lds * (MOE_GEMM_THREADS / 64), s, p);
  return hipGetLastError();
}

template <int AT, int WF, int GQ>
static hipError_t launch_o(bool gateup, int odt, const GemmParams &p, int grid, hipStream_t s) {
  if (gateup) {
    if (odt == DT_BF16) return launch_t<AT, WF, GQ, true, DT_BF16>(p, grid, s);
    if (odt == DT_F16) return launch_t<AT, WF, GQ, true, DT_F16>(p, grid, s);
  } else {
    if (odt == DT_F32) return launch_t<AT, WF, GQ, false, DT_F32>(p, grid, s);
    if (odt == DT_BF16) return launch_t<AT, WF, GQ, false, DT_BF16>(p, grid, s);
    if (odt == DT_F16) return launch_t<AT, WF, GQ, false, DT_F16>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int AT>
static hipError_t launch_w(int wfmt, int group, bool gateup, int odt, const GemmParams &p, int grid, hipStream_t s) {
  if (wfmt == WF_DENSE) return launch_o<AT, WF_DENSE, 0>(gateup, odt, p, grid, s);
  if (wfmt == WF_MXFP4) return launch_o<AT, WF_MXFP4, 0>(gateup, odt, p, grid, s);
  if (wfmt == WF_AFFINE4) {
    if (group == 32) return launch_o<AT, WF_AFFINE4, 32>(gateup, odt, p, grid, s);
    if (group == 64) return launch_o<AT, WF_AFFINE4, 64>(gateup, odt, p, grid, s);
    if (group == 128) return launch_o<AT, WF_AFFINE4, 128>(gateup, odt, p, grid, s);
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
