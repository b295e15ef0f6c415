// moe_gemm_tall.hip - grouped expert GEMM for prefill-sized segments (gfx950).
//
// Same computation, packed weight stream and epilogues as the decode kernel of
// moe_gemm.hip (GATEUP: h = silu(clamp(gate z + b_g)) * clamp(up z + b_u); LINEAR:
// o = W a + b (+ f32 residual)), laid out for the MFMA pipe instead of the HBM stream:
//
//   * work unit = (m-tile of up to 128 activation rows, block of 256 weight rows); a
//     512-thread workgroup (8 waves, 1 per CU) owns it, every wave one 32-row block of
//     the packed stream (GATEUP: 16 gate + the 16 up rows of the same outputs), so each
//     weight is dequantised once per 128 tokens and each activation fragment read from
//     LDS feeds two MFMAs;
//   * the activation tile goes HBM -> LDS with gfx950's 16-byte direct loads
//     (global_load_lds_dwordx4), no registers and no VALU on the way, in a multi-stage
//     ring (two 64 KB stages for 4-bit weights, four 16 KB stages for DENSE) with one
//     barrier per stage; a stage is one record (reduction chunk) of the packed stream;
//   * LDS rows are 16-byte-block XOR-swizzled by row, so the MFMA fragment reads (16
//     rows, one block each) spread over the banks while every direct load still writes
//     1 KB contiguously;
//   * the m-tile's 16-row blocks that hold rows are a compile-time count (2, 4, 6 or 8),
//     so the inner loop is straight-line code the compiler can software-pipeline (ds_read
//     of the next step's fragments and the dequantisation of the next weights under the
//     current MFMAs).
//
// Dequantisation (per weight, fp32 then one rounding to the MFMA's 16-bit type):
//   AFFINE4  w = scale*(1024+q) + (qbias - 1024*scale), q exact in f16 as 1024+q
//   MXFP4    the scaled FP4 conversion (exact)
//   DENSE    bf16 as is (rounded to f16 for f16 activations)
// Reduction elements past the matrix width are zero in the packed stream and the matching
// activation blocks are read from a zero block, so tails need no special arithmetic.
#include <hip/hip_ext.h>

#include "moe_mfma.h"

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// source of the activation blocks past the reduction length
__device__ u32x4_t g_zero_block = {0u, 0u, 0u, 0u};

// 16-byte direct load: lane i's 16 bytes land at lds + 16 i (lds must be wave-uniform)
MOE_DEV void load_lds16(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t *)src, (lds_void_t *)lds, 16, 0, 0);
}

// barrier without the compiler's release fence (which would drain every outstanding load,
// the prefetched stages included); callers wait for their own loads first.  LDS reads are
// drained here (lgkmcnt 0, vmcnt and expcnt untouched), so no wave's direct loads can
// overwrite a stage that another wave is still reading.
MOE_DEV void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int WF, int GQ>
struct TallCfg {
  static constexpr int NW = 8;                           // waves per workgroup
  static constexpr int MT = 128;                         // rows per m-tile
  static constexpr int KC = pk_kc(WF);                   // reduction elements per stage (one record)
  static constexpr int BPR = KC / 8;                     // 16-byte blocks per staged row
  static constexpr int ROWB = KC * 2;                    // bytes per staged row
  static constexpr int ABUF = MT * ROWB;                 // bytes per stage
  static constexpr int NBUF = WF == WF_DENSE ? 4 : 2;    // stages resident in LDS
  static constexpr int D = NBUF - 1;                     // stages loaded ahead
  static constexpr int NI = ABUF / (NW * 1024);          // direct loads per wave per stage
  static constexpr int RPI = 1024 / ROWB;                // rows per direct load
  static constexpr int NU = pk_nu(WF, GQ);
  static constexpr int NSL = WF == WF_AFFINE4 ? (NU == 8 ? 4 : 2) : (WF == WF_MXFP4 ? 2 : 0);  // scale loads
  static constexpr int LPS = NI + 4 + NSL;               // vector-memory loads per stage per lane
  static_assert(NI * NW * 1024 == ABUF && RPI * ROWB == 1024, "stage = whole 1 KB loads");
  static_assert(NW * (MT / NW) == MT && (MT / NW) == NI * RPI, "each wave stages 16 rows");
};

// 16-byte block slot of block b in staged row r: XOR with the row so that the 16 rows of
// one fragment read fall on 16 different bank groups (rows of >= 256 bytes: row & 15;
// 128-byte rows: two rows share a 256-byte bank line, so (row >> 1) & 7)
template <int BPR>
MOE_DEV int row_swizzle(int r) {
  return BPR >= 16 ? (r & 15) : ((r >> 1) & 7);
}

template <int AT, int WF, int GQ, bool GATEUP, int OT, int NMB>
MOE_DEV void tall_unit(const GemmParams &p, bool sh, int4 tile, int nb, char *sA, int64_t *sRow) {
  using C = TallCfg<WF, GQ>;
  constexpr bool AFF = (WF == WF_AFFINE4);
  constexpr bool MX = (WF == WF_MXFP4);
  constexpr int KC = C::KC, BPR = C::BPR, ROWB = C::ROWB, ABUF = C::ABUF, NBUF = C::NBUF, D = C::D;
  constexpr int NI = C::NI, RPI = C::RPI, NU = C::NU, LPS = C::LPS;
  constexpr int UE = pk_ue(WF, GQ);                        // elements per unit
  constexpr int SPU = UE / 32;                             // MFMA steps per unit
  constexpr int QE = UE / 4;                               // elements per lane quarter per unit
  constexpr int LPU = pk_lb(WF, GQ) / 4;                   // weight words per lane, unit and half
  constexpr int RB = pk_record_bytes(WF, GQ);
  constexpr int NSW = AFF ? 2 * NU : (MX ? 4 : 1);
  constexpr float MAGIC = 1024.0f;
  static_assert(2 * NU * LPU == 16, "64 weight bytes per lane per record");

  // lane-dependent values are recomputed per unit (opaque thread id): hoisted out of the
  // unit loop they would stay live across it and crowd the registers
  const int tid = (int)in_vgpr(threadIdx.x), lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, kq = lane >> 4;
  const uint32_t msk = in_vgpr(0x000F000Fu);
  const uint32_t mag = in_vgpr(0x64006400u);

  const int e = sh ? 0 : tile.x;
  const int r0 = tile.y, nr = tile.z;

#define SF(f) (sh ? p.seg[1].f : p.seg[0].f)
  const char *Ab = (const char *)SF(A.a);
  const int64_t lda = SF(A.lda);
  const int32_t *gat = SF(A.gather);
  const int gdiv = SF(A.gdiv), rsub = SF(A.row_sub);
  const int Kd = SF(K);
  const float limit = SF(limit);
  const WMat W0 = sh ? p.seg[1].w0 : p.seg[0].w0;
  const uint16_t *bias1 = (const uint16_t *)(GATEUP ? SF(w1.bias) : W0.bias);  // bias of tile half 1
#undef SF

  // tile row t (0..31) of this wave -> weight matrix row; GATEUP: rows 0-15 gate, 16-31 up
  const int col0 = GATEUP ? nb * 128 + wave * 16 : nb * 256 + wave * 32;
  const bool act = col0 < W0.rows;
  auto row_of = [&](int t) { return GATEUP ? col0 + (t & 15) : col0 + t; };
  auto row_ok = [&](int t) { return row_of(t) < W0.rows; };
  const int nst = (Kd + KC - 1) / KC;

  const char *wbase = W0.pk + (int64_t)e * W0.pk_mat +
                      (int64_t)min(nb * C::NW + wave, W0.pk_nblk - 1) * W0.pk_nch * RB;
  struct Ch {
    u32x4_t w[4];
    uint32_t s[NSW];
  };
  auto load_w = [&](int c, Ch &ch) {
    const char *rec = wbase + (int64_t)c * RB;
#pragma unroll
    for (int i = 0; i < 4; ++i) ch.w[i] = *(const u32x4_t *)(rec + i * 1024 + lane * 16);
    if constexpr (AFF) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const char *sp = rec + 4096 + (h * 16 + n16) * NU * 4;
        if constexpr (NU == 8) {
          const u32x4_t x0 = *(const u32x4_t *)sp, x1 = *(const u32x4_t *)(sp + 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ch.s[h * 8 + j] = x0[j];
            ch.s[h * 8 + 4 + j] = x1[j];
          }
        } else if constexpr (NU == 4) {
          const u32x4_t x0 = *(const u32x4_t *)sp;
#pragma unroll
          for (int j = 0; j < 4; ++j) ch.s[h * 4 + j] = x0[j];
        } else {
          const u32x2_t x0 = *(const u32x2_t *)sp;
          ch.s[h * 2] = x0[0];
          ch.s[h * 2 + 1] = x0[1];
        }
      }
    } else if constexpr (MX) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x2_t x0 = *(const u32x2_t *)(rec + 4096 + (h * 16 + n16) * 8);
        ch.s[h * 2] = x0[0];
        ch.s[h * 2 + 1] = x0[1];
      }
    } else {
      ch.s[0] = 0u;
    }
  };

  // output bias of this lane's two tile rows
  float bo[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 16 * h + n16;
    const uint16_t *bp = h ? bias1 : (const uint16_t *)W0.bias;
    bo[h] = bp ? bf16_bits_to_f32(bp[(int64_t)e * W0.rows + (row_ok(t) ? row_of(t) : 0)]) : 0.f;
  }

  // activation rows of the tile (rows past nr read row 0: their results are never stored)
  if (tid < C::MT) {
    const int t = tid < nr ? tid : 0;
    const int64_t arow = gat ? (int64_t)(gat[r0 + t] / gdiv) : (int64_t)(r0 + t - rsub);
    sRow[tid] = arow * lda * 2;
  }
  __syncthreads();

  // this lane's direct-load sources: load n of the wave stages tile row
  // rr = 16 wave + n RPI + lane / BPR into LDS slot lane % BPR, which holds block
  // (lane % BPR) ^ swizzle(rr) of that row
  auto load_a = [&](int c) {
    const int kc = c * KC;
    char *dst = sA + (c % NBUF) * ABUF + wave * (NI * 1024);
    const bool tail = kc + KC > Kd;
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int rr = 16 * wave + n * RPI + lane / BPR;
      const int blk = (lane % BPR) ^ row_swizzle<BPR>(rr);
      const char *src = Ab + sRow[rr] + blk * 16 + (int64_t)kc * 2;
      load_lds16((!tail || kc + blk * 8 < Kd) ? (const void *)src : (const void *)&g_zero_block, dst + n * 1024);
    }
  };

  f32x4_t acc[NMB][2];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[mb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment reads: lane (n16, kq) reads block uu*(UE/8) + kq*(QE/8) + s of rows 16 mb + n16;
  // the lane part of its slot is kq*(QE/8) ^ swizzle(n16) (disjoint bits from the rest)
  const int lx = (kq * (QE / 8)) ^ row_swizzle<BPR>(n16);
  // one MFMA step t = uu*SPU + s of a stage: the B fragments of both halves ...
  auto deq_step = [&](const Ch &ch, int t, u32x4_t (&b)[2]) {
    const int uu = t / SPU, s = t % SPU;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if constexpr (AFF) {
        const uint32_t v = ch.s[h * NU + uu];
        const float sc = __uint_as_float(v << 16);
        const float cc = fmaf(-MAGIC, sc, __uint_as_float(v & 0xFFFF0000u));
        const int q = (uu * 2 + h) * LPU + s;
        b[h] = deq_affine<AT>(ch.w[q >> 2][q & 3], msk, mag, sc, cc);
      } else if constexpr (MX) {
        const uint32_t v = ch.s[h * 2 + (uu >> 1)];
        const float sc = e8m0_to_f32((v >> (8 * (2 * (uu & 1) + (kq >> 1)))) & 0xFFu);
        const int q = (uu * 2 + h) * LPU + s;
        b[h] = cvt_mxfp4<AT>(ch.w[q >> 2][q & 3], sc);
      } else {
        const int q = (uu * 2 + h) * LPU + 4 * s;
        b[h] = cvt_dense<AT>(ch.w[q >> 2]);
      }
    }
  };
  // ... and the A fragments of its NMB row blocks
  auto read_a = [&](const char *sAb, int t, u32x4_t (&a)[NMB]) {
    const int uu = t / SPU, s = t % SPU;
    const char *ap = sAb + (((uu * (UE / 8) + s) ^ lx) << 4);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) a[mb] = *(const u32x4_t *)(ap + mb * 16 * ROWB);
  };
  // a stage, software-pipelined by hand: step t+1's fragment reads and dequantisation are
  // issued with step t's MFMAs; nothing moves across steps, which bounds the live registers
  auto compute = [&](int c, const Ch &ch) {
    constexpr int NS = NU * SPU;
    const char *sAb = sA + (c % NBUF) * ABUF + n16 * ROWB;
    u32x4_t a[NMB], bC[2], bN[2];
    read_a(sAb, 0, a);
    deq_step(ch, 0, bC);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if (t + 1 < NS) deq_step(ch, t + 1, bN);
      const char *apn = sAb + ((((t + 1) / SPU * (UE / 8) + (t + 1) % SPU) ^ lx) << 4);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        acc[mb][0] = mfma16<AT>(a[mb], bC[0], acc[mb][0]);
        acc[mb][1] = mfma16<AT>(a[mb], bC[1], acc[mb][1]);
        if (t + 1 < NS) a[mb] = *(const u32x4_t *)(apn + mb * 16 * ROWB);  // next step's fragment
      }
      __builtin_amdgcn_sched_barrier(0);
      bC[0] = bN[0];
      bC[1] = bN[1];
    }
  };

  // ---- stage pipeline: stages c .. c+D-1 in flight; one barrier per stage (it also
  // tells every wave that stage c-1's buffer, the one stage c+D reuses, has been read)
  Ch ring[NBUF];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    if (j < nst) {
      load_a(j);
      load_w(j, ring[j]);
    }
  }
  for (int c0 = 0; c0 < nst; c0 += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      const int c = c0 + j;
      if (c < nst) {
        if (c + D <= nst)
          wait_vmcnt<(D - 1) * LPS>();
        else
          wait_vmcnt<0>();
        stage_barrier();
        if (c + D < nst) {
          load_a(c + D);
          load_w(c + D, ring[(j + D) % NBUF]);
        }
        if (act) compute(c, ring[j]);
      }
    }
  }

  // ---- epilogue: acc[mb][h][i] is token 16*mb + 4*kq + i of the m-tile, tile row 16*h + n16
  if (act) {
    bool ok[2];
    int wrow[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ok[h] = row_ok(16 * h + n16);
      wrow[h] = row_of(16 * h + n16);
    }
    const int mrem = nr - 4 * kq;                       // token 16*mb + i of this lane exists iff < mrem
    const int64_t obase = (int64_t)(r0 + 4 * kq) * p.ldo;
    const int64_t rbase = (int64_t)(r0 + 4 * kq) * p.ldr;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * mb + i;
        if (m < mrem) {
          const int64_t orow = obase + (int64_t)m * p.ldo;
          if constexpr (GATEUP) {
            float g = acc[mb][0][i] + bo[0], up = acc[mb][1][i] + bo[1];
            if (limit > 0.f) {
              g = fminf(fmaxf(g, -limit), limit);
              up = fminf(fmaxf(up, -limit), limit);
            }
            if (ok[0]) store_act<OT>(p.out, orow + wrow[0], silu_f(g) * up);
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              if (ok[h]) {
                float v = acc[mb][h][i] + bo[h];
                if (p.resid) v += p.resid[rbase + (int64_t)m * p.ldr + wrow[h]];
                store_act<OT>(p.out, orow + wrow[h], v);
              }
            }
          }
        }
      }
    }
  }
}

}  // namespace

template <int AT, int WF, int GQ, bool GATEUP, int OT>
__global__ __launch_bounds__(512, 2) void expert_gemm_tall(const GemmParams p) {
  using C = TallCfg<WF, GQ>;
  __shared__ __attribute__((aligned(1024))) char sA[C::NBUF * C::ABUF];
  __shared__ int64_t sRow[C::MT];

  // units: segment 1 (shared expert / plain rows) first, then the routed m-tiles
  const int nblk0 = p.seg[0].nblk, nblk1 = max(p.seg[1].nblk, 1);
  const int ns = p.seg[1].nblk > 0 ? (p.sh_rows + C::MT - 1) / C::MT : 0;
  const int units_s = ns * nblk1;
  const int nr_routed = p.tiles ? p.tile_count[0] : 0;

  // consecutive units (the column blocks of one m-tile, which share its activation rows) on
  // one XCD, so that they share its L2
  const int G = gridDim.x;
  const int b0 = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int u = b0;; u += G) {
    const bool sh = u < units_s;
    int ti, nb;
    int4 tile;
    if (sh) {
      ti = u / nblk1;
      nb = u - ti * nblk1;
      tile = make_int4(0, p.sh_row0 + ti * C::MT, min(C::MT, p.sh_rows - ti * C::MT), 0);
    } else {
      const int v = u - units_s;
      ti = v / max(nblk0, 1);
      nb = v - ti * nblk0;
      if (!p.tiles) break;
      tile = p.tiles[min(ti, p.max_tiles - 1)];  // in bounds even past the end of the list
      if (ti >= nr_routed) break;
    }
    __syncthreads();  // the previous unit is done with sRow and the stages
    const int nmb = (min(tile.z, C::MT) + 15) >> 4;
    if (nmb <= 2)
      tall_unit<AT, WF, GQ, GATEUP, OT, 2>(p, sh, tile, nb, sA, sRow);
    else if (nmb <= 4)
      tall_unit<AT, WF, GQ, GATEUP, OT, 4>(p, sh, tile, nb, sA, sRow);
    else if (nmb <= 6)
      tall_unit<AT, WF, GQ, GATEUP, OT, 6>(p, sh, tile, nb, sA, sRow);
    else
      tall_unit<AT, WF, GQ, GATEUP, OT, 8>(p, sh, tile, nb, sA, sRow);
  }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
template <int AT, int WF, int GQ, bool GU, int OT>
static void launch_t(const GemmParams &p, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  auto kern = expert_gemm_tall<AT, WF, GQ, GU, OT>;
  if (e0)
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, e0, e1, 0, p);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, p);
}

template <int AT, int WF, int GQ>
static hipError_t launch_o(bool gateup, int odt, const GemmParams &p, int grid, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  if (gateup) {
    if (odt == DT_BF16) launch_t<AT, WF, GQ, true, DT_BF16>(p, grid, s, e0, e1);
    else if (odt == DT_F16) launch_t<AT, WF, GQ, true, DT_F16>(p, grid, s, e0, e1);
    else return hipErrorInvalidValue;
  } else {
    if (odt == DT_F32) launch_t<AT, WF, GQ, false, DT_F32>(p, grid, s, e0, e1);
    else if (odt == DT_BF16) launch_t<AT, WF, GQ, false, DT_BF16>(p, grid, s, e0, e1);
    else if (odt == DT_F16) launch_t<AT, WF, GQ, false, DT_F16>(p, grid, s, e0, e1);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int AT>
static hipError_t launch_w(int wfmt, int group, bool gateup, int odt, const GemmParams &p, int grid, hipStream_t s,
                           hipEvent_t e0, hipEvent_t e1) {
  if (wfmt == WF_DENSE) return launch_o<AT, WF_DENSE, 0>(gateup, odt, p, grid, s, e0, e1);
  if (wfmt == WF_MXFP4) return launch_o<AT, WF_MXFP4, 0>(gateup, odt, p, grid, s, e0, e1);
  if (wfmt == WF_AFFINE4) {
    if (group == 32) return launch_o<AT, WF_AFFINE4, 32>(gateup, odt, p, grid, s, e0, e1);
    if (group == 64) return launch_o<AT, WF_AFFINE4, 64>(gateup, odt, p, grid, s, e0, e1);
    if (group == 128) return launch_o<AT, WF_AFFINE4, 128>(gateup, odt, p, grid, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_expert_gemm_tall(int adt, int wfmt, int group, bool gateup, int odt, const GemmParams &p,
                                   int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (grid <= 0) return hipSuccess;
  if (adt == DT_BF16) return launch_w<DT_BF16>(wfmt, group, gateup, odt, p, grid, s, e0, e1);
  if (adt == DT_F16) return launch_w<DT_F16>(wfmt, group, gateup, odt, p, grid, s, e0, e1);
  return hipErrorInvalidValue;
}
