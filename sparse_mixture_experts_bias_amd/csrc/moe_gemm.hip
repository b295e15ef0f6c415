// moe_gemm.hip - grouped expert GEMM for decode-sized segments on gfx950 (the gather_qmm
// pattern); prefill-sized segments go to moe_gemm_tall.hip.
//
// One launch applies a stack of expert weight matrices to activation rows that
// are grouped by expert (the sorted slots of the permutation), plus optionally
// one more segment for the shared expert.  Two epilogues:
//   GATEUP: h = silu(clamp(gate z + b_g)) * clamp(up z + b_u)  (SwiGLU, w1 = gate,
//           w3 = up of ferrox-models latent_moe.rs; the swiglu_limit clamp of
//           libmir-metal's gate/up kernel, read as a clamp of both to [-L, L])
//   LINEAR: o = W a + b (+ an f32 residual)      (down projections, latent maps)
//
// Work unit = (m-tile of up to 16 activation rows of one segment, block of output
// columns).  A 256-thread workgroup (4 waves) stages the m-tile's rows in
// LDS one reduction chunk at a time; each wave streams its own 32 weight rows from
// HBM and feeds v_mfma_f32_16x16x32_{bf16,f16} with tokens as the A operand and
// weight rows as the B operand (two 16-row halves per wave).
//
// Weight formats (see moe_linear in include/moe.h):
//   AFFINE4 (mlxcel issue #974's affine gather_qmm plane): a nibble q becomes the
//     16-bit value MAGIC+q by OR-ing it into the mantissa of MAGIC, which is exact;
//     every quantisation group is folded in fp32:
//       acc += scale * sum((MAGIC+q) a) + (qbias - MAGIC*scale) * sum(a),
//     which equals sum (scale*q + qbias) a with the weights never rounded; the
//     group sums of a come from one extra MFMA against a vector of ones.
//     The packed words hold the codes in pair order, so the nibble pairs come out
//     as adjacent elements (q_2j, q_2j+1) and the activations are used as stored.
//   MXFP4 (libmir-metal ExpertLayout blocks/scales): gfx950's scaled FP4
//     conversion turns E2M1 codes times the block's 2^(e-127) into bf16/f16
//     exactly; the block scale is applied in that conversion.
//   DENSE bf16: used as is (converted to f16 when the activations are f16).
#include <hip/hip_ext.h>

#include "moe_mfma.h"

// Every wave owns one 32-row weight tile, one row block of the packed stream: GATEUP: 16
// gate rows (half 0) and the 16 up rows of the same outputs (half 1); LINEAR: 32 output
// rows.  Lane l works on tile rows l%16 and 16 + l%16 and on the m-tile's tokens
// l%16 (A operand) / 4*(l/16) + i (D).
//
// Weight stream: a chunk record of the wave's row block is 4 KB of weights already in MFMA
// lane order plus the chunk's scales, contiguous in HBM; every lane loads its own 64 bytes
// with four 16-byte loads (each instruction reads 1 KB contiguous) and its scale words,
// two chunks ahead of the MFMAs, straight into registers.  Only the activations go through
// LDS (shared by the four waves).
//
// Reduction order: a "unit" of UE elements (AFFINE4: one quantisation group; MXFP4: 64;
// DENSE: 32) is split into four contiguous quarters, one per lane quarter l/16; MFMA step s
// of the unit takes elements [8s, 8s+8) of every quarter, so each step stays inside one group.
//
// SHORT (decode tiles with at most three chunks, e.g. down projections of a few hundred
// reduction elements): the whole unit is loaded at once, weights into registers and the
// activations into three LDS tiles, then computed without further barriers; the smaller
// register footprint gives four workgroups per CU.
template <int AT, int WF, int GQ, bool GATEUP, int OT, bool SHORT = false>
__global__ __launch_bounds__(MOE_GEMM_THREADS, SHORT ? 4 : 3) void expert_gemm(const GemmParams p) {
  constexpr bool AFF = (WF == WF_AFFINE4);
  constexpr bool MX = (WF == WF_MXFP4);
  constexpr bool DENSE = (WF == WF_DENSE);
  constexpr int MT = 16;                                   // rows per m-tile
  constexpr int UE = pk_ue(WF, GQ);                        // elements per unit
  constexpr int SPU = UE / 32;                             // MFMA steps per unit
  constexpr int QE = UE / 4;                               // elements per lane quarter per unit
  constexpr int LPU = pk_lb(WF, GQ) / 4;                   // weight words per lane, unit and half
  constexpr int KC = pk_kc(WF);                            // reduction elements per chunk
  constexpr int NU = pk_nu(WF, GQ);                        // units per chunk
  constexpr int RB = pk_record_bytes(WF, GQ);              // bytes per chunk record
  constexpr int NSW = AFF ? 2 * NU : (MX ? 4 : 1);         // scale words per lane per chunk
  constexpr int BPR = KC / 8;                              // 8-element activation blocks per chunk row
  constexpr int RPI = MOE_GEMM_THREADS / BPR;              // activation rows staged per iteration
  constexpr int SIT = (MT + RPI - 1) / RPI;                // activation staging iterations
  constexpr int LDA = KC + 8;                              // padded LDS activation row (16-bit elements)
  constexpr int NSA = SHORT ? 3 : 2;                       // activation tiles (double-buffered)
  constexpr float MAGIC = AT == DT_BF16 ? 128.0f : 1024.0f;
  static_assert(2 * NU * LPU == 16, "64 weight bytes per lane per chunk");
  static_assert(KC % UE == 0 && UE % 32 == 0, "units of whole MFMA steps");
  __shared__ __attribute__((aligned(16))) uint16_t sAbuf[NSA][MT * LDA];
  __shared__ int64_t sRow[MT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, kq = lane >> 4;
  const int sblk = tid % BPR, srow0 = tid / BPR;
  const uint32_t msk = in_vgpr(0x000F000Fu);
  const uint32_t mag = in_vgpr(AT == DT_BF16 ? 0x43004300u : 0x64006400u);

  // units: segment 1 (shared expert / plain rows, m-tiles computed here) first, then the
  // routed m-tiles of the tile list
  const int nblk0 = p.seg[0].nblk, nblk1 = max(p.seg[1].nblk, 1);
  const int ns = p.seg[1].nblk > 0 ? (p.sh_rows + MT - 1) / MT : 0;
  const int units_s = ns * nblk1;
  const int nr_routed = p.tiles ? min(p.tile_count[0], p.max_tiles) : 0;

  const int G = gridDim.x;
  const int U = units_s + (p.tiles ? nr_routed * nblk0 : 0);
  for (int r = 0;; ++r) {
    const int u = sched_unit(blockIdx.x, r, G, U);
    if (u < 0) break;
    const bool sh = u < units_s;
    int ti, nb;
    int4 tile;
    if (sh) {
      ti = u / nblk1;
      nb = u - ti * nblk1;
      tile = make_int4(0, p.sh_row0 + ti * MT, min(MT, p.sh_rows - ti * MT), 0);
    } else {
      const int v = u - units_s;
      ti = v / max(nblk0, 1);
      nb = v - ti * nblk0;
      if (!p.tiles) break;
      tile = p.tiles[min(ti, p.max_tiles - 1)];  // in bounds even past the end of the list
      if (ti >= nr_routed) break;
    }
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
    const uint16_t *bias1 = (const uint16_t *)(GATEUP ? SF(w1.bias) : W0.bias);  // bias of tile half 1
#undef SF

    // tile row t (0..31) -> weight matrix row; GATEUP: rows 0-15 gate, 16-31 up
    const int col0 = GATEUP ? nb * 64 + wave * 16 : nb * 128 + wave * 32;
    const bool act = col0 < W0.rows;
    auto row_of = [&](int t) { return GATEUP ? col0 + (t & 15) : col0 + t; };
    auto row_ok = [&](int t) { return row_of(t) < W0.rows; };
    const int nchunks = (Kd + KC - 1) / KC;

    // this wave's row block of the packed stream (a clamped valid block when the wave idles)
    const char *wbase = W0.pk + (int64_t)e * W0.pk_mat +
                        (int64_t)min(nb * 4 + wave, W0.pk_nblk - 1) * W0.pk_nch * RB;
    struct Ch {
      u32x4_t w[4];
      uint32_t s[NSW];
    };
    auto load_ch = [&](int kc, Ch &ch) {
      const char *rec = wbase + (int64_t)(min(kc, (nchunks - 1) * KC) / KC) * RB;
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

    // output bias of this lane's two tile rows, loaded now so that the epilogue waits on nothing
    float bo[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 16 * h + n16;
      const uint16_t *bp = h ? bias1 : (const uint16_t *)W0.bias;
      bo[h] = bp ? bf16_bits_to_f32(bp[(int64_t)e * W0.rows + (row_ok(t) ? row_of(t) : 0)]) : 0.f;
    }

    Ch cA, cB, cC;  // weight ring: chunk c, c+1 in flight, c+2 being loaded
    load_ch(0, cA);  // in flight during the set-up below
    load_ch(KC, cB);
    if constexpr (SHORT) load_ch(2 * KC, cC);

    __syncthreads();  // the previous unit is done with sRow / sA
    if (tid < nr) {
      const int64_t arow = gat ? (int64_t)(gat[r0 + tid] / gdiv) : (int64_t)(r0 + tid - rsub);
      sRow[tid] = arow * lda;
    }
    __syncthreads();

    // ---- activation staging: raw bits only; every call issues the same loads (addresses
    // clamped into valid memory) so the compiler can count them; out-of-range data is zeroed
    // when stored
    auto load_a = [&](int kc, u32x4_t (&areg)[SIT]) {
      const int kcc = min(kc, (nchunks - 1) * KC);
      const int kn = min(KC, Kd - kcc);
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int row = srow0 + RPI * it;
        const int rr = row < nr ? row : 0;
        const int cc = sblk * 8 < kn ? sblk * 8 : 0;
        areg[it] = *(const u32x4_t *)(Ab + sRow[rr] + kcc + cc);
      }
    };
    // branch-free (rows past nr and columns past K are written as zeros), so that the
    // compiler can count the loads still in flight instead of draining them all
    auto store_a = [&](int kc, const u32x4_t (&areg)[SIT]) {
      uint16_t *sA = sAbuf[(kc / KC) % NSA];
      const bool colok = sblk * 8 < Kd - kc;
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int row = srow0 + RPI * it;
        if (RPI * SIT <= MT || row < MT) {
          u32x4_t v = areg[it];
          const bool ok = colok && row < nr;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = ok ? v[q] : 0u;
          *(u32x4_t *)&sA[row * LDA + sblk * 8] = v;
        }
      }
    };

    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};

    auto compute = [&](int kc, const Ch &ch) {
      if (!act) return;
      const int nunits = min(KC, Kd - kc) / UE;
      const uint16_t *sA = sAbuf[(kc / KC) % NSA];
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) {
        if (uu >= nunits) break;
        const int eoff = uu * UE + kq * QE;          // first element of this lane's quarter
        uint32_t wv[2][LPU];
        float sc[2], cc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int wi = 0; wi < LPU; ++wi) {
            const int q = (uu * 2 + h) * LPU + wi;   // compile-time
            wv[h][wi] = ch.w[q >> 2][q & 3];
          }
          if constexpr (AFF) {
            const uint32_t v = ch.s[h * NU + uu];
            sc[h] = __uint_as_float(v << 16);
            cc[h] = fmaf(-MAGIC, sc[h], __uint_as_float(v & 0xFFFF0000u));
          } else if constexpr (MX) {
            const uint32_t v = ch.s[h * 2 + (uu >> 1)];
            sc[h] = e8m0_scale((v >> (8 * (2 * (uu & 1) + (kq >> 1)))) & 0xFFu);
            cc[h] = 0.f;
          } else {
            sc[h] = cc[h] = 0.f;
          }
        }
        const uint16_t *arow = &sA[n16 * LDA + eoff];
        if constexpr (AFF) {
          // exact group fold: both halves share the A fragment and the group sums
          constexpr uint32_t ONE2 = (AT == DT_BF16) ? 0x3F803F80u : 0x3C003C00u;  // (1.0, 1.0)
          const u32x4_t ones = {ONE2, ONE2, ONE2, ONE2};
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          f32x4_t g0 = z, g1 = z, sx = z;
#pragma unroll
          for (int s = 0; s < SPU; ++s) {
            const u32x4_t av = *(const u32x4_t *)(arow + 8 * s);
            g0 = mfma16<AT>(av, magic_pairs(wv[0][s], msk, mag), g0);
            g1 = mfma16<AT>(av, magic_pairs(wv[1][s], msk, mag), g1);
            sx = mfma16<AT>(av, ones, sx);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[0][i] = fmaf(sc[0], g0[i], fmaf(cc[0], sx[i], acc[0][i]));
            acc[1][i] = fmaf(sc[1], g1[i], fmaf(cc[1], sx[i], acc[1][i]));
          }
        } else {
#pragma unroll
          for (int s = 0; s < SPU; ++s) {
            u32x4_t b[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              if constexpr (MX)
                b[h] = cvt_mxfp4<AT>(wv[h][s], sc[h]);
              else
                b[h] = cvt_dense<AT>(u32x4_t{wv[h][4 * s], wv[h][4 * s + 1], wv[h][4 * s + 2], wv[h][4 * s + 3]});
            }
            const u32x4_t av = *(const u32x4_t *)(arow + 8 * s);
            acc[0] = mfma16<AT>(av, b[0], acc[0]);
            acc[1] = mfma16<AT>(av, b[1], acc[1]);
          }
        }
      }
    };

    if constexpr (SHORT) {
      u32x4_t a0[SIT], a1[SIT], a2[SIT];
      load_a(0, a0);
      load_a(KC, a1);
      load_a(2 * KC, a2);
      store_a(0, a0);
      store_a(KC, a1);
      store_a(2 * KC, a2);
      __syncthreads();
      compute(0, cA);
      if (nchunks > 1) compute(KC, cB);
      if (nchunks > 2) compute(2 * KC, cC);
    } else {
      // activations and weights two chunks ahead (3-deep register rings); the
      // activation tile is double-buffered, so one barrier per chunk suffices: a wave stores
      // chunk c+1 only after every wave has passed chunk c's barrier, i.e. has finished
      // computing chunk c-1, the last reader of that buffer.
      u32x4_t aA[SIT], aB[SIT], aC[SIT];
      auto chunk = [&](int c, const Ch &ccur, Ch &cnext2, const u32x4_t (&acur)[SIT], u32x4_t (&anext2)[SIT]) {
        const int kc = c * KC;
        store_a(kc, acur);  // chunks past the end stage clamped data that nobody reads
        load_a(kc + 2 * KC, anext2);
        load_ch(kc + 2 * KC, cnext2);
        __syncthreads();
        if (c < nchunks) compute(kc, ccur);
      };
      load_a(0, aA);
      __builtin_amdgcn_sched_barrier(0);  // keep chunk 0's loads ahead of chunk 1's (in-order vmcnt)
      load_a(KC, aB);
      for (int c = 0; c < nchunks; c += 3) {
        chunk(c, cA, cC, aA, aC);
        chunk(c + 1, cB, cA, aB, aA);
        chunk(c + 2, cC, cB, aC, aB);
        // the next iteration starts on the loads of chunk c+1 (aA, cA); only chunk c+2's may
        // stay in flight.  Waiting here, where it is due anyway, keeps the compiler from
        // draining every load at the loop header.
        wait_vmcnt<LOADS_PER_CHUNK<WF, GQ, SIT>()>();
      }
    }

    // ---- epilogue: acc[h][i] is token 4*kq + i of the m-tile, tile row 16*h + n16
    if (act) {
      bool ok[2];
      int wrow[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ok[h] = row_ok(16 * h + n16);
        wrow[h] = row_of(16 * h + n16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * kq + i;
        if (m < nr) {
          if constexpr (GATEUP) {
            float g = acc[0][i] + bo[0], up = acc[1][i] + bo[1];
            if (limit > 0.f) {
              g = clamp_act(g, limit);
              up = clamp_act(up, limit);
            }
            if (ok[0]) store_act<OT>(p.out, (int64_t)(r0 + m) * p.ldo + wrow[0], silu_f(g) * up);
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              if (ok[h]) {
                float v = acc[h][i] + bo[h];
                if (p.resid) v += p.resid[(int64_t)(r0 + m) * p.ldr + wrow[h]];
                store_act<OT>(p.out, (int64_t)(r0 + m) * p.ldo + wrow[h], v);
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
      v0 = clamp_act(v0, p.limit);
      v1 = clamp_act(v1, p.limit);
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
// e0/e1: optional events stamped at the kernel's start and end (timing).  mb == 0 selects
// the SHORT decode variant (LINEAR only).
template <int AT, int WF, int GQ, bool GU, int OT>
static hipError_t launch_t(int mb, const GemmParams &p, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  auto go = [&](auto kern) {
    if (e0)
      hipExtLaunchKernelGGL(kern, dim3(grid), dim3(MOE_GEMM_THREADS), 0, s, e0, e1, 0, p);
    else
      hipLaunchKernelGGL(kern, dim3(grid), dim3(MOE_GEMM_THREADS), 0, s, p);
  };
  if constexpr (!GU) {
    if (mb == 0) {
      go(expert_gemm<AT, WF, GQ, GU, OT, true>);
      return hipGetLastError();
    }
  }
  if (mb == 1)
    go(expert_gemm<AT, WF, GQ, GU, OT>);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int AT, int WF, int GQ>
static hipError_t launch_o(bool gateup, int odt, int mb, const GemmParams &p, int grid, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  if (gateup) {
    if (odt == DT_BF16) return launch_t<AT, WF, GQ, true, DT_BF16>(mb, p, grid, s, e0, e1);
    if (odt == DT_F16) return launch_t<AT, WF, GQ, true, DT_F16>(mb, p, grid, s, e0, e1);
  } else {
    if (odt == DT_F32) return launch_t<AT, WF, GQ, false, DT_F32>(mb, p, grid, s, e0, e1);
    if (odt == DT_BF16) return launch_t<AT, WF, GQ, false, DT_BF16>(mb, p, grid, s, e0, e1);
    if (odt == DT_F16) return launch_t<AT, WF, GQ, false, DT_F16>(mb, p, grid, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

template <int AT>
static hipError_t launch_w(int wfmt, int group, bool gateup, int odt, int mb, const GemmParams &p, int grid,
                           hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (wfmt == WF_DENSE) return launch_o<AT, WF_DENSE, 0>(gateup, odt, mb, p, grid, s, e0, e1);
  if (wfmt == WF_MXFP4) return launch_o<AT, WF_MXFP4, 0>(gateup, odt, mb, p, grid, s, e0, e1);
  if (wfmt == WF_AFFINE4) {
    if (group == 32) return launch_o<AT, WF_AFFINE4, 32>(gateup, odt, mb, p, grid, s, e0, e1);
    if (group == 64) return launch_o<AT, WF_AFFINE4, 64>(gateup, odt, mb, p, grid, s, e0, e1);
    if (group == 128) return launch_o<AT, WF_AFFINE4, 128>(gateup, odt, mb, p, grid, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_expert_gemm(int adt, int wfmt, int group, bool gateup, int odt, int mb, const GemmParams &p,
                              int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (grid <= 0) return hipSuccess;
  if (adt == DT_BF16) return launch_w<DT_BF16>(wfmt, group, gateup, odt, mb, p, grid, s, e0, e1);
  if (adt == DT_F16) return launch_w<DT_F16>(wfmt, group, gateup, odt, mb, p, grid, s, e0, e1);
  return hipErrorInvalidValue;
}

hipError_t launch_f32_gemm(const F32GemmParams &p, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int cols = p.ncols_r > p.ncols_s ? p.ncols_r : p.ncols_s;
  hipLaunchKernelGGL(f32_gemm_kernel, dim3(rows, (cols + 63) / 64), dim3(64), 0, s, p);
  return hipGetLastError();
}
