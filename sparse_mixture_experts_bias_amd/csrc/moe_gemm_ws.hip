// moe_gemm_ws.hip - grouped expert GEMM for decode-sized segments with 4-bit weights
// (AFFINE4, MXFP4): the bandwidth-bound LDS-staged path of the gather_qmm pattern.
//
// Same units, arithmetic and epilogues as the decode kernel of moe_gemm.hip (unit = m-tile
// of up to 16 rows x 4 row blocks of the packed stream; AFFINE4 codes enter the MFMA as
// the exact values MAGIC + q and each quantisation group is folded in fp32 with its scale
// and bias; MXFP4 blocks convert exactly with their E8M0 scale), with the memory stream
// taken off the waves that compute:
//
//   * a 512-thread workgroup has four compute waves (one row block each, as before) and
//     four loader waves.  The loaders copy every chunk record (weights + scales) and the
//     m-tile's activation rows HBM -> LDS with direct loads (no registers, no VALU) into a
//     ring of NBUF stages and run NBUF - 1 stages ahead; one barrier per stage hands a stage
//     over.  Two stage buffers per workgroup leave room for three workgroups per CU (twelve
//     compute waves), which measured faster than three buffers at two per CU.  A compute wave never waits for memory itself, so the stream keeps going while
//     it dequantises and multiplies (with loads and arithmetic on the same waves they
//     alternate instead of overlapping);
//   * the stage sequence runs across the workgroup's units, so the next unit's records
//     stream in while the current one finishes and stores its outputs;
//   * activation rows sit in LDS with 16-byte blocks XOR-swizzled by row, so the fragment
//     reads of 16 rows spread over the banks; the loaders read them through a buffer
//     resource (fixed per-lane offsets, bytes past the matrix read as zero) and take the
//     row gather indices from the scalar cache.
#include <hip/hip_ext.h>

#include "moe_ws.h"


template <int AT, int WF, int GQ, bool GATEUP, int OT>
__global__ __launch_bounds__(512, 6) void expert_gemm_ws(const GemmParams p) {  // 3 workgroups per CU
  using C = WsCfg<WF, GQ>;
  constexpr bool AFF = C::AFF, MX = C::MX;
  constexpr int MT = 16, KC = C::KC, UE = C::UE, SPU = C::SPU, QE = C::QE, LPU = C::LPU, NU = C::NU;
  constexpr int RB = C::RB, SW = C::SW, STAGE = C::STAGE, NBUF = C::NBUF, NDMA = C::NDMA;
  constexpr float MAGIC = AT == DT_BF16 ? 128.0f : 1024.0f;
  __shared__ __attribute__((aligned(16))) char smem[NBUF * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // units: segment 1 (shared expert / plain rows) first, then the routed m-tiles.  The
  // arguments the schedule needs are read in one batch (materialised together, so that the
  // compiler does not fetch them one dependent round trip at a time)
  const int nblk0 = p.seg[0].nblk, nb1 = p.seg[1].nblk, sh_rows = p.sh_rows, sh_row0 = p.sh_row0;
  const int max_tiles = p.max_tiles;
  const int4 *const tiles = p.tiles;
  const int *const tcount = p.tile_count;
  asm volatile("" ::"s"(nblk0), "s"(nb1), "s"(sh_rows), "s"(sh_row0), "s"(max_tiles), "s"(tiles), "s"(tcount));
  const int nblk1 = max(nb1, 1);
  const int ns = nb1 > 0 ? (sh_rows + MT - 1) / MT : 0;
  const int units_s = ns * nblk1;
  // workgroup g's first unit is unit g, its later ones g + G, g + 2G, ... (round-robin over
  // the XCDs: decode-sized activation rows fit any L2); the first unit's tile is read
  // together with the tile count
  const int G = gridDim.x, g = blockIdx.x;
  int nr_routed = 0;
  int4 t_first = make_int4(0, 0, 0, 0);
  if (tiles && max_tiles > 0) {
    const int ti = min(max(g - units_s, 0) / max(nblk0, 1), max_tiles - 1);
    load_uniform_int_int4(tcount, tiles + ti, nr_routed, t_first);
    nr_routed = min(nr_routed, max_tiles);
  }
  const int U = units_s + nr_routed * nblk0;

  struct Unit {
    bool sh;
    int e, r0, nr, nb;
  };
  auto unit_at = [&](int u, bool first) {
    Unit x;
    x.sh = u < units_s;
    if (x.sh) {
      const int ti = u / nblk1;
      x.nb = u - ti * nblk1;
      x.e = 0;
      x.r0 = sh_row0 + ti * MT;
      x.nr = min(MT, sh_rows - ti * MT);
    } else {
      const int v = u - units_s;
      const int ti = v / nblk0;
      x.nb = v - ti * nblk0;
      const int4 t = first ? t_first : load_uniform_int4(p.tiles + ti);
      x.e = t.x;
      x.r0 = t.y;
      x.nr = t.z;
    }
    return x;
  };
  // a field of the unit's segment (selected field by field: a selected struct would go to scratch)
#define SEG(x, f) ((x).sh ? p.seg[1].f : p.seg[0].f)
  auto nch_of = [&](int u) { return ((u < units_s ? p.seg[1].K : p.seg[0].K) + KC - 1) / KC; };

  if (wave >= 4) {
    // ---------------- loader waves: row block lw's records, activation rows 4 lw .. 4 lw + 3
    const int lw = wave - 4;
    __amdgpu_buffer_rsrc_t wrs, ars;
    uint32_t wvo = 0, svo = 0, avo[2] = {0u, 0u};
    bool aon[2] = {true, true};  // the activation load holds a row of the m-tile
    int cu = g, cc = 0, cn = 0;  // the stage to issue next: unit, chunk, chunks of the unit
    // unit x's weights and scales (no memory access) ...
    auto enter_w = [&](const Unit &x, int u) {
      const SegSet &S = p.seg[x.sh ? 1 : 0];
      cn = nch_of(u);
      const int64_t pk_mat = S.w0.pk_mat;
      wrs = __builtin_amdgcn_make_buffer_rsrc((void *)(S.w0.pk + (int64_t)x.e * pk_mat), (short)0, (int)pk_mat,
                                              0x00020000);
      const uint32_t rbo = (uint32_t)min(x.nb * 4 + lw, S.w0.pk_nblk - 1) * (uint32_t)(S.w0.pk_nch * RB);
      wvo = rbo + lane * 16;
      svo = rbo + 4096 + lane * (C::SB == 1024 ? 16 : 4);
    };
    // ... and its activation rows (reads the gather indices)
    auto enter_a = [&](const Unit &x) {
      const SegSet &S = p.seg[x.sh ? 1 : 0];
      const int64_t lda = S.A.lda;
      ars = __builtin_amdgcn_make_buffer_rsrc((void *)S.A.a, (short)0, (int)(S.A.rows * lda * 2),
                                              0x00020000);
      const int32_t *gat = S.A.gather;
      const int gdiv = S.A.gdiv, rsub = S.A.row_sub;
      uint32_t ro[4];
      int gi[4];
      if (gat) {
        const int *g0 = gat + x.r0;
        load_uniform_ints4(g0 + min(4 * lw, x.nr - 1), g0 + min(4 * lw + 1, x.nr - 1), g0 + min(4 * lw + 2, x.nr - 1),
                           g0 + min(4 * lw + 3, x.nr - 1), gi);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int m = min(4 * lw + k, x.nr - 1);
        const int arow = gat ? gi[k] / gdiv : x.r0 + m - rsub;
        ro[k] = (uint32_t)arow * (uint32_t)lda * 2u;
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        aon[n] = 4 * lw + 2 * n < x.nr;
        const int r = 4 * lw + 2 * n + (lane >> 5);
        avo[n] = (lane < 32 ? ro[2 * n] : ro[2 * n + 1]) + (uint32_t)(((lane & 31) ^ (r & 15)) << 4);
      }
    };
    auto issue_w = [&](int b) {
      char *base = smem + b * STAGE;
      const int so = cc * RB;
      char *wl = base + lw * RB;
      WS_DMA(16, 0, wrs, wl, wvo, so);
      WS_DMA(16, 1024, wrs, wl, wvo, so);
      WS_DMA(16, 2048, wrs, wl, wvo, so);
      WS_DMA(16, 3072, wrs, wl, wvo, so);
      if constexpr (C::SB == 1024) {
        WS_DMA(16, 0, wrs, wl + 4096, svo, so);
      } else {
        WS_DMA(4, 0, wrs, wl + 4096, svo, so);
        if constexpr (C::NSD == 2) WS_DMA(4, 256, wrs, wl + 4096, svo, so);
      }
    };
    auto issue_a = [&](int b) {
      char *base = smem + b * STAGE;
      // activation rows past the m-tile are never stored: a 4-byte load keeps the count
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        if (aon[n])
          WS_DMA(16, 0, ars, base + SW + (2 * lw + n) * 1024, avo[n], cc * KC * 2);
        else
          WS_DMA(4, 0, ars, base + SW + (2 * lw + n) * 1024, avo[n], cc * KC * 2);
      }
    };
    // past the last unit the cursor stays on the last stage (reloaded into free buffers)
    auto advance = [&]() {
      if (cc + 1 < cn) {
        ++cc;
      } else if (cu + G < U) {
        cu += G;
        const Unit x = unit_at(cu, false);
        enter_w(x, cu);
        enter_a(x);
        cc = 0;
      }
    };
    if (g >= U) return;
    {
      // the first stage's weights go out before the gather indices are read
      const Unit x = unit_at(g, true);
      enter_w(x, g);
      issue_w(0);
      enter_a(x);
      issue_a(0);
      advance();
    }
#pragma unroll
    for (int j = 1; j < NBUF - 1; ++j) {
      issue_w(j);
      issue_a(j);
      advance();
    }
    wait_vmcnt<(NBUF - 2) * NDMA>();  // stage 0 has landed
    int s = 0;
    for (int u = g; u < U; u += G) {
      const int n = nch_of(u);
      for (int c = 0; c < n; ++c, ++s) {
        stage_barrier();  // stage s is handed over; the buffer of stage s - 1 is free
        issue_w((s + NBUF - 1) % NBUF);
        issue_a((s + NBUF - 1) % NBUF);
        advance();
        wait_vmcnt<(NBUF - 2) * NDMA>();  // stage s + 1 has landed
      }
    }
    wait_vmcnt<0>();  // no direct load may still write this workgroup's LDS
    return;
  }

  // ---------------- compute waves: row block `wave` of the unit
  const int n16 = lane & 15, kq = lane >> 4;
  const uint32_t msk = in_vgpr(0x000F000Fu);
  const uint32_t mag = in_vgpr(AT == DT_BF16 ? 0x43004300u : 0x64006400u);
  int s = 0;
  for (int u = g; u < U; u += G) {
    const Unit x = unit_at(u, u == g);
    const int Kd = SEG(x, K), n = nch_of(u), rows = SEG(x, w0.rows);
    const float limit = SEG(x, limit);
    const int col0 = GATEUP ? x.nb * 64 + wave * 16 : x.nb * 128 + wave * 32;
    const bool act = col0 < rows;
    auto row_of = [&](int t) { return GATEUP ? col0 + (t & 15) : col0 + t; };
    auto row_ok = [&](int t) { return row_of(t) < rows; };
    // output bias of the lane's two tile rows (GATEUP: gate and up of one output): loaded now
    // (from a valid dummy address when absent), first used by the epilogue
    const uint16_t *bp[2] = {(const uint16_t *)SEG(x, w0.bias),
                             (const uint16_t *)(GATEUP ? SEG(x, w1.bias) : SEG(x, w0.bias))};
    uint32_t bbits[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 16 * h + n16;
      const uint16_t *ba = bp[h] ? bp[h] + (int64_t)x.e * rows + (row_ok(t) ? row_of(t) : 0)
                                 : (const uint16_t *)p.out;
      bbits[h] = *ba;
    }
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    for (int c = 0; c < n; ++c, ++s) {
      stage_barrier();
      if (!act) continue;
      const char *buf = smem + (s % NBUF) * STAGE;
      const char *rec = buf + wave * RB;
      u32x4_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = *(const u32x4_t *)(rec + i * 1024 + lane * 16);
      uint32_t sw[2][NU];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (AFF) {
          const char *sp = rec + 4096 + (h * 16 + n16) * NU * 4;
#pragma unroll
          for (int q = 0; q < NU; q += 2) {
            const u32x2_t v2 = *(const u32x2_t *)(sp + q * 4);
            sw[h][q] = v2[0];
            sw[h][q + 1] = v2[1];
          }
        } else {
          const u32x2_t v2 = *(const u32x2_t *)(rec + 4096 + (h * 16 + n16) * 8);
          sw[h][0] = v2[0];
          sw[h][1] = v2[1];
        }
      }
      const char *arow = buf + SW + n16 * (KC * 2);
      const int nunits = min(KC, Kd - c * KC) / UE;
      // group uu: scales, weight words, activation fragments, MFMAs, fold
      auto scales = [&](int uu, float (&sc)[2], float (&cc)[2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if constexpr (AFF) {
            const uint32_t v = sw[h][uu];
            sc[h] = __uint_as_float(v << 16);
            cc[h] = fmaf(-MAGIC, sc[h], __uint_as_float(v & 0xFFFF0000u));
          } else {
            sc[h] = e8m0_scale((sw[h][uu >> 1] >> (8 * (2 * (uu & 1) + (kq >> 1)))) & 0xFFu);
            cc[h] = 0.f;
          }
        }
      };
      auto word = [&](int uu, int h, int st) {
        const int q = (uu * 2 + h) * LPU + st;
        return w[q >> 2][q & 3];
      };
      auto afrag = [&](int uu, int st) {
        const int blk = (uu * UE + kq * QE + 8 * st) >> 3;
        return *(const u32x4_t *)(arow + ((blk ^ n16) << 4));
      };
      struct GS {
        f32x4_t g0, g1, sx;
      };
      // AFFINE4: the three MFMA chains of a group (magic-valued codes of both halves, ones)
      auto mfmas = [&](int uu) {
        constexpr uint32_t ONE2 = (AT == DT_BF16) ? 0x3F803F80u : 0x3C003C00u;  // (1.0, 1.0)
        const u32x4_t ones = {ONE2, ONE2, ONE2, ONE2};
        const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        GS r = {z, z, z};
#pragma unroll
        for (int st = 0; st < SPU; ++st) {
          const u32x4_t av = afrag(uu, st);
          r.g0 = mfma16<AT>(av, magic_pairs(word(uu, 0, st), msk, mag), r.g0);
          r.g1 = mfma16<AT>(av, magic_pairs(word(uu, 1, st), msk, mag), r.g1);
          r.sx = mfma16<AT>(av, ones, r.sx);
        }
        return r;
      };
      auto fold = [&](int uu, const GS &r) {
        float sc[2], cc[2];
        scales(uu, sc, cc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[0][i] = fmaf(sc[0], r.g0[i], fmaf(cc[0], r.sx[i], acc[0][i]));
          acc[1][i] = fmaf(sc[1], r.g1[i], fmaf(cc[1], r.sx[i], acc[1][i]));
        }
      };
      auto mx_group = [&](int uu) {
        float sc[2], cc[2];
        scales(uu, sc, cc);
#pragma unroll
        for (int st = 0; st < SPU; ++st) {
          const u32x4_t av = afrag(uu, st);
          acc[0] = mfma16<AT>(av, cvt_mxfp4<AT>(word(uu, 0, st), sc[0]), acc[0]);
          acc[1] = mfma16<AT>(av, cvt_mxfp4<AT>(word(uu, 1, st), sc[1]), acc[1]);
        }
      };
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) {
        if (uu >= nunits) break;
        if constexpr (AFF)
          fold(uu, mfmas(uu));
        else
          mx_group(uu);
      }
    }
    // ---- epilogue: acc[h][i] is token 4*kq + i of the m-tile, tile row 16*h + n16
    float bo[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) bo[h] = bp[h] ? bf16_bits_to_f32(bbits[h]) : 0.f;
    if (act) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * kq + i;
        if (m >= x.nr) continue;
        if constexpr (GATEUP) {
          if (row_ok(n16)) {
            float g = acc[0][i] + bo[0], up = acc[1][i] + bo[1];
            if (limit > 0.f) {
              g = clamp_act(g, limit);
              up = clamp_act(up, limit);
            }
            store_act<OT>(p.out, (int64_t)(x.r0 + m) * p.ldo + row_of(n16), silu_f(g) * up);
          }
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int t = 16 * h + n16;
            if (row_ok(t)) {
              float v = acc[h][i] + bo[h];
              if (p.resid) v += p.resid[(int64_t)(x.r0 + m) * p.ldr + row_of(t)];
              store_act<OT>(p.out, (int64_t)(x.r0 + m) * p.ldo + row_of(t), v);
            }
          }
        }
      }
    }
  }
#undef SEG
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
namespace {

template <int AT, int WF, int GQ, bool GU, int OT>
hipError_t ws_launch_t(const GemmParams &p, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  auto kern = expert_gemm_ws<AT, WF, GQ, GU, OT>;
  if (e0)
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, e0, e1, 0, p);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, p);
  return hipGetLastError();
}

template <int AT, int WF, int GQ>
hipError_t ws_launch_o(bool gateup, int odt, const GemmParams &p, int grid, hipStream_t s, hipEvent_t e0,
                       hipEvent_t e1) {
  if (gateup) {
    if (odt == DT_BF16) return ws_launch_t<AT, WF, GQ, true, DT_BF16>(p, grid, s, e0, e1);
    if (odt == DT_F16) return ws_launch_t<AT, WF, GQ, true, DT_F16>(p, grid, s, e0, e1);
  } else {
    if (odt == DT_F32) return ws_launch_t<AT, WF, GQ, false, DT_F32>(p, grid, s, e0, e1);
    if (odt == DT_BF16) return ws_launch_t<AT, WF, GQ, false, DT_BF16>(p, grid, s, e0, e1);
    if (odt == DT_F16) return ws_launch_t<AT, WF, GQ, false, DT_F16>(p, grid, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

template <int AT>
hipError_t ws_launch_w(int wfmt, int group, bool gateup, int odt, const GemmParams &p, int grid, hipStream_t s,
                       hipEvent_t e0, hipEvent_t e1) {
  if (wfmt == WF_MXFP4) return ws_launch_o<AT, WF_MXFP4, 0>(gateup, odt, p, grid, s, e0, e1);
  if (wfmt == WF_AFFINE4) {
    if (group == 32) return ws_launch_o<AT, WF_AFFINE4, 32>(gateup, odt, p, grid, s, e0, e1);
    if (group == 64) return ws_launch_o<AT, WF_AFFINE4, 64>(gateup, odt, p, grid, s, e0, e1);
    if (group == 128) return ws_launch_o<AT, WF_AFFINE4, 128>(gateup, odt, p, grid, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int ws_wgs_per_cu(int wfmt, int group) {
  if (wfmt == WF_MXFP4) return WsCfg<WF_MXFP4, 0>::WGS_PER_CU;
  if (group == 32) return WsCfg<WF_AFFINE4, 32>::WGS_PER_CU;
  if (group == 128) return WsCfg<WF_AFFINE4, 128>::WGS_PER_CU;
  return WsCfg<WF_AFFINE4, 64>::WGS_PER_CU;
}

hipError_t launch_expert_gemm_ws(int adt, int wfmt, int group, bool gateup, int odt, const GemmParams &p, int grid,
                                 hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (grid <= 0) return hipSuccess;
  if (adt == DT_BF16) return ws_launch_w<DT_BF16>(wfmt, group, gateup, odt, p, grid, s, e0, e1);
  if (adt == DT_F16) return ws_launch_w<DT_F16>(wfmt, group, gateup, odt, p, grid, s, e0, e1);
  return hipErrorInvalidValue;
}
