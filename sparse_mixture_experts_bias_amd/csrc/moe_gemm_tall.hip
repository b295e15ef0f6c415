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
typedef __attribute__((address_space(1))) const char glb_char_t;
// a pointer known to be the same in every lane, as a scalar value
MOE_DEV const char *uniform_ptr(const char *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char *)(((uint64_t)hi << 32) | lo);
}
// same, from a wave-uniform global base plus a per-lane 32-bit byte offset (saddr form)
MOE_DEV void load_lds16_off(const char *base, uint32_t off, void *lds) {
  glb_char_t *g = (glb_char_t *)base;
  __builtin_amdgcn_global_load_lds((glb_void_t *)(g + off), (lds_void_t *)lds, 16, 0, 0);
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

// A stage is the reduction slice that one barrier covers: half a packed record for the
// 4-bit formats (128 elements: two of its four 1 KB weight pieces), one record for DENSE
// (64 elements).  The activation ring holds NBUF stages in LDS and the weight ring NBUF
// stages in registers; loads run D = NBUF - 1 stages ahead of the MFMAs.
template <int WF, int GQ>
struct TallCfg {
  static constexpr bool AFF = WF == WF_AFFINE4, MX = WF == WF_MXFP4, DENSE = WF == WF_DENSE;
  static constexpr int NW = 8;                           // waves per workgroup
  static constexpr int MT = 128;                         // rows per m-tile
  static constexpr int KC = pk_kc(WF);                   // reduction elements per packed record
  static constexpr int SPR = DENSE ? 1 : 2;              // stages per record
  static constexpr int KS = KC / SPR;                    // reduction elements per stage
  static constexpr int PPS = 4 / SPR;                    // 1 KB weight pieces per stage
  static constexpr int BPR = KS / 8;                     // 16-byte blocks per staged row
  static constexpr int ROWB = KS * 2;                    // bytes per staged row
  static constexpr int ABUF = MT * ROWB;                 // activation bytes per stage
  static constexpr int NBUF = DENSE ? 3 : 4;             // stages resident (LDS and registers)
  static constexpr int D = NBUF - 1;                     // stages loaded ahead
  static constexpr int NI = ABUF / (NW * 1024);          // direct loads per wave per stage
  static constexpr int RPI = 1024 / ROWB;                // rows per direct load
  static constexpr int NU = pk_nu(WF, GQ);               // units per record
  static constexpr int NUS = NU / SPR;                   // units per stage
  static constexpr int NSW = AFF ? 2 * NUS : (MX ? 2 : 0);  // scale words per lane per stage
  static constexpr int NSL = NSW ? 2 : 0;                // scale loads per stage (one per half)
  static constexpr int LPS = NI + PPS + NSL;             // vector-memory loads per stage per lane
  static_assert(NI * NW * 1024 == ABUF && RPI * ROWB == 1024, "stage = whole 1 KB loads");
  static_assert(NW * (MT / NW) == MT && (MT / NW) == NI * RPI, "each wave stages 16 rows");
  static_assert(NUS * SPR == NU, "whole units per stage");
};

// 16-byte block slot of block b in staged row r: XOR with the row so that the 16 rows of
// one fragment read fall on 16 different bank groups (rows of >= 256 bytes: row & 15;
// 128-byte rows: two rows share a 256-byte bank line, so (row >> 1) & 7)
template <int BPR>
MOE_DEV int row_swizzle(int r) {
  return BPR >= 16 ? (r & 15) : ((r >> 1) & 7);
}

// the activation stages: one LDS variable each, so that the compiler can tell a stage's
// direct loads from the fragment reads of another (accesses to one variable may alias:
// every read of it would then wait for all direct loads in flight)
struct StageBufs {
  char *b[4];
};

// four adjacent outputs (nv of them valid): one 8- or 16-byte store when aligned
template <int OT>
MOE_DEV void store4(void *out, int64_t idx, const float (&v)[4], int nv, bool vec) {
  if (vec && nv == 4) {
    if constexpr (OT == DT_F32) {
      *(f32x4_t *)((float *)out + idx) = f32x4_t{v[0], v[1], v[2], v[3]};
    } else if constexpr (OT == DT_BF16) {
      const bf16x2_t a = {(__bf16)v[0], (__bf16)v[1]}, b = {(__bf16)v[2], (__bf16)v[3]};
      *(u32x2_t *)((uint16_t *)out + idx) = u32x2_t{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
    } else {
      const f16x2_t a = {(_Float16)v[0], (_Float16)v[1]}, b = {(_Float16)v[2], (_Float16)v[3]};
      *(u32x2_t *)((uint16_t *)out + idx) = u32x2_t{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < nv) store_act<OT>(out, idx + i, v[i]);
  }
}

template <int AT, int WF, int GQ, bool GATEUP, int OT, int NMB>
MOE_DEV void tall_unit(const GemmParams &p, bool sh, int4 tile, int nb, const StageBufs &sA, int64_t *sRow) {
  using C = TallCfg<WF, GQ>;
  constexpr bool AFF = C::AFF, MX = C::MX;
  constexpr int KS = C::KS, SPR = C::SPR, PPS = C::PPS, BPR = C::BPR, ROWB = C::ROWB, ABUF = C::ABUF;
  constexpr int NBUF = C::NBUF, D = C::D, NI = C::NI, RPI = C::RPI, NU = C::NU, NUS = C::NUS;
  constexpr int NSW = C::NSW, LPS = C::LPS;
  constexpr int UE = pk_ue(WF, GQ);                        // elements per unit
  constexpr int SPU = UE / 32;                             // MFMA steps per unit
  constexpr int QE = UE / 4;                               // elements per lane quarter per unit
  constexpr int LPU = pk_lb(WF, GQ) / 4;                   // weight words per lane, unit and half
  constexpr int RB = pk_record_bytes(WF, GQ);
  static_assert(2 * NU * LPU == 16, "64 weight bytes per lane per record");

  // lane-dependent values are recomputed per unit (opaque thread id): hoisted out of the
  // unit loop they would stay live across it and crowd the registers
  const int tid = (int)in_vgpr(threadIdx.x), lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, kq = lane >> 4;
  const uint32_t m0 = in_vgpr(0x000F000Fu), m1 = in_vgpr(0x00F000F0u);
  const uint32_t g0 = in_vgpr(0x64006400u), g1 = in_vgpr(0x54005400u);

  // the tile is the same for the whole workgroup: keep it (and what derives from it) scalar
  const int e = sh ? 0 : __builtin_amdgcn_readfirstlane(tile.x);
  const int r0 = __builtin_amdgcn_readfirstlane(tile.y), nr = __builtin_amdgcn_readfirstlane(tile.z);

#define SF(f) (sh ? p.seg[1].f : p.seg[0].f)
  const char *Ab = (const char *)SF(A.a);
  const int64_t lda = SF(A.lda);
  const int64_t arows = SF(A.rows);
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
  const int nst = (Kd + KS - 1) / KS;                      // stages (the last record may hold one)

  const char *wbase = W0.pk + (int64_t)e * W0.pk_mat +
                      (int64_t)min(nb * C::NW + wave, W0.pk_nblk - 1) * W0.pk_nch * RB;
  // weight ring slot: the stage's PPS pieces (the lane's 16 bytes of each) and scale words
  struct Ch {
    u32x4_t w[PPS];
    uint32_t s[NSW > 0 ? NSW : 1];
  };
  // load k (0 .. PPS + NSL - 1) of stage c's weights into ring slot ch: the weight pieces,
  // then one scale load per tile half.  The slot's old values are "used" right before the
  // load, so that the registers stay the slot's until it is reloaded: reused for something
  // else in between, they would carry a false wait on the load in flight.
  auto load_w1 = [&](int c, Ch &ch, int k) {
    const char *rec = wbase + (int64_t)(c / SPR) * RB;
    const int half = c % SPR;
    if (k < PPS) {
      asm volatile("" : "+v"(ch.w[k]));
      ch.w[k] = *(const u32x4_t *)(rec + (half * PPS + k) * 1024 + lane * 16);
    } else if constexpr (AFF) {
      const int h = k - PPS;
#pragma unroll
      for (int j = 0; j < NUS; ++j) asm volatile("" : "+v"(ch.s[h * NUS + j]));
      const char *sp = rec + 4096 + ((h * 16 + n16) * NU + half * NUS) * 4;
      if constexpr (NUS == 4) {
        const u32x4_t x = *(const u32x4_t *)sp;
#pragma unroll
        for (int j = 0; j < 4; ++j) ch.s[h * 4 + j] = x[j];
      } else if constexpr (NUS == 2) {
        const u32x2_t x = *(const u32x2_t *)sp;
        ch.s[h * 2] = x[0];
        ch.s[h * 2 + 1] = x[1];
      } else {
        ch.s[h] = *(const uint32_t *)sp;
      }
    } else if constexpr (MX) {
      const int h = k - PPS;
      asm volatile("" : "+v"(ch.s[h]));
      ch.s[h] = *(const uint32_t *)(rec + 4096 + (h * 16 + n16) * 8 + half * 4);
    }
  };
  auto load_w = [&](int c, Ch &ch) {
#pragma unroll
    for (int k = 0; k < PPS + C::NSL; ++k) load_w1(c, ch, k);
  };

  // output bias of this lane's tile rows 16 h + 4 kq + i: loaded now (no bias: from a zero
  // block) and kept as raw bits, so nothing waits for them before the epilogue
  uint16_t bo_raw[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint16_t *bp = h ? bias1 : (const uint16_t *)W0.bias;
    const uint16_t *bz = (const uint16_t *)&g_zero_block;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * h + 4 * kq + i;
      bo_raw[h][i] = bp ? bp[(int64_t)e * W0.rows + (row_ok(t) ? row_of(t) : 0)] : bz[0];
    }
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
  // (lane % BPR) ^ swizzle(rr) of that row.  Byte offsets from the activation base fit in
  // 32 bits (checked by the host), so full stages issue the loads with a scalar base and a
  // fixed vector offset per load.
  uint32_t aoff[NI];
  int ablk[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const int rr = 16 * wave + n * RPI + lane / BPR;
    ablk[n] = (lane % BPR) ^ row_swizzle<BPR>(rr);
    aoff[n] = (uint32_t)sRow[rr] + (uint32_t)(ablk[n] * 16);
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // direct load n (0 .. NI-1) of stage c's activations into LDS stage buffer buf, through a
  // buffer resource over the activation rows: the lane's byte offset is the fixed aoff[n],
  // the stage's column offset a scalar, and bytes past the rows read as zero.  (Keeping the
  // lane's address register fixed matters: rewriting a register that a direct load in flight
  // addresses makes the compiler wait for that load.)
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)Ab, (short)0, (int)(uint32_t)(arows * lda * 2), 0x00020000);
  auto load_a1 = [&](int c, int buf, int n) {
    char *dst = sA.b[buf] + wave_u * (NI * 1024) + n * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_void_t *)dst, 16, aoff[n], c * KS * 2, 0, 0);
  };
  // the stage that holds the end of the reduction: its blocks past Kd hold the next row's
  // elements (or zeros past the rows); each lane zeroes its own, once its loads are in
  // (before the stage's barrier)
  auto zero_tail = [&](int c, int buf) {
    const int kc = c * KS;
#pragma unroll
    for (int n = 0; n < NI; ++n)
      if (kc + ablk[n] * 8 >= Kd)
        *(u32x4_t *)(sA.b[buf] + wave_u * (NI * 1024) + n * 1024 + lane * 16) = u32x4_t{0u, 0u, 0u, 0u};
  };
  auto load_a = [&](int c, int buf) {
#pragma unroll
    for (int n = 0; n < NI; ++n) load_a1(c, buf, n);
  };
  // load k (0 .. LPS-1) of stage c: activations first, then the weights
  auto load_k = [&](int c, int buf, Ch &ch, int k) {
    if (k < NI)
      load_a1(c, buf, k);
    else
      load_w1(c, ch, k - NI);
  };

  f32x4_t acc[NMB][2];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[mb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fragment reads: lane (n16, kq) reads block uu*(UE/8) + kq*(QE/8) + s of rows 16 mb + n16
  // (uu: unit within the stage); the lane part of its slot is kq*(QE/8) ^ swizzle(n16)
  // (disjoint bits from the rest)
  const int lx = (kq * (QE / 8)) ^ row_swizzle<BPR>(n16);
  // one MFMA step t = uu*SPU + s of a stage: the B fragments of both halves ...
  auto deq_step = [&](const Ch &ch, int t, u32x4_t (&b)[2]) {
    const int uu = t / SPU, s = t % SPU;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = (uu * 2 + h) * LPU + (C::DENSE ? 4 * s : s);   // word of the stage's lane sequence
      if constexpr (AFF) {
        const uint32_t v = ch.s[h * NUS + uu];
        const float sc = __uint_as_float(v << 16), qb = __uint_as_float(v & 0xFFFF0000u);
        b[h] = deq_affine<AT>(ch.w[q >> 2][q & 3], m0, m1, g0, g1, sc, fmaf(-1024.0f, sc, qb), fmaf(-64.0f, sc, qb));
      } else if constexpr (MX) {
        const float sc = e8m0_to_f32((ch.s[h] >> (8 * (2 * uu + (kq >> 1)))) & 0xFFu);
        b[h] = cvt_mxfp4<AT>(ch.w[q >> 2][q & 3], sc);
      } else {
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
  // issued with step t's MFMAs, interleaved (per row block: MFMA, VALU, MFMA, VALU, LDS read)
  // so that the conversion work runs under the matrix pipe; nothing moves across steps,
  // which bounds the live registers
  constexpr int VPS = AFF ? 40 : 12;                       // VALU of one step's dequantisation
  constexpr int VPM = (VPS + 2 * NMB - 1) / (2 * NMB);     // ... per MFMA
  // The loads of stage cl are issued from inside the MFMA steps, LPS/NS per step:
  // issued all at once they stall every wave on the address path for ~100 cycles each.
  auto compute = [&](int c, int buf, const Ch &ch, bool issue, int cl, int bufl, Ch &chl) {
    constexpr int NS = NUS * SPU;
    constexpr int LPT = (LPS + NS - 1) / NS;               // loads issued per step
    const char *sAb = sA.b[buf] + n16 * ROWB;
    u32x4_t a[NMB], bC[2], bN[2];
    read_a(sAb, 0, a);
    deq_step(ch, 0, bC);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      if (issue) {
#pragma unroll
        for (int k = t * LPT; k < (t + 1) * LPT && k < LPS; ++k) load_k(cl, bufl, chl, k);
      }
      if (t + 1 < NS) deq_step(ch, t + 1, bN);
      const char *apn = sAb + ((((t + 1) / SPU * (UE / 8) + (t + 1) % SPU) ^ lx) << 4);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        acc[mb][0] = mfma16<AT>(bC[0], a[mb], acc[mb][0]);
        acc[mb][1] = mfma16<AT>(bC[1], a[mb], acc[mb][1]);
        if (t + 1 < NS) a[mb] = *(const u32x4_t *)(apn + mb * 16 * ROWB);  // next step's fragment
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // LDS read
        if (mb < LPT) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
      }
      __builtin_amdgcn_sched_barrier(0);
      bC[0] = bN[0];
      bC[1] = bN[1];
    }
  };

  // ---- stage pipeline: stages c .. c+D-1 in flight; one barrier per stage (it also
  // tells every wave that stage c-1's buffer, the one stage c+D reuses, has been read).
  // Whole groups of NBUF stages run in a branch-free loop (its back edge is then only taken
  // with exactly D stages of loads in flight, which lets the compiler count them exactly);
  // every stage there issues LPS loads, past the last stage repeats of the last stage's
  // sources into the buffer and ring slot that no later stage reads.  The remaining < NBUF
  // stages follow, in ring slots 0.., loading nothing.  The unit-start barrier (a full
  // __syncthreads) drains the repeats.
  Ch ring[NBUF];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int cj = min(j, nst - 1);
    load_a(cj, j);
    load_w(cj, ring[j]);
  }
  // waves past the matrix's rows (act false) run the same code on a clamped row block and
  // drop the result: one code path keeps the compiler's wait counts exact
  int c0 = 0;
  for (; c0 + NBUF <= nst; c0 += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      const int c = c0 + j;
      wait_vmcnt<(D - 1) * LPS>();
      if ((c + 1) * KS > Kd) zero_tail(c, j);
      stage_barrier();
      compute(c, j, ring[j], true, min(c + D, nst - 1), (j + D) % NBUF, ring[(j + D) % NBUF]);
    }
  }
  // remainder stage c0 + j: its loads were issued D stages before it, followed by those of
  // D - 1 - j more stages
  auto last = [&](int j, auto wait) {
    const int c = c0 + j;
    wait();
    if ((c + 1) * KS > Kd) zero_tail(c, j);
    stage_barrier();
    compute(c, j, ring[j], false, 0, 0, ring[j]);
  };
  if (c0 < nst) {
    last(0, [] { wait_vmcnt<(D - 1) * LPS>(); });
    if constexpr (NBUF > 2) {
      if (c0 + 1 < nst) {
        last(1, [] { wait_vmcnt<(D - 2) * LPS>(); });
        if constexpr (NBUF > 3) {
          if (c0 + 2 < nst) last(2, [] { wait_vmcnt<0>(); });
        }
      }
    }
  }

  // ---- epilogue: acc[mb][h][i] is tile row 16*h + 4*kq + i (weights are the MFMA's A
  // operand) and token 16*mb + n16, so every lane holds four adjacent output columns of
  // one token row and writes them with one store
  if (act) {
    float bo[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) bo[h][i] = bf16_bits_to_f32(bo_raw[h][i]);
    const bool vec = (p.ldo & 3) == 0 && ((uintptr_t)p.out & (OT == DT_F32 ? 15 : 7)) == 0;
    const bool rvec = p.resid && (p.ldr & 3) == 0 && ((uintptr_t)p.resid & 15) == 0;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const int tok = 16 * mb + n16;
      if (tok < nr) {
        const int64_t orow = (int64_t)(r0 + tok) * p.ldo;
        if constexpr (GATEUP) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float g = acc[mb][0][i] + bo[0][i], up = acc[mb][1][i] + bo[1][i];
            if (limit > 0.f) {
              g = fminf(fmaxf(g, -limit), limit);
              up = fminf(fmaxf(up, -limit), limit);
            }
            v[i] = silu_f(g) * up;
          }
          const int col = row_of(4 * kq);
          store4<OT>(p.out, orow + col, v, min(4, W0.rows - col), vec);
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int col = row_of(16 * h + 4 * kq);
            const int nv = min(4, W0.rows - col);
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = acc[mb][h][i] + bo[h][i];
            if (p.resid) {
              const float *rp = p.resid + (int64_t)(r0 + tok) * p.ldr + col;
              if (rvec && nv == 4) {
                const f32x4_t r = *(const f32x4_t *)rp;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] += r[i];
              } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (i < nv) v[i] += rp[i];
              }
            }
            store4<OT>(p.out, orow + col, v, nv, vec);
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
  __shared__ __attribute__((aligned(1024))) char sA0[C::ABUF];
  __shared__ __attribute__((aligned(1024))) char sA1[C::ABUF];
  __shared__ __attribute__((aligned(1024))) char sA2[C::ABUF];
  __shared__ __attribute__((aligned(1024))) char sA3[C::NBUF > 3 ? C::ABUF : 16];
  const StageBufs sA = {{sA0, sA1, sA2, sA3}};
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
  // the last unit's look-ahead loads (repeats of its last stage) may still be writing LDS
  __builtin_amdgcn_s_waitcnt(0);
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
