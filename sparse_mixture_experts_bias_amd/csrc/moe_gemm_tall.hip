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
//   * the activation tile goes HBM -> LDS with gfx950's 16-byte direct loads, no
//     registers and no VALU on the way, in a ring of four stages with one barrier per
//     stage; a stage is half a packed record (32 KB of activations) for the 4-bit formats
//     and one record (16 KB) for DENSE, and its weights travel in a register ring;
//   * LDS rows are 16-byte-block XOR-swizzled by row, so the MFMA fragment reads (16
//     rows, one block each) spread over the banks while every direct load still writes
//     1 KB contiguously;
//   * the m-tile's 16-row blocks that hold rows are a compile-time count (2, 4, 6 or 8),
//     so the inner loop is straight-line code the compiler can software-pipeline (ds_read
//     of the next step's fragments and the dequantisation of the next weights under the
//     current MFMAs).
//
// Dequantisation (per weight, fp32 then one rounding to the MFMA's 16-bit type):
//   AFFINE4  w = scale*(1024+q) + (qbias - 1024*scale), q exact in f16 as 1024+q (f16
//            activations: packed half-precision q = (1024+q) - 1024, then scale*q + qbias)
//   MXFP4    the scaled FP4 conversion (exact)
//   DENSE    bf16 as is (rounded to f16 for f16 activations)
//   WF_MXS   none: MXFP4 codes and E8M0 scales go to the block-scaled 16x16x128 FP4 x FP8
//            MFMA as stored (moe_pack_weights_scaled stream), against activations split
//            into two e4m3 terms with E8M0 block scales (split_fp8_kernel); a stage is one
//            MFMA step, and the activations' scale pairs travel in a small LDS ring of
//            their own (one more direct load per stage)
// Reduction elements past the matrix width are zero in the packed stream and the matching
// activation blocks are read from a zero block, so tails need no special arithmetic.
#include <hip/hip_ext.h>

#include "moe_mfma.h"

namespace {

// zeros: the source of absent biases
__device__ u32x4_t g_zero_block = {0u, 0u, 0u, 0u};

// A stage is the reduction slice that one barrier covers: half a packed record for the
// 4-bit formats (128 elements: two of its four 1 KB weight pieces), one record for DENSE
// (64 elements).  The activation ring holds NBUF stages in LDS and the weight ring NBUF
// stages in registers; loads run D = NBUF - 1 stages ahead of the MFMAs.
template <int WF, int GQ>
struct TallCfg {
  static constexpr bool AFF = WF == WF_AFFINE4, MX = WF == WF_MXFP4, DENSE = WF == WF_DENSE, MXS = WF == WF_MXS;
  static constexpr int NW = 8;                           // waves per workgroup
  static constexpr int MT = 128;                         // rows per m-tile
  static constexpr int KC = pk_kc(WF);                   // reduction elements per packed record
  static constexpr int SPR = DENSE ? 1 : 2;              // stages per record
  static constexpr int KS = KC / SPR;                    // reduction elements per stage
  static constexpr int PPS = 4 / SPR;                    // 1 KB weight pieces per stage
  static constexpr int BPR = KS / 8;                     // 16-byte blocks per staged row
  static constexpr int ROWB = KS * 2;                    // bytes per staged row
  static constexpr int ABUF = MT * ROWB;                 // activation bytes per stage
  static constexpr int NBUF = 4;                         // stages resident (LDS and registers)
  static constexpr int D = NBUF - 1;                     // stages loaded ahead
  static constexpr int NI = ABUF / (NW * 1024);          // direct loads per wave per stage
  static constexpr int RPI = 1024 / ROWB;                // rows per direct load
  static constexpr int NU = pk_nu(WF, GQ);               // units per record
  static constexpr int NUS = NU / SPR;                   // units per stage
  static constexpr int NSW = AFF ? 2 * NUS : (MX ? 2 : (MXS ? 1 : 0));  // scale words per lane per stage
  static constexpr int NSL = NSW ? (MXS ? 1 : 2) : 0;    // scale loads per stage (one per half; MXS: one)
  static constexpr int NAS = MXS ? 1 : 0;                // activation-scale direct loads per stage
  static constexpr int LPS = NI + NAS + PPS + NSL;       // vector-memory loads per stage per lane
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
  char *s[4];  // WF_MXS: the activations' scale pairs of each stage (8 waves x 256 bytes)
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

// A work unit: the m-tile and column block, with everything its loads and epilogue read
// (all wave-uniform, so it lives in scalar registers).
struct TallUnit {
  bool sh;
  int e, r0, nr, nb, Kd;
  float limit;
  const char *Ab;
  int64_t lda, arows;
  const uint16_t *As;       // WF_MXS: activation scale pairs and their row stride (elements)
  int64_t ldas;
  const int32_t *gat;
  int gdiv, rsub;
  int rows;                 // weight rows (output columns, GATEUP: per half)
  const char *pk;           // packed stream, its matrix stride and row blocks
  int64_t pk_mat;
  int pk_nblk, pk_nch;
  const uint16_t *bias0;    // output bias of tile half 0 (GATEUP: the gate rows)
  const uint16_t *bias1;    // ... and of tile half 1 (GATEUP: the up rows)
};

template <bool GATEUP>
MOE_DEV TallUnit tall_unit_of(const GemmParams &p, bool sh, int4 tile, int nb) {
  TallUnit t;
  t.sh = sh;
  t.e = sh ? 0 : __builtin_amdgcn_readfirstlane(tile.x);
  t.r0 = __builtin_amdgcn_readfirstlane(tile.y);
  t.nr = __builtin_amdgcn_readfirstlane(tile.z);
  t.nb = nb;
#define SF(f) (sh ? p.seg[1].f : p.seg[0].f)
  t.Ab = (const char *)SF(A.a);
  t.lda = SF(A.lda);
  t.arows = SF(A.rows);
  t.As = SF(A.as);
  t.ldas = SF(A.ldas);
  t.gat = SF(A.gather);
  t.gdiv = SF(A.gdiv);
  t.rsub = SF(A.row_sub);
  t.Kd = SF(K);
  t.limit = SF(limit);
  t.rows = SF(w0.rows);
  t.pk = SF(w0.pk);
  t.pk_mat = SF(w0.pk_mat);
  t.pk_nblk = SF(w0.pk_nblk);
  t.pk_nch = SF(w0.pk_nch);
  t.bias0 = (const uint16_t *)SF(w0.bias);
  t.bias1 = (const uint16_t *)(GATEUP ? SF(w1.bias) : SF(w0.bias));
#undef SF
  return t;
}

// byte offsets of the unit's activation rows (rows past nr read row 0: their results are
// never stored), written by the first MT threads
template <int MT>
MOE_DEV void tall_fill_rows(const TallUnit &u, int64_t *sRow, int tid) {
  if (tid < MT) {
    const int t = tid < u.nr ? tid : 0;
    const int64_t arow = u.gat ? (int64_t)(u.gat[u.r0 + t] / u.gdiv) : (int64_t)(u.r0 + t - u.rsub);
    sRow[tid] = arow * u.lda * 2;
  }
}

// weight ring slot: one stage's PPS weight pieces (the lane's 16 bytes of each) and scales
template <int WF, int GQ>
struct TallSlot {
  u32x4_t w[TallCfg<WF, GQ>::PPS];
  uint32_t s[TallCfg<WF, GQ>::NSW > 0 ? TallCfg<WF, GQ>::NSW : 1];
};

// what a lane needs to issue a unit's loads
template <int WF, int GQ, bool GATEUP>
struct TallLoader {
  using C = TallCfg<WF, GQ>;
  static constexpr int NI = C::NI, PPS = C::PPS, NU = C::NU, NUS = C::NUS, SPR = C::SPR, KS = C::KS, NAS = C::NAS;
  static constexpr int RB = pk_record_bytes(WF, GQ);
  __amdgpu_buffer_rsrc_t arsrc;
  uint32_t aoff[NI];
  __amdgpu_buffer_rsrc_t srsrc;  // WF_MXS: the activation scale pairs
  uint32_t soff;
  int ablk[NI];
  const char *wbase;
  int wave_u, lane, n16, Kd, nst;

  // this lane's direct-load sources: load n of the wave stages tile row
  // rr = 16 wave + n RPI + lane / BPR into LDS slot lane % BPR, which holds block
  // (lane % BPR) ^ swizzle(rr) of that row.  The activations are read through a buffer
  // resource over their rows: the lane's byte offset is the fixed aoff[n] (32 bits, checked
  // by the host), the stage's column offset a scalar, and bytes past the rows read as zero.
  // (Keeping a lane's address register fixed matters: rewriting a register that a direct
  // load in flight addresses makes the compiler wait for that load.)
  __device__ __forceinline__ TallLoader(const TallUnit &u, const int64_t *sRow, int wave, int lane_) {
    lane = lane_;
    n16 = lane & 15;
    wave_u = __builtin_amdgcn_readfirstlane(wave);
    // a wave whose 16 staged rows all lie past the m-tile (never stored) reads past the
    // buffer's range: the loads return zeros without touching memory
    const bool aon = 16 * wave_u < u.nr;
    Kd = u.Kd;
    nst = (u.Kd + KS - 1) / KS;
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int rr = 16 * wave + n * C::RPI + lane / C::BPR;
      ablk[n] = (lane % C::BPR) ^ row_swizzle<C::BPR>(rr);
      aoff[n] = aon ? (uint32_t)sRow[rr] + (uint32_t)(ablk[n] * 16) : 0xF0000000u;
    }
    arsrc = __builtin_amdgcn_make_buffer_rsrc((void *)u.Ab, (short)0, (int)(uint32_t)(u.arows * u.lda * 2), 0x00020000);
    if constexpr (C::MXS) {
      // lanes 0..31 stage the 8 bytes (4 blocks x (Eh, El)) of the wave's 16 rows for the
      // stage, two lanes a row; lanes 32..63 read past the range (zeros, no traffic)
      const int rr = 16 * wave + ((lane & 31) >> 1);
      const uint32_t arow = (uint32_t)sRow[rr] / (uint32_t)(u.lda * 2);
      soff = (aon && lane < 32) ? arow * (uint32_t)(u.ldas * 2) + (uint32_t)(lane & 1) * 4u : 0xF0000000u;
      srsrc = __builtin_amdgcn_make_buffer_rsrc((void *)u.As, (short)0, (int)(uint32_t)(u.arows * u.ldas * 2), 0x00020000);
    }
    wbase = u.pk + (int64_t)u.e * u.pk_mat + (int64_t)min(u.nb * C::NW + wave, u.pk_nblk - 1) * u.pk_nch * RB;
  }
  // direct load n (0 .. NI-1) of stage c's activations into LDS stage buffer dst
  __device__ __forceinline__ void load_a1(int c, char *buf, int n) const {
    char *dst = buf + wave_u * (NI * 1024) + n * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_void_t *)dst, 16, aoff[n], c * KS * 2, 0, 0);
  }
  // the scale pairs of stage c's activations into scale buffer dst (WF_MXS)
  __device__ __forceinline__ void load_as(int c, char *buf) const {
    char *dst = buf + wave_u * 256;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, (lds_void_t *)dst, 4, soff, c * 8, 0, 0);
  }
  // load k (0 .. PPS + NSL - 1) of stage c's weights into ring slot ch: the weight pieces,
  // then one scale load per tile half.  The slot's old values are "used" right before the
  // load, so that the registers stay the slot's until it is reloaded: reused for something
  // else in between, they would carry a false wait on the load in flight.
  __device__ __forceinline__ void load_w1(int c, TallSlot<WF, GQ> &ch, int k) const {
    const char *rec = wbase + (int64_t)(c / SPR) * RB;
    const int half = c % SPR;
    if (k < PPS) {
      asm volatile("" : "+v"(ch.w[k]));
      ch.w[k] = *(const u32x4_t *)(rec + (half * PPS + k) * 1024 + lane * 16);
    } else if constexpr (C::MXS) {
      asm volatile("" : "+v"(ch.s[0]));
      ch.s[0] = *(const uint32_t *)(rec + 4096 + lane * 4);
    } else if constexpr (C::AFF) {
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
    } else if constexpr (C::MX) {
      const int h = k - PPS;
      asm volatile("" : "+v"(ch.s[h]));
      ch.s[h] = *(const uint32_t *)(rec + 4096 + (h * 16 + n16) * 8 + half * 4);
    }
  }
  // load k (0 .. LPS-1) of stage c into stage buffer bi: activations (and their scales)
  // first, then the weights
  __device__ __forceinline__ void load_k(int c, const StageBufs &sA, int bi, TallSlot<WF, GQ> &ch, int k) const {
    if (k < NI)
      load_a1(c, sA.b[bi], k);
    else if (k < NI + NAS)
      load_as(c, sA.s[bi]);
    else
      load_w1(c, ch, k - NI - NAS);
  }
  // the activations of the unit's first D stages (repeats of its last stage if it has fewer)
  __device__ __forceinline__ void load_first_a(const StageBufs &sA) const {
#pragma unroll
    for (int j = 0; j < C::D; ++j) {
#pragma unroll
      for (int n = 0; n < NI; ++n) load_a1(min(j, nst - 1), sA.b[j], n);
      if constexpr (C::MXS) load_as(min(j, nst - 1), sA.s[j]);
    }
  }
  // ... and their weights
  __device__ __forceinline__ void load_first_w(TallSlot<WF, GQ> (&ring)[C::NBUF]) const {
#pragma unroll
    for (int j = 0; j < C::D; ++j)
#pragma unroll
      for (int k = 0; k < PPS + C::NSL; ++k) load_w1(min(j, nst - 1), ring[j], k);
  }
};

// One unit's stages and epilogue.  On entry the activations of its first D stages are in
// flight (buffers 0 .. D-1); before the epilogue it issues those of the next unit (has_nxt),
// whose rows are in sRow_nxt, so that they load while this epilogue runs.
template <int AT, int WF, int GQ, bool GATEUP, int OT, int NMB>
MOE_DEV void tall_unit(const GemmParams &p, const TallUnit &u, const int64_t *sRow, const StageBufs &sA,
                       bool has_nxt, bool nsh, int4 ntile, int nnb, const int64_t *sRow_nxt) {
  using C = TallCfg<WF, GQ>;
  using L = TallLoader<WF, GQ, GATEUP>;
  using Ch = TallSlot<WF, GQ>;
  constexpr bool AFF = C::AFF, MX = C::MX;
  constexpr int KS = C::KS, ROWB = C::ROWB, BPR = C::BPR;
  constexpr int NBUF = C::NBUF, D = C::D, NI = C::NI, NUS = C::NUS, LPS = C::LPS;
  constexpr int WPS = C::PPS + C::NSL;                     // weight loads per stage
  constexpr int UE = pk_ue(WF, GQ);                        // elements per unit
  constexpr int SPU = UE / 32;                             // MFMA steps per unit
  constexpr int QE = UE / 4;                               // elements per lane quarter per unit
  constexpr int LPU = pk_lb(WF, GQ) / 4;                   // weight words per lane, unit and half
  static_assert(2 * C::NU * LPU == 16, "64 weight bytes per lane per record");

  // lane-dependent values are recomputed per unit (opaque thread id): hoisted out of the
  // unit loop they would stay live across it and crowd the registers
  const int tid = (int)in_vgpr(threadIdx.x), lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, kq = lane >> 4;
  const uint32_t m0 = in_vgpr(0x000F000Fu), m1 = in_vgpr(0x00F000F0u);
  const uint32_t g0 = in_vgpr(0x64006400u), g1 = in_vgpr(0x54005400u);

  const int rows = u.rows;
  // tile row t (0..31) of this wave -> weight matrix row; GATEUP: rows 0-15 gate, 16-31 up
  const int col0 = GATEUP ? u.nb * 128 + wave * 16 : u.nb * 256 + wave * 32;
  const bool act = col0 < rows;
  auto row_of = [&](int t) { return GATEUP ? col0 + (t & 15) : col0 + t; };
  auto row_ok = [&](int t) { return row_of(t) < rows; };
  const L ld(u, sRow, wave, lane);
  const int nst = ld.nst, Kd = u.Kd;
  Ch ring[NBUF];
  ld.load_first_w(ring);

  // output bias of this lane's tile rows 16 h + 4 kq + i: loaded now (no bias: from a zero
  // block) and kept as raw bits until the epilogue, so nothing waits for them
  uint32_t bo_raw[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint16_t *bp = h ? u.bias1 : u.bias0;
    const uint16_t *bz = (const uint16_t *)&g_zero_block;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * h + 4 * kq + i;
      bo_raw[h][i] = bp ? bp[(int64_t)u.e * rows + (row_ok(t) ? row_of(t) : 0)] : bz[0];
    }
  }

  // the stage that holds the end of the reduction: its blocks past Kd hold the next row's
  // elements (or zeros past the rows); each lane zeroes its own, once its loads are in
  // (before the stage's barrier)
  auto zero_tail = [&](int c, int buf) {
    const int kc = c * KS;
#pragma unroll
    for (int n = 0; n < NI; ++n)
      if (kc + ld.ablk[n] * 8 >= Kd)
        *(u32x4_t *)(sA.b[buf] + ld.wave_u * (NI * 1024) + n * 1024 + lane * 16) = u32x4_t{0u, 0u, 0u, 0u};
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
    if constexpr (C::MXS) {  // the block-scaled MFMA takes the stored codes as they are
      b[0] = b[1] = u32x4_t{0u, 0u, 0u, 0u};
      return;
    }
    const int uu = t / SPU, s = t % SPU;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int q = (uu * 2 + h) * LPU + (C::DENSE ? 4 * s : s);   // word of the stage's lane sequence
      if constexpr (AFF) {
        const uint32_t v = ch.s[h * NUS + uu];
        const float sc = __uint_as_float(v << 16), qb = __uint_as_float(v & 0xFFFF0000u);
        if constexpr (AT == DT_F16)
          b[h] = deq_affine_h16(ch.w[q >> 2][q & 3], m0, m1, g0, g1, h16_pair(sc), h16_pair(qb));
        else
          b[h] = deq_affine<AT>(ch.w[q >> 2][q & 3], m0, m1, g0, g1, sc, fmaf(-1024.0f, sc, qb), fmaf(-64.0f, sc, qb));
      } else if constexpr (MX) {
        const float sc = e8m0_scale((ch.s[h] >> (8 * (2 * uu + (kq >> 1)))) & 0xFFu);
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
  // which bounds the live registers.  The loads of stage cl are issued from inside the
  // steps, LPS/NS per step: issued all at once they stall every wave on the address path.
  // The wave priority falls with the step, so that the wave of a SIMD pair that is behind
  // issues first and the pair reaches the stage barrier together.
  constexpr int VPS = AFF ? (AT == DT_F16 ? 28 : 40) : 12;  // VALU of one step's dequantisation
  constexpr int VPM = (VPS + 2 * NMB - 1) / (2 * NMB);     // ... per MFMA
  // (b0: step 0's B fragments, dequantised before the stage barrier, while the wave waits for
  // the others)
  // WF_MXS: a stage is one step of the block-scaled 16x16x128 MFMA.  Per row block: the
  // FP8 operand pair of the 16 tokens (hi: 16-byte blocks kq and 4 + kq of the staged row,
  // lo: 8 + kq and 12 + kq -- the operand's two 16-element halves, K = 16 kq .. and
  // 64 + 16 kq ..), the pair's E8M0 scales (Eh | El << 8) of the lane's block kq, then four
  // MFMAs: each weight half (FP4 codes as stored, E8M0 byte 2 * (c % 2) + h of the slot's
  // scale word) times hi and lo, accumulated in fp32.
  auto compute_mxs = [&](int c, int buf, const Ch &ch, bool issue, int cl, int bufl, Ch &chl) {
    constexpr int LPT = (LPS + NMB - 1) / NMB;
    const char *sAb = sA.b[buf];
    const char *sSb = sA.s[buf] + n16 * 8 + kq * 2;
    typedef int v8i_t __attribute__((ext_vector_type(8)));
    v8i_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[h] = v8i_t{(int)ch.w[h][0], (int)ch.w[h][1], (int)ch.w[h][2], (int)ch.w[h][3], 0, 0, 0, 0};
    const int sa = (int)ch.s[0];
    // row block mb's operands: read one block ahead of its MFMAs, nothing moved across blocks
    struct Ops {
      v8i_t hi, lo;
      int sb;
    };
    auto read_ops = [&](int mb) {
      const char *rp = sAb + (16 * mb + n16) * ROWB;
      const int sw = row_swizzle<BPR>(16 * mb + n16);
      const u32x4_t h0 = *(const u32x4_t *)(rp + ((kq ^ sw) << 4));
      const u32x4_t h1 = *(const u32x4_t *)(rp + (((4 + kq) ^ sw) << 4));
      const u32x4_t l0 = *(const u32x4_t *)(rp + (((8 + kq) ^ sw) << 4));
      const u32x4_t l1 = *(const u32x4_t *)(rp + (((12 + kq) ^ sw) << 4));
      Ops o;
      o.sb = (int)*(const uint16_t *)(sSb + mb * 256);
      o.hi = v8i_t{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], (int)h1[2], (int)h1[3]};
      o.lo = v8i_t{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
      return o;
    };
    Ops cur = read_ops(0);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      if (issue) {
#pragma unroll
        for (int k = mb * LPT; k < (mb + 1) * LPT && k < LPS; ++k) ld.load_k(cl, sA, bufl, chl, k);
      }
      Ops nxt = cur;
      if (mb + 1 < NMB) nxt = read_ops(mb + 1);
      if (c & 1) {
        acc[mb][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[0], cur.hi, acc[mb][0], 4, 0, 2, sa, 0, cur.sb);
        acc[mb][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[1], cur.hi, acc[mb][1], 4, 0, 3, sa, 0, cur.sb);
        acc[mb][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[0], cur.lo, acc[mb][0], 4, 0, 2, sa, 1, cur.sb);
        acc[mb][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[1], cur.lo, acc[mb][1], 4, 0, 3, sa, 1, cur.sb);
      } else {
        acc[mb][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[0], cur.hi, acc[mb][0], 4, 0, 0, sa, 0, cur.sb);
        acc[mb][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[1], cur.hi, acc[mb][1], 4, 0, 1, sa, 0, cur.sb);
        acc[mb][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[0], cur.lo, acc[mb][0], 4, 0, 0, sa, 1, cur.sb);
        acc[mb][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[1], cur.lo, acc[mb][1], 4, 0, 1, sa, 1, cur.sb);
      }
      // (the MFMAs are pure: without a use here they would sink to the epilogue, and every
      // stage's operands would stay live until then)
      asm volatile("" : "+v"(acc[mb][0]), "+v"(acc[mb][1]));
      __builtin_amdgcn_sched_barrier(0);
      cur = nxt;
    }
  };
  auto compute = [&](int c, int buf, const Ch &ch, const u32x4_t (&b0)[2], bool issue, int cl, int bufl, Ch &chl) {
    if constexpr (C::MXS) {
      compute_mxs(c, buf, ch, issue, cl, bufl, chl);
      return;
    }
    constexpr int NS = NUS * SPU;
    constexpr int LPT = (LPS + NS - 1) / NS;               // loads issued per step
    const char *sAb = sA.b[buf] + n16 * ROWB;
    u32x4_t a[NMB], bC[2] = {b0[0], b0[1]}, bN[2];
    read_a(sAb, 0, a);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      switch (3 - (t * 4) / NS) {
        case 3: __builtin_amdgcn_s_setprio(3); break;
        case 2: __builtin_amdgcn_s_setprio(2); break;
        case 1: __builtin_amdgcn_s_setprio(1); break;
        default: __builtin_amdgcn_s_setprio(0); break;
      }
      if (issue) {
#pragma unroll
        for (int k = t * LPT; k < (t + 1) * LPT && k < LPS; ++k) ld.load_k(cl, sA, bufl, chl, k);
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
  // sources into the buffer and ring slot that no later stage of the unit reads.  The
  // remaining < NBUF stages follow, in ring slots 0.., loading nothing.
  // Waves past the matrix's rows (act false) run the same code on a clamped row block and
  // drop the result: one code path keeps the compiler's wait counts exact.
  // (stage j < D of the first group: its weights were issued last in the unit's prologue,
  // followed by those of the D - 1 - j later prologue stages and the j stages' loads issued
  // since; its activations are older)
  int c0 = 0;
  for (; c0 + NBUF <= nst; c0 += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      const int c = c0 + j;
      if (j < D && c0 == 0) {
        switch (j) {   // j is known after unrolling
          case 0: wait_vmcnt<(D - 1) * WPS>(); break;
          case 1: wait_vmcnt<(D - 2) * WPS + LPS>(); break;
          default: wait_vmcnt<(D - 3 > 0 ? D - 3 : 0) * WPS + 2 * LPS>(); break;
        }
      } else {
        wait_vmcnt<(D - 1) * LPS>();
      }
      if ((c + 1) * KS > Kd) zero_tail(c, j);
      u32x4_t b0[2];
      deq_step(ring[j], 0, b0);
      asm volatile("" : "+v"(b0[0]), "+v"(b0[1]));
      stage_barrier();
      compute(c, j, ring[j], b0, true, min(c + D, nst - 1), (j + D) % NBUF, ring[(j + D) % NBUF]);
    }
  }
  // remainder stage c0 + j: its loads were issued D stages before it, followed by those of
  // D - 1 - j more stages (whole stages after the loop; only weights when it did not run)
  auto last = [&](int j, auto wait_full, auto wait_w) {
    const int c = c0 + j;
    if (c0 > 0)
      wait_full();
    else
      wait_w();
    if ((c + 1) * KS > Kd) zero_tail(c, j);
    u32x4_t b0[2];
    deq_step(ring[j], 0, b0);
    asm volatile("" : "+v"(b0[0]), "+v"(b0[1]));
    stage_barrier();
    compute(c, j, ring[j], b0, false, 0, 0, ring[j]);
  };
  if (c0 < nst) {
    last(0, [] { wait_vmcnt<(D - 1) * LPS>(); }, [] { wait_vmcnt<(D - 1) * WPS>(); });
    if constexpr (NBUF > 2) {
      if (c0 + 1 < nst) {
        last(1, [] { wait_vmcnt<(D - 2) * LPS>(); }, [] { wait_vmcnt<(D - 2) * WPS>(); });
        if constexpr (NBUF > 3) {
          if (c0 + 2 < nst) last(2, [] { wait_vmcnt<0>(); }, [] { wait_vmcnt<0>(); });
        }
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);

  // every wave is done with the stages: the next unit's first stages can load
  stage_barrier();
  if (has_nxt) {
    const L ldn(tall_unit_of<GATEUP>(p, nsh, ntile, nnb), sRow_nxt, wave, lane);
    ldn.load_first_a(sA);
  }

  // ---- epilogue: acc[mb][h][i] is tile row 16*h + 4*kq + i (weights are the MFMA's A
  // operand) and token 16*mb + n16, so every lane holds four adjacent output columns of
  // one token row and writes them with one store
  if (act) {
    float bo[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t b = bo_raw[h][i];
        asm volatile("" : "+v"(b));   // converted here, not next to the load
        bo[h][i] = bf16_bits_to_f32(b);
      }
    const float limit = u.limit;
    const int nr = u.nr, r0 = u.r0;
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
              g = clamp_act(g, limit);
              up = clamp_act(up, limit);
            }
            v[i] = silu_f(g) * up;
          }
          const int col = row_of(4 * kq);
          store4<OT>(p.out, orow + col, v, min(4, rows - col), vec);
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int col = row_of(16 * h + 4 * kq);
            const int nv = min(4, rows - col);
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
  constexpr int SSB = C::MXS ? C::NW * 256 : 16;  // scale pairs of one stage (WF_MXS)
  __shared__ __attribute__((aligned(256))) char sS0[SSB];
  __shared__ __attribute__((aligned(256))) char sS1[SSB];
  __shared__ __attribute__((aligned(256))) char sS2[SSB];
  __shared__ __attribute__((aligned(256))) char sS3[SSB];
  const StageBufs sA = {{sA0, sA1, sA2, sA3}, {sS0, sS1, sS2, sS3}};
  __shared__ int64_t sRow[2][C::MT];

  // units: segment 1 (shared expert / plain rows) first, then the routed m-tiles
  const int nblk0 = p.seg[0].nblk, nblk1 = max(p.seg[1].nblk, 1);
  const int smt = p.sh_mt > 0 ? min(p.sh_mt, C::MT) : C::MT;  // segment 1's m-tile rows
  const int ns = p.seg[1].nblk > 0 ? (p.sh_rows + smt - 1) / smt : 0;
  const int units_s = ns * nblk1;
  const int nr_routed = p.tiles ? min(p.tile_count[0], p.max_tiles) : 0;
  auto decode = [&](int u, bool &sh, int4 &tile, int &nb) {
    sh = u < units_s;
    if (sh) {
      const int ti = u / nblk1;
      nb = u - ti * nblk1;
      tile = make_int4(0, p.sh_row0 + ti * smt, min(smt, p.sh_rows - ti * smt), 0);
    } else {
      const int v = u - units_s;
      const int ti = v / max(nblk0, 1);
      nb = v - ti * nblk0;
      if (!p.tiles) return false;
      tile = p.tiles[min(ti, p.max_tiles - 1)];  // in bounds even past the end of the list
      if (ti >= nr_routed) return false;
    }
    tile.x = __builtin_amdgcn_readfirstlane(tile.x);
    tile.y = __builtin_amdgcn_readfirstlane(tile.y);
    tile.z = __builtin_amdgcn_readfirstlane(tile.z);
    return true;
  };

  const int G = gridDim.x, g = blockIdx.x;
  const int U = units_s + (p.tiles ? nr_routed * nblk0 : 0);
  const int tid = threadIdx.x;
  int r = 0, u = sched_unit(g, 0, G, U);
  bool csh, nsh;
  int4 ctile, ntile;
  int cnb, nnb;
  if (u < 0 || !decode(u, csh, ctile, cnb)) return;
  {
    const TallUnit cur = tall_unit_of<GATEUP>(p, csh, ctile, cnb);
    tall_fill_rows<C::MT>(cur, sRow[0], tid);
    __syncthreads();
    const TallLoader<WF, GQ, GATEUP> ld(cur, sRow[0], tid >> 6, tid & 63);
    ld.load_first_a(sA);
  }
  for (int par = 0;; par ^= 1) {
    const int un = sched_unit(g, r + 1, G, U);
    const bool has_nxt = un >= 0 && decode(un, nsh, ntile, nnb);
    // the next unit's rows: published by this unit's stage barriers
    if (has_nxt) tall_fill_rows<C::MT>(tall_unit_of<GATEUP>(p, nsh, ntile, nnb), sRow[par ^ 1], tid);
    const TallUnit cur = tall_unit_of<GATEUP>(p, csh, ctile, cnb);
    const int nmb = (min(cur.nr, C::MT) + 15) >> 4;
    if (nmb <= 2)
      tall_unit<AT, WF, GQ, GATEUP, OT, 2>(p, cur, sRow[par], sA, has_nxt, nsh, ntile, nnb, sRow[par ^ 1]);
    else if (nmb <= 4)
      tall_unit<AT, WF, GQ, GATEUP, OT, 4>(p, cur, sRow[par], sA, has_nxt, nsh, ntile, nnb, sRow[par ^ 1]);
    else if (nmb <= 6)
      tall_unit<AT, WF, GQ, GATEUP, OT, 6>(p, cur, sRow[par], sA, has_nxt, nsh, ntile, nnb, sRow[par ^ 1]);
    else
      tall_unit<AT, WF, GQ, GATEUP, OT, 8>(p, cur, sRow[par], sA, has_nxt, nsh, ntile, nnb, sRow[par ^ 1]);
    if (!has_nxt) break;
    csh = nsh;
    ctile = ntile;
    cnb = nnb;
    u = un;
    ++r;
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
  if (wfmt == WF_MXS) {  // split FP8 activations (their f16 source type names the kernel)
    if constexpr (AT == DT_F16) {
      if (odt == DT_F16) {
        if (gateup) launch_t<AT, WF_MXS, 0, true, DT_F16>(p, grid, s, e0, e1);
        else launch_t<AT, WF_MXS, 0, false, DT_F16>(p, grid, s, e0, e1);
        return hipGetLastError();
      }
    }
    return hipErrorInvalidValue;
  }
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
