// moe_decode.hip - the two kernels of a decode-sized batch (the weighted combine follows as
// a third launch, moe_combine.hip).
// (libmir-metal's execute hands the gate/up kernel the routing indices and the clamp limit,
// and the down kernel the same indices with the routing weights, which makes the layer
// output; mlxcel PR #1044, "Validation", describes a fused MoE kernel for one-token decode.)
//
// decode_route (ceil(T/16) * ceil(R/16) workgroups, R = experts + the blend head's 2 rows):
//   workgroup (tt, rt) computes one 16-token x 16-row tile of the router logits.  For up to
//   16 tokens the last tile to finish selects for every token (one half-wave each); for
//   more, tile (tt, rt) selects tokens 16 tt + rt + nRT h of its block once the block's
//   tiles are in.  The last selection to finish builds counts, offsets, sorted_slot,
//   slot_pos and the m-tile list.
//   The launch also clears the m-tile counters of the experts launch that follows, and the
//   permuting workgroup clears the launch's own counters.
// decode_fused (persistent: at most what the device holds at once):
//   the work units of the loader-wave decode GEMM (moe_gemm_ws.hip: m-tile of up to 16 rows x
//   4 row blocks of the packed stream; loader waves stream records HBM -> LDS, compute waves
//   fold each quantisation group exactly), gate/up units first, then down units, so the down
//   weights stream while gate/up work finishes elsewhere; a down unit waits until every
//   gate/up wave of its m-tile has stored its h rows.  The per-slot outputs o are written in
//   token order (row t*K + j, then T*K + t for the shared expert), which the combine launch
//   reads.  (Combining in this launch, by the wave whose down unit completed a 32-column
//   block of o, put the combine's loads on the launch's tail and measured slower.)
//
// The single launch (opt-in, up to 16 tokens: decode_fused with ONE): workgroups g < R/16
// first compute the router tiles; the last of them selects and permutes, stores the ids,
// weights, coefficients and m-tile list at device scope and sets a flag kept in 32 lines.
// The units are ordered [gate/up shared][down shared][gate/up routed][down routed], so the
// shared expert runs while the routing is computed; workgroup g takes units G-1-g, 2G-1-g,
// ... (the router workgroups the last ones), and a routed unit waits for the flag.  Each
// down wave counts its 32 output columns once its o rows are stored, and the wave that
// completes a column block (the last m-tile to get there) combines those columns for every
// token, in the combine launch's arithmetic.  Each call clears the other of two counter
// blocks for the next call, so no grid-wide count is needed at the end.  It gives the three
// launches' bits and is no faster than them on MI355X (1 and 8 tokens: the same, 16: slower,
// with two workgroups per CU), so it is not the default.
//
// Hand-overs between workgroups (on different XCDs, each with its own L2) carry their data
// as device-scope stores (sc1: the instructions the compiler emits for agent-scope relaxed
// atomic stores, coherent across the XCDs), wait until those have completed (vmcnt 0), then
// bump a counter; the reader sees the count and reads with device-scope loads.  No L2
// write-back or invalidate is needed; an agent-scope release fence per wave and unit, which
// writes back the whole L2 of the XCD, made the launch several times slower.  Counters sit
// one per 128-byte line and are polled every ~0.25 us (back-to-back polling of one line
// loaded a memory channel enough to slow the launch threefold).  Every wait is bounded: one
// that gives up (only possible if the grid were not co-resident) sets the status word and
// lets the waves run to their end.
#include <hip/hip_ext.h>

#include "moe_topk.h"
#include "moe_ws.h"

namespace {

// A device-scope poll goes to memory (it must not be served by a stale L2 line), so polls are
// spaced out (~0.25 us: s_sleep 10 is 640 clocks).
constexpr int kSpinLimit = 1 << 19;  // polls of a counter, ~0.15 s in all
constexpr int kSC1 = 16;             // cache-policy bit of device-scope (sc1) buffer accesses

// waits until *c >= target (device-scope loads of the counter by the calling lane `lane` of
// the wave's active lanes; lane 0 when the whole wave calls)
MOE_DEV bool wait_count(const int *c, int target, int *status, int lane) {
  for (int it = 0; it < kSpinLimit; ++it) {
    int v = 0;
    if (lane == 0) v = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__builtin_amdgcn_readfirstlane(v) >= target) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      return true;
    }
    __builtin_amdgcn_s_sleep(10);
  }
  if (lane == 0) __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// the calling wave's stores have completed (device-scope stores: visible to every XCD),
// then lane 0 adds 1 to *c; returns the value before the add (wave-uniform)
MOE_DEV int publish(int *c, int lane) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_amdgcn_readfirstlane(old);
}

}  // namespace

// router tiles, selection and permutation (see the top of the file); SL: logits per lane of
// a half-wave in the selection (E <= 32 SL)
template <int SL>
__global__ __launch_bounds__(512) void decode_route(const FusedParams p) {
  __shared__ float red[8][16][17];
  __shared__ int el[16][16];
  __shared__ float esc[16][16];
  __shared__ int32_t sidx[16 * 16];  // the selected ids of a single token block (K <= 16)
  __shared__ DecodePermSmem<512> perm;
  __shared__ int last;
  const int tid = threadIdx.x, g = blockIdx.x, G = gridDim.x;
  const TopkArgs &ta = p.ta;
  const int T = ta.T, E = ta.E;
  const int nTT = (T + 15) / 16, nRT = (E + (p.cw ? 2 : 0) + 15) / 16;
  if (g == 0 && tid == 0) *p.status = 0;
  // the experts launch's m-tile counters
  for (int i = g * 512 + tid; i < p.n_tile_cnt; i += G * 512) p.cnt[kTileCnt0 + i * kCntStride] = 0;
  const int tt = g / nRT, rt = g - tt * nRT;
  // the selection biases, in case this workgroup is the one that selects (loaded now, so
  // that the selection does not wait for them)
  const int half = tid >> 5, l32 = tid & 31;
  float sb[SL];
  topk_half_sbias<SL>(ta, l32, sb);
  router_tile_bf16<true>(p.x, p.Wr, p.lbias, (float *)ta.logits, T, p.H, E, p.cw, p.cb, (float *)ta.clog, tt, rt,
                         red);
  wait_vmcnt<0>();  // this thread's logit stores have completed
  __syncthreads();
  if (nTT == 1) {
    // a single token block: the last tile to finish selects for every token (one half-wave
    // each) and permutes, the ids kept in LDS
    if (tid == 0)
      last = __hip_atomic_fetch_add(p.cnt + kTileDone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1;
    __syncthreads();
    if (!last) return;
    // only the waves with a live token (a dead half-wave of one works on a token past the
    // end and stores nothing): idle waves would share the SIMDs' issue slots
    if ((tid >> 6) < (T + 1) / 2) topk_half<SL, true>(ta, half, l32, el[half], esc[half], sidx, false);
    __syncthreads();
    decode_permute<512, false, true>(sidx, T, ta.K, E, p.counts, p.offsets, (int32_t *)p.gu.seg[0].A.gather,
                                     p.slot_pos, (int4 *)p.gu.tiles, (int *)p.gu.tile_count, 16, perm);
    if (tid == 0) p.cnt[kTileDone] = 0;  // every other workgroup has counted itself: clear
    return;
  }
  // several token blocks: once every tile of its block is in, tile (tt, rt) selects tokens
  // 16 tt + rt + nRT h of the block, half-wave h each (spreading the selections over the
  // block's workgroups keeps each to one short pass, where the selection arithmetic of 16
  // tokens on one workgroup took ~4 us), and the last workgroup to finish selecting
  // permutes.  The waits are on tiles of the same small grid, all resident at once.
  if (tid == 0) __hip_atomic_fetch_add(p.cnt + kTtCnt0 + tt * kCntStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int nbt = min(16, T - 16 * tt);  // tokens of this block
  if (rt >= nbt) return;                 // no token for this tile
  const int nh = (nbt - 1 - rt) / nRT + 1;  // its tokens: half-waves 0 .. nh - 1
  if (tid == 0) wait_count(p.cnt + kTtCnt0 + tt * kCntStride, nRT, p.status, 0);
  __syncthreads();
  if ((tid >> 6) < (nh + 1) / 2) {  // waves with a token; a half without one works on a
                                    // token past the end and stores nothing
    float lg[SL];
    float2 cp;
    const int tq = half < nh ? 16 * tt + rt + nRT * half : T;
    topk_half_load<SL, true>(ta, tq, l32, lg, cp);
    topk_half_select<SL>(ta, tq, l32, lg, cp, sb, el[half], esc[half], nullptr, true);
    wait_vmcnt<0>();  // this thread's id, weight and coefficient stores have completed
  }
  __syncthreads();
  // selecting workgroups: min(nRT, tokens) per block
  int nsel = 0;
  for (int b = 0; b < nTT; ++b) nsel += min(nRT, min(16, T - 16 * b));
  if (tid == 0)
    last = __hip_atomic_fetch_add(p.cnt + kSelCnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsel - 1;
  __syncthreads();
  if (!last) return;
  decode_permute<512, false>(ta.idx, T, ta.K, E, p.counts, p.offsets, (int32_t *)p.gu.seg[0].A.gather, p.slot_pos,
                             (int4 *)p.gu.tiles, (int *)p.gu.tile_count, 16, perm);
  // every workgroup with a token has passed its wait and counted itself: clear
  for (int i = tid; i <= nTT; i += 512) p.cnt[i == 0 ? kSelCnt : kTtCnt0 + (i - 1) * kCntStride] = 0;
}

// ONE: the single launch of up to 16 tokens (router tiles, selection and permutation first,
// the combine at the end; see the top of the file)
template <int AT, int WF, int GQ, int IT, bool ONE>
__global__ __launch_bounds__(512, ONE ? 4 : 6) void decode_fused(const FusedParams p) {
  using C = WsCfg<WF, GQ>;
  constexpr bool AFF = C::AFF;
  constexpr int MT = 16, KC = C::KC, UE = C::UE, SPU = C::SPU, QE = C::QE, LPU = C::LPU, NU = C::NU;
  constexpr int RB = C::RB, SW = C::SW, STAGE = C::STAGE, NBUF = C::NBUF, NDMA = C::NDMA;
  constexpr float MAGIC = AT == DT_BF16 ? 128.0f : 1024.0f;
  __shared__ __attribute__((aligned(16))) char smem[NBUF * STAGE];
  __shared__ int uq[2];  // ONE: the workgroup's next units (-1: none left)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = gridDim.x, g = blockIdx.x;

  // ---- the unit list: [gate/up: shared m-tiles, routed m-tiles][down: shared, routed]
  const int nbg0 = p.gu.seg[0].nblk, nbg1 = p.gu.seg[1].nblk, nbd0 = p.dn.seg[0].nblk, nbd1 = p.dn.seg[1].nblk;
  const int sh_rows = p.gu.sh_rows, sh_row0 = p.gu.sh_row0, max_tiles = p.gu.max_tiles, n_exp = p.gu.E;
  const int4 *const tiles = p.gu.tiles;
  const int *const tcount = p.gu.tile_count;
  asm volatile("" ::"s"(nbg0), "s"(nbg1), "s"(nbd0), "s"(nbd1), "s"(sh_rows), "s"(sh_row0), "s"(max_tiles),
               "s"(tiles), "s"(tcount));
  const int ns = nbg1 > 0 ? (sh_rows + MT - 1) / MT : 0;  // shared m-tiles
  // routed m-tiles: written by the routing launch, or (ONE) by this launch's routing, known
  // once the routing flag is set
  int nr = ONE ? 0 : min(max(load_uniform_int(tcount), 0), max_tiles);
  const int Ug_s = ns * nbg1, Ud_s = ns * nbd1;
  int Ug = Ug_s + nr * nbg0;
  const int U = Ug + Ud_s + nr * nbd0;  // (not ONE)
  // counters, one per 128-byte line: gate/up waves done per m-tile [ns + max_tiles]
  int *const tile_cnt = p.cnt + kTileCnt0;

  struct Unit {
    bool dn, sh;
    int e, r0, nr, nb, tile;
  };
  // the routed m-tile ti of the list (ONE: written in this launch, read at device scope)
  auto tile_entry = [&](int ti) {
    const int4 *tp = tiles + min(max(ti, 0), max_tiles - 1);
    if constexpr (ONE) {
      const int *q = (const int *)tp;
      int4 t;
      t.x = __builtin_amdgcn_readfirstlane(__hip_atomic_load(q + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      t.y = __builtin_amdgcn_readfirstlane(__hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      t.z = __builtin_amdgcn_readfirstlane(__hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      t.w = 0;
      return t;
    } else {
      return load_uniform_int4(tp);
    }
  };
  // unit u: not ONE [gate/up: shared, routed][down: shared, routed]; ONE [gate/up shared]
  // [down shared][gate/up routed][down routed], so that the shared units come before the
  // routing is known
  auto unit_at = [&](int u) {
    Unit x;
    int v, us;
    if constexpr (ONE) {
      const int Us = Ug_s + Ud_s;
      if (u < Us) {
        x.dn = u >= Ug_s;
        v = x.dn ? u - Ug_s : u;
        us = v + 1;  // shared
      } else {
        const int w = u - Us, ugr = nr * nbg0;
        x.dn = w >= ugr;
        v = x.dn ? w - ugr : w;
        us = 0;  // routed
      }
    } else {
      x.dn = u >= Ug;
      v = x.dn ? u - Ug : u;
      us = x.dn ? Ud_s : Ug_s;
    }
    x.sh = v < us;
    if (x.sh) {
      const int nb1 = max(x.dn ? nbd1 : nbg1, 1);
      const int ti = min(v / nb1, max(ns - 1, 0));
      x.nb = v - ti * nb1;
      x.e = 0;
      x.r0 = sh_row0 + ti * MT;
      x.nr = min(MT, sh_rows - ti * MT);
      x.tile = ti;
    } else {
      v -= us;
      const int nb0 = max(x.dn ? nbd0 : nbg0, 1);
      const int ti = min(v / nb0, max_tiles - 1);
      x.nb = v - ti * nb0;
      // (clamped into range: whatever the list held, no access leaves its buffer)
      const int4 t = tile_entry(ti);
      x.e = min(max(t.x, 0), n_exp - 1);
      x.r0 = min(max(t.y, 0), sh_row0 - 1);
      x.nr = min(max(t.z, 1), min(MT, sh_row0 - x.r0));
      x.tile = ns + ti;
    }
    return x;
  };
  // a field of the unit's segment, selected field by field (a selected struct would go to scratch)
#define SEG(x, f) \
  ((x).dn ? ((x).sh ? p.dn.seg[1].f : p.dn.seg[0].f) : ((x).sh ? p.gu.seg[1].f : p.gu.seg[0].f))
  auto nch_of = [&](const Unit &x) { return (SEG(x, K) + KC - 1) / KC; };
  auto nch_u = [&](int u) {  // the same from the unit index alone (no tile read; not ONE)
    const bool dn = u >= Ug;
    const int v = dn ? u - Ug : u;
    const bool sh = v < (dn ? Ud_s : Ug_s);
    const int Kd = dn ? (sh ? p.dn.seg[1].K : p.dn.seg[0].K) : (sh ? p.gu.seg[1].K : p.gu.seg[0].K);
    return (Kd + KC - 1) / KC;
  };
  // ONE: the routing flag (this workgroup's copy) holds 1 + the routed m-tile count once the
  // routing is stored
  const int *const flag = p.cnt + kFlag0 + (g % kFlagCopies) * kCntStride;
  bool have_nr = !ONE;
  auto set_nr = [&](int f) {
    nr = min(max(f - 1, 0), min(max_tiles, p.nr_ub));
    Ug = Ug_s + nr * nbg0;
    have_nr = true;
  };
  // the count, once the flag has been seen set (by this wave, or by loader wave 0 before a
  // barrier this wave has passed)
  auto learn_nr = [&]() {
    if (!have_nr) set_nr(__builtin_amdgcn_readfirstlane(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)));
  };
  // ONE: unit u of this workgroup's sequence if it exists (a routed one waits for the routing)
  auto unit_if = [&](int u) {
    const int Us = Ug_s + Ud_s;
    if (u < Us) return u;
    if (!have_nr) {
      int f = 0;
      for (int it = 0; it < kSpinLimit; ++it) {
        f = __builtin_amdgcn_readfirstlane(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (f > 0) break;
        __builtin_amdgcn_s_sleep(10);
      }
      if (f <= 0 && lane == 0) __hip_atomic_store(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      set_nr(f);
    }
    return u < Us + nr * (nbg0 + nbd0) ? u : -1;
  };
  // gate/up waves that write an m-tile's h rows: 4 per column block of its segment
  auto tile_target = [&](const Unit &x) { return 4 * (x.sh ? nbg1 : nbg0); };

  int v0 = g;  // the first unit (not ONE: units g, g + G, ...)
  if constexpr (ONE) {
    const TopkArgs &ta = p.ta;
    const int T = ta.T, E = ta.E;
    const int nRT = (E + (p.cw ? 2 : 0) + 15) / 16;
    if (g == 0 && tid == 0) __hip_atomic_store(p.status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the next call's counters start at zero
    if (g == G - 1) {
      for (int i = tid; i < 1 + kMaxTileCnt + kMaxColCnt + kFlagCopies; i += 512) {
        // kTileDone, then the m-tile counters, the column counters and the flag copies (one
        // contiguous run of lines from kTileCnt0 on)
        p.cnt_next[i == 0 ? kTileDone : kTileCnt0 + (i - 1) * kCntStride] = 0;
      }
    }
    if (g < nRT) {
      // router tile (0, g); the last tile to finish selects for every token (one half-wave
      // each) and permutes; the ids, weights, coefficients and m-tile list are stored at
      // device scope for the workgroups of this launch, then the routing flag is set.  Its
      // LDS is the stage buffers', unused until the units start.
      float (*red)[16][17] = (float (*)[16][17])smem;
      int (*el)[16] = (int (*)[16])(smem + 8 * 16 * 17 * 4);
      float (*esc)[16] = (float (*)[16])(smem + 8 * 16 * 17 * 4 + 1024);
      int32_t *sidx = (int32_t *)(smem + 8 * 16 * 17 * 4 + 2048);
      DecodePermSmem<512> &perm = *(DecodePermSmem<512> *)(smem + 8 * 16 * 17 * 4 + 3072);
      static_assert(8 * 16 * 17 * 4 + 3072 + sizeof(DecodePermSmem<512>) <= NBUF * STAGE, "routing LDS");
      const int half = tid >> 5, l32 = tid & 31;
      router_tile_bf16<true>(p.x, p.Wr, p.lbias, (float *)ta.logits, T, p.H, E, p.cw, p.cb, (float *)ta.clog, 0, g,
                             red);
      wait_vmcnt<0>();  // this thread's logit stores have completed
      __syncthreads();
      if (tid == 0)
        uq[1] = __hip_atomic_fetch_add(p.cnt + kTileDone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nRT - 1;
      __syncthreads();
      if (uq[1]) {
        if ((tid >> 6) < (T + 1) / 2) topk_half<8, true>(ta, half, l32, el[half], esc[half], sidx, true);
        __syncthreads();
        const int ntl = decode_permute<512, true, true>(sidx, T, ta.K, E, p.counts, p.offsets,
                                                        (int32_t *)p.gu.seg[0].A.gather, p.slot_pos,
                                                        (int4 *)p.gu.tiles, (int *)p.gu.tile_count, 16, perm);
        wait_vmcnt<0>();  // this thread's stores have completed
        __syncthreads();
        if (tid < kFlagCopies)
          __hip_atomic_store(p.cnt + kFlag0 + tid * kCntStride, 1 + ntl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();  // the routing LDS is free
    }
    // units G-1-g, 2G-1-g, ...: the router workgroups take the last ones
    if (wave == 4) {
      const int v = unit_if(G - 1 - g);
      if (lane == 0) uq[0] = v;
    }
    stage_barrier();
    v0 = __builtin_amdgcn_readfirstlane(uq[0]);
    if (v0 < 0) return;
  } else {
    if (g >= U) return;
  }

  if (wave >= 4) {
    // ---------------- loader waves: row block lw's records, activation rows 4 lw .. 4 lw + 3
    const int lw = wave - 4;
    __amdgpu_buffer_rsrc_t wrs, ars;
    uint32_t wvo = 0, svo = 0, avo[2] = {0u, 0u};
    bool aon[2] = {true, true};
    int cu = g, cc = 0, cn = 0;
    Unit cur;
    bool a_pending = false;  // the current unit's activation rows are not yet addressed
    auto enter_w = [&](const Unit &x) {
      cn = nch_of(x);
      const char *pk = SEG(x, w0.pk);
      const int64_t pk_mat = SEG(x, w0.pk_mat);
      const int pk_nblk = SEG(x, w0.pk_nblk), pk_nch = SEG(x, w0.pk_nch);
      wrs = __builtin_amdgcn_make_buffer_rsrc((void *)(pk + (int64_t)x.e * pk_mat), (short)0, (int)pk_mat,
                                              0x00020000);
      const uint32_t rbo = (uint32_t)min(x.nb * 4 + lw, pk_nblk - 1) * (uint32_t)(pk_nch * RB);
      wvo = rbo + lane * 16;
      svo = rbo + 4096 + lane * (C::SB == 1024 ? 16 : 4);
    };
    // the unit's activation rows: gathered x rows (gate/up), or its h rows once every gate/up
    // wave of its m-tile has stored them (down)
    auto enter_a = [&](const Unit &x) {
      if (x.dn) wait_count(tile_cnt + x.tile * kCntStride, tile_target(x), p.status, lane);
      const void *a = SEG(x, A.a);
      const int64_t lda = SEG(x, A.lda), arows = SEG(x, A.rows);
      ars = __builtin_amdgcn_make_buffer_rsrc((void *)a, (short)0, (int)(arows * lda * 2), 0x00020000);
      const int32_t *gat = SEG(x, A.gather);
      const int gdiv = SEG(x, A.gdiv), rsub = SEG(x, A.row_sub);
      uint32_t ro[4];
      int gi[4];
      if (gat) {
        const int *g0 = gat + x.r0;
        if (ONE && !x.sh) {  // the gather list of this launch's routing: device scope
#pragma unroll
          for (int k = 0; k < 4; ++k)
            gi[k] = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(g0 + min(4 * lw + k, x.nr - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        } else {
          load_uniform_ints4(g0 + min(4 * lw, x.nr - 1), g0 + min(4 * lw + 1, x.nr - 1),
                             g0 + min(4 * lw + 2, x.nr - 1), g0 + min(4 * lw + 3, x.nr - 1), gi);
        }
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
    // one stage: the weights first, then (after a down unit's wait) the activation rows
    auto issue = [&](int b) {
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
      if (a_pending) {
        enter_a(cur);
        a_pending = false;
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        lds_void_t *dst = (lds_void_t *)(base + SW + (2 * lw + n) * 1024);
        const int so2 = cc * KC * 2;
        if (cur.dn) {  // h rows written by other workgroups in this launch: device scope
          if (aon[n])
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, dst, 16, avo[n], so2, 0, kSC1);
          else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, dst, 4, avo[n], so2, 0, kSC1);
        } else {
          if (aon[n])
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, dst, 16, avo[n], so2, 0, 0);
          else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, dst, 4, avo[n], so2, 0, 0);
        }
      }
    };
    if constexpr (ONE) {
      // the unit sequence G-1-g, + G, ...: loader wave 0 finds the next unit once the
      // current one's last stage is on its way, and hands it over through LDS.  (A routed
      // unit is decoded only with the routed m-tile count: loader wave 0 has seen the routing
      // flag before the barrier that handed the unit over.)
      if (v0 >= Ug_s + Ud_s) learn_nr();
      cur = unit_at(v0);
      cn = nch_of(cur);
      enter_w(cur);
      a_pending = true;
      issue(0);
      for (int st = 0, k = 0, un = v0;; ++st) {
        if (cc == cn - 1 && lw == 0) {
          const int v = unit_if(un + G);
          if (lane == 0) uq[(k + 1) & 1] = v;
        }
        wait_vmcnt<0>();  // stage st has landed
        stage_barrier();  // stage st is handed over; the buffer of stage st - 1 is free
        if (cc + 1 < cn) {
          ++cc;
        } else {
          const int v = __builtin_amdgcn_readfirstlane(uq[(k + 1) & 1]);
          if (v < 0) break;
          ++k;
          un = v;
          if (v >= Ug_s + Ud_s) learn_nr();
          cur = unit_at(v);
          cn = nch_of(cur);
          enter_w(cur);
          a_pending = true;
          cc = 0;
        }
        issue((st + 1) % NBUF);
      }
      wait_vmcnt<0>();
      return;
    }
    // past the last unit the cursor stays on the last stage (reloaded into free buffers)
    auto advance = [&]() {
      if (cc + 1 < cn) {
        ++cc;
      } else if (cu + G < U) {
        cu += G;
        cur = unit_at(cu);
        enter_w(cur);
        a_pending = true;
        cc = 0;
      }
    };
    cur = unit_at(g);
    enter_w(cur);
    a_pending = true;
    issue(0);
    advance();
    wait_vmcnt<0>();  // stage 0 has landed
    int s = 0;
    for (int u = g; u < U; u += G) {
      const int n = nch_u(u);
      for (int c = 0; c < n; ++c, ++s) {
        stage_barrier();  // stage s is handed over; the buffer of stage s - 1 is free
        issue((s + 1) % NBUF);
        advance();
        wait_vmcnt<0>();  // stage s + 1 has landed
      }
    }
    wait_vmcnt<0>();
    return;
  }
  static_assert(NBUF == 2, "one stage in flight");
  (void)NDMA;

  // ---------------- compute waves: row block `wave` of the unit
  const int n16 = lane & 15, kq = lane >> 4;
  const uint32_t msk = in_vgpr(0x000F000Fu);
  const uint32_t mag = in_vgpr(AT == DT_BF16 ? 0x43004300u : 0x64006400u);
  const int Dout = p.Dout;
  // ONE: y for columns c0 .. c0 + 31 of every token, from the o rows of this launch (device
  // scope): the weighted sum over the slots in ascending order, then the shared expert added
  // or blended, in the combine launch's arithmetic.  Lane: token lane / 4, 8 columns.
  auto combine_cols = [&](int c0) {
    const TopkArgs &ta = p.ta;
    const int T = ta.T, K = ta.K, t = lane >> 2, c = c0 + 8 * (lane & 3);
    if (t >= T) return;
    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
        p.dn.out, (short)0, (int)((int64_t)(T * K + (p.mode >= 2 ? T : 0)) * Dout * 2), 0x00020000);
    auto row8 = [&](int r, float (&f)[8]) {
      const u32x4_t v = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ors, (uint32_t)(((int64_t)r * Dout + c) * 2), 0, kSC1));
      unpack8<DT_BF16>(v, f);
    };
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < K; ++j) {
      const float w = __uint_as_float(
          __hip_atomic_load((const uint32_t *)ta.w + (int64_t)t * K + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      float f[8];
      row8(t * K + j, f);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = fmaf(w, f[q], v[q]);
    }
    if (p.mode >= 2) {
      float sv[8];
      row8(T * K + t, sv);
      if (p.mode == 2) {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] += sv[q];
      } else {
        const float c0b = __uint_as_float(
            __hip_atomic_load((const uint32_t *)ta.coef + 2 * t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        const float c1b = __uint_as_float(
            __hip_atomic_load((const uint32_t *)ta.coef + 2 * t + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = fmaf(c0b, v[q], c1b * sv[q]);
      }
    }
    const int64_t yi = (int64_t)t * p.ldy + c;
    if (p.ydt == DT_F32) {
      float *yp = (float *)p.y + yi;
      *(f32x4_t *)yp = f32x4_t{v[0], v[1], v[2], v[3]};
      *(f32x4_t *)(yp + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
    } else {
      u32x4_t wv;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        wv[q] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * q]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v[2 * q + 1]) << 16);
      *(u32x4_t *)((uint16_t *)p.y + yi) = wv;
    }
  };
  int s = 0;
  for (int k = 0, u = v0; ONE ? u >= 0 : u < U; ++k, u = ONE ? __builtin_amdgcn_readfirstlane(uq[k & 1]) : u + G) {
    if (ONE && u >= Ug_s + Ud_s) learn_nr();
    const Unit x = unit_at(u);
    const bool gu = !x.dn;
    const int Kd = SEG(x, K), n = nch_of(x), rows = SEG(x, w0.rows);
    const float limit = SEG(x, limit);
    const int col0 = gu ? x.nb * 64 + wave * 16 : x.nb * 128 + wave * 32;
    const bool act = col0 < rows;
    auto row_of = [&](int t) { return gu ? col0 + (t & 15) : col0 + t; };
    auto row_ok = [&](int t) { return row_of(t) < rows; };
    const uint16_t *bp[2] = {(const uint16_t *)SEG(x, w0.bias),
                             (const uint16_t *)(gu ? SEG(x, w1.bias) : SEG(x, w0.bias))};
    uint32_t bbits[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 16 * h + n16;
      const uint16_t *ba = bp[h] ? bp[h] + (int64_t)x.e * rows + (row_ok(t) ? row_of(t) : 0)
                                 : (const uint16_t *)p.cnt;
      bbits[h] = *ba;
    }
    // down units: the o row of each of the lane's tokens 4 kq + i (token order: the slot,
    // whose number the gather list holds, or T*K + t for the shared expert's rows)
    int orow[4];
    if (x.dn) {
      const int32_t *gat = p.gu.seg[0].A.gather;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = min(4 * kq + i, x.nr - 1);
        const int gs = x.sh ? 0
                   : (ONE ? __hip_atomic_load(gat + x.r0 + m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : gat[x.r0 + m]);
        orow[i] = x.sh ? x.r0 + m : min(max(gs, 0), sh_row0 - 1);
      }
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
      auto mfmas = [&](int uu) {
        constexpr uint32_t ONE2 = (AT == DT_BF16) ? 0x3F803F80u : 0x3C003C00u;
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
    if (gu) {
      if (act) {
        // h = silu(g) * u for token 4 kq + i and output col0 + n16; lanes n16 and n16 + 1
        // pair their values so each pair goes out as one 32-bit device-scope store
        uint32_t *hout = (uint32_t *)p.gu.out;
        const int64_t ldh = p.gu.ldo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * kq + i;
          float gv = acc[0][i] + bo[0], up = acc[1][i] + bo[1];
          if (limit > 0.f) {
            gv = clamp_act(gv, limit);
            up = clamp_act(up, limit);
          }
          uint16_t hb;
          if constexpr (IT == DT_BF16)
            hb = __builtin_bit_cast(uint16_t, (__bf16)(silu_f(gv) * up));
          else
            hb = __builtin_bit_cast(uint16_t, (_Float16)(silu_f(gv) * up));
          const uint32_t nb_bits = (uint32_t)__shfl_xor((int)hb, 1, 64) & 0xFFFFu;
          if (m < x.nr && !(n16 & 1) && row_ok(n16))
            __hip_atomic_store(hout + (((int64_t)(x.r0 + m) * ldh + row_of(n16)) >> 1), (uint32_t)hb | (nb_bits << 16),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      // every wave of the unit reports, whether or not it had rows to write.  Now, not
      // deferred: the loaders of this workgroup may already wait for this m-tile's count
      // before the next stage barrier, which the compute waves reach only after reporting
      publish(tile_cnt + x.tile * kCntStride, lane);
    } else if constexpr (ONE) {
      // o in token order at device scope (lanes n16 and n16 + 1 pair their values into one
      // 32-bit store), then the count of this wave's 32 output columns; the wave that completes
      // them (the last of the m-tiles) combines those columns for every token
      uint32_t *o32 = (uint32_t *)p.dn.out;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * kq + i;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = 16 * h + n16;
          const uint16_t hb = __builtin_bit_cast(uint16_t, (__bf16)(acc[h][i] + bo[h]));
          const uint32_t nb_bits = (uint32_t)__shfl_xor((int)hb, 1, 64) & 0xFFFFu;
          if (act && m < x.nr && !(n16 & 1) && row_ok(t))
            __hip_atomic_store(o32 + (((int64_t)orow[i] * Dout + row_of(t)) >> 1), (uint32_t)hb | (nb_bits << 16),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (col0 < Dout) {
        const int cb = col0 / 32;
        const int old = publish(p.cnt + kColCnt0 + cb * kCntStride, lane);
        // before the routing is stored no routed down unit has run, so this one is not the
        // last of its columns (there is at least one routed m-tile)
        if (!have_nr) {
          const int f = __builtin_amdgcn_readfirstlane(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          if (f > 0) set_nr(f);
        }
        if (have_nr && old == ns + nr - 1) combine_cols(col0);
      }
    } else {
      // o in token order; the combine launch that follows reads it (plain stores: the launch
      // boundary orders them)
      if (act) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * kq + i;
          if (m >= x.nr) continue;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int t = 16 * h + n16;
            if (row_ok(t)) store_act<IT>(p.dn.out, (int64_t)orow[i] * Dout + row_of(t), acc[h][i] + bo[h]);
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

template <int AT, int WF, int GQ, int IT, bool ONE>
hipError_t fused_launch_t(const FusedParams &p, int units_ub, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  auto kern = decode_fused<AT, WF, GQ, IT, ONE>;
  // persistent: every workgroup must be resident at once (the down units wait for gate/up
  // units of other workgroups), so the grid is capped at what the device holds
  static int per_cu[64] = {0};  // (per instantiation)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!per_cu[dev]) {
    int n = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 512, 0);
    if (e != hipSuccess) return e;
    per_cu[dev] = n > 0 ? n : -1;
  }
  if (per_cu[dev] < 0) return hipErrorInvalidConfiguration;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return hipErrorInvalidDevice;
  const int cap = per_cu[dev] * cus;
  int grid = units_ub < cap ? units_ub : cap;
  if (ONE) {  // at least the router tiles
    const int nrt = (p.ta.E + (p.cw ? 2 : 0) + 15) / 16;
    if (nrt > cap) return hipErrorInvalidConfiguration;
    grid = grid > nrt ? grid : nrt;
  }
  if (grid <= 0) return hipSuccess;
  if (e0)
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, e0, e1, 0, p);
  else
    hipLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_route(const FusedParams &p, hipStream_t s) {
  const int E = p.ta.E;
  if (p.ta.T <= 0 || p.ta.T > MOE_ROUTE_SMALL_T || E > 256 || p.H % 32 != 0) return hipErrorInvalidValue;
  const int grid = (p.ta.T + 15) / 16 * ((E + (p.cw ? 2 : 0) + 15) / 16);
  if (E <= 128)
    hipLaunchKernelGGL(decode_route<4>, dim3(grid), dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL(decode_route<8>, dim3(grid), dim3(512), 0, s, p);
  return hipGetLastError();
}

// h and o are stored in the MFMA type of the down projection (bf16 activations: bf16)
template <bool ONE>
static hipError_t fused_dispatch(int wfmt, int group, int idt, const FusedParams &p, int units_ub, hipStream_t s,
                                 hipEvent_t e0, hipEvent_t e1) {
  if (idt != DT_BF16) return hipErrorInvalidValue;
  if (wfmt == WF_MXFP4) return fused_launch_t<DT_BF16, WF_MXFP4, 0, DT_BF16, ONE>(p, units_ub, s, e0, e1);
  if (wfmt == WF_AFFINE4) {
    if (group == 32) return fused_launch_t<DT_BF16, WF_AFFINE4, 32, DT_BF16, ONE>(p, units_ub, s, e0, e1);
    if (group == 64) return fused_launch_t<DT_BF16, WF_AFFINE4, 64, DT_BF16, ONE>(p, units_ub, s, e0, e1);
    if (group == 128) return fused_launch_t<DT_BF16, WF_AFFINE4, 128, DT_BF16, ONE>(p, units_ub, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_fused(int wfmt, int group, int idt, const FusedParams &p, int units_ub, hipStream_t s,
                               hipEvent_t e0, hipEvent_t e1) {
  return fused_dispatch<false>(wfmt, group, idt, p, units_ub, s, e0, e1);
}

// one launch for a batch of up to 16 tokens: router, selection, permutation, gate/up, down and
// the combine (y of ydt DT_F32 or DT_BF16, hidden a multiple of 32 and at most 32 kMaxColCnt)
hipError_t launch_decode_one(int wfmt, int group, int idt, const FusedParams &p, int units_ub, hipStream_t s,
                             hipEvent_t e0, hipEvent_t e1) {
  if (p.ta.T <= 0 || p.ta.T > 16 || p.ta.E > 256 || p.H % 32 != 0 || p.Dout % 32 != 0 ||
      p.Dout > 32 * kMaxColCnt || (p.ydt != DT_F32 && p.ydt != DT_BF16) || !(p.mode == 0 || p.mode == 2 || p.mode == 3) ||
      p.cnt_next == nullptr || p.cnt_next == p.cnt)
    return hipErrorInvalidValue;
  return fused_dispatch<true>(wfmt, group, idt, p, units_ub, s, e0, e1);
}
