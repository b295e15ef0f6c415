// moe_topk.h - scores, selection and the decode-sized permutation, shared by the routing
// kernels (moe_route.hip) and the one-launch decode experts (moe_decode.hip).
//
// Selection follows mlxcel PR #1044 point 3 (sigmoid scores in fp32, a per-expert bias added
// to a copy used only for ranking, weights gathered from the unbiased scores, optional
// renormalisation) and ferrox-models latent_moe.rs (route_top_k_sigmoid_with_bias); ties in
// the selection key go to the lower expert id and a token's K chosen ids are written in
// ascending order.
#pragma once

#include "moe_mfma.h"

namespace {

MOE_DEV uint32_t ord_key(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);  // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int CTRL>
MOE_DEV uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

MOE_DEV uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// maximum over the 64 lanes (every lane must be active); the result is wave-uniform
MOE_DEV uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp64<0xB1>(v));   // quad_perm [1,0,3,2]
  v = umax64(v, dpp64<0x4E>(v));   // quad_perm [2,3,0,1]
  v = umax64(v, dpp64<0x141>(v));  // row_half_mirror
  v = umax64(v, dpp64<0x140>(v));  // row_mirror: every lane holds its row's maximum
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * r);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * r);
    m = umax64(m, ((uint64_t)hi << 32) | lo);
  }
  return m;
}

// v[j] += the partial sums of slices 1 .. slices-1 at row[z * zs + ec[j]], added in slice
// order.  Four slices per trip, every load of a trip issued before the first add (a slice
// past the last is read at the last one's address and not added).
template <int N>
MOE_DEV void add_slices(float (&v)[N], const float *row, const int (&ec)[N], int slices,
                        int64_t zs) {
  for (int z = 1; z < slices; z += 4) {
    float u[4][N];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float *pq = row + min(z + q, slices - 1) * zs;
#pragma unroll
      for (int j = 0; j < N; ++j) u[q][j] = pq[ec[j]];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool on = z + q < slices;
#pragma unroll
      for (int j = 0; j < N; ++j) v[j] = on ? v[j] + u[q][j] : v[j];
    }
  }
}

// this lane's share of the blend-head logits of token t: slice l of [slices][T][2] on lane
// l < slices, zero elsewhere (read at a valid address whatever the lane and whether or not
// the head exists, so the load is unconditional).
MOE_DEV float2 clog_part(const TopkArgs &a, int t, int l) {
  const float *base = a.clog ? a.clog : a.logits;
  const float2 v = *(const float2 *)(base + (int64_t)min(l, a.slices - 1) * 2 * a.T + 2 * t);
  return (a.clog && l < a.slices) ? v : make_float2(0.f, 0.f);
}

// token t on the calling wave (all 64 lanes).  sl: E floats of LDS, el: K ints of LDS,
// both private to the wave.  sidx: optional copy of the chosen ids ([T][K], LDS).
MOE_DEV void topk_token(const TopkArgs &a, int t, int lane, float *sl, int *el, int32_t *sidx) {
  constexpr int EPL = MOE_MAX_EXPERTS / 64;
  const float *lrow = a.logits + (int64_t)t * a.E;
  // every load issued before the first use (clamped ids; out-of-range slots masked below)
  float s[EPL], sb[EPL];
  int ec[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    ec[j] = min(lane + 64 * j, a.E - 1);
    s[j] = lrow[ec[j]];
    sb[j] = a.sbias ? a.sbias[ec[j]] : 0.f;
  }
  const float2 cp = clog_part(a, t, lane);
  add_slices<EPL>(s, lrow, ec, a.slices, (int64_t)a.T * a.E);
  if (a.logits_out) {
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j < a.E) a.logits_out[(int64_t)t * a.E + lane + 64 * j] = s[j];
  }
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (lane + 64 * j >= a.E) s[j] = -INFINITY;
  if (a.scoring == 1) {  // softmax over experts, max-subtracted, fp32
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < EPL; ++j) mx = fmaxf(mx, s[j]);
    mx = wave_max(mx);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      s[j] = (e < a.E) ? expf(s[j] - mx) : 0.f;
      sum += s[j];
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int j = 0; j < EPL; ++j) s[j] *= inv;
  } else {  // sigmoid
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      s[j] = (e < a.E) ? 1.0f / (1.0f + expf(-s[j])) : 0.f;
    }
  }
  uint64_t key[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    if (e < a.E) {
      sl[e] = s[j];
      const float sel = s[j] + sb[j];
      key[j] = ((uint64_t)ord_key(sel) << 32) | (uint32_t)~e;
    } else {
      key[j] = 0;
    }
  }
  int my_e = 0;
  for (int k = 0; k < a.K; ++k) {
    uint64_t loc = key[0];
#pragma unroll
    for (int j = 1; j < EPL; ++j) loc = umax64(loc, key[j]);
    const uint64_t best = wave_max_u64(loc);
    const int be = (int)~(uint32_t)best;
    if (lane == k) my_e = be;
    if ((be & 63) == lane) {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (j == (be >> 6)) key[j] = 0;
    }
  }
  if (lane < a.K) el[lane] = my_e;
  // the chosen ids in ascending order, their unbiased scores and the weight sum
  const float my_s = lane < a.K ? sl[my_e] : 0.f;
  const float wsum = wave_sum(my_s);
  if (lane < a.K) {
    int rank = 0;
    for (int i = 0; i < a.K; ++i) rank += (el[i] < my_e) ? 1 : 0;
    float w = a.norm ? my_s / wsum : my_s;
    w *= a.rscale;
    a.idx[(int64_t)t * a.K + rank] = my_e;
    a.w[(int64_t)t * a.K + rank] = w;
    if (sidx) sidx[t * a.K + rank] = my_e;
  }
  // blend coefficients: softmax over the 2-way head's logits, fp32
  if (a.clog) {
    const float c0 = wave_sum(cp.x), c1 = wave_sum(cp.y);
    if (lane == 0) {
      const float m = fmaxf(c0, c1);
      const float x0 = expf(c0 - m), x1 = expf(c1 - m);
      a.coef[2 * t] = x0 / (x0 + x1);
      a.coef[2 * t + 1] = x1 / (x0 + x1);
    }
  }
}

// ---- 32 lanes per token (two DPP rows), 2 tokens per wave.  Lane l32 of the half-wave
// holds experts l32 + 32*j, j < SL.  Reductions: DPP within each 16-lane row, then
// v_permlane16_swap, which hands every lane the value of the same lane in the other row
// of its half (the pair it returns holds both rows' values, in either order).

template <int CTRL>
MOE_DEV float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
MOE_DEV uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
MOE_DEV uint32_t half_max_u32(uint32_t v) {
  v = max(v, dppu<0xB1>(v));
  v = max(v, dppu<0x4E>(v));
  v = max(v, dppu<0x141>(v));
  v = max(v, dppu<0x140>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((uint32_t)r[0], (uint32_t)r[1]);
}
MOE_DEV uint32_t half_min_u32(uint32_t v) {
  v = min(v, dppu<0xB1>(v));
  v = min(v, dppu<0x4E>(v));
  v = min(v, dppu<0x141>(v));
  v = min(v, dppu<0x140>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return min((uint32_t)r[0], (uint32_t)r[1]);
}
MOE_DEV float half_max_f32(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// the two rows are added in the same order in every lane, so all 32 lanes agree bitwise
MOE_DEV float half_sum_f32(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  v += dppf<0x140>(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// token t on one half-wave (both halves of the wave call this together; a half with
// t >= T computes on a clamped token and stores nothing).  el / esc: 16 ints / floats of
// LDS private to the half (chosen ids and their unbiased scores, in selection order).
MOE_DEV float ld_dev(const float *p) {  // a device-scope (sc1) load
  return __uint_as_float(__hip_atomic_load((const uint32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
MOE_DEV void st_dev(float *p, float v) {  // a device-scope (sc1) store
  __hip_atomic_store((uint32_t *)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// the logits of token t (the router's slices summed in order) for this lane's experts
// l32 + 32 j of a half-wave, and the lane's share of the blend-head logits.  COH_IN: the
// logits (one slice) and the blend-head logits come from other workgroups of the same launch
// and are read at device scope.
template <int SL, bool COH_IN = false>
MOE_DEV void topk_half_load(const TopkArgs &a, int t, int l32, float (&lg)[SL], float2 &cp) {
  const bool live = t < a.T;
  const float *lrow = a.logits + (int64_t)(live ? t : a.T - 1) * a.E;
  int ec[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    ec[j] = min(l32 + 32 * j, a.E - 1);
    lg[j] = COH_IN ? ld_dev(lrow + ec[j]) : lrow[ec[j]];
  }
  if constexpr (COH_IN) {  // one slice: lane 0 holds the head's two logits
    const int tc = live ? t : a.T - 1;
    const bool on = a.clog && l32 == 0;
    cp = on ? make_float2(ld_dev(a.clog + 2 * tc), ld_dev(a.clog + 2 * tc + 1)) : make_float2(0.f, 0.f);
  } else {
    cp = clog_part(a, live ? t : a.T - 1, l32);
  }
  add_slices<SL>(lg, lrow, ec, a.slices, (int64_t)a.T * a.E);
}

// the selection bias of this lane's experts (0 without one)
template <int SL>
MOE_DEV void topk_half_sbias(const TopkArgs &a, int l32, float (&sb)[SL]) {
#pragma unroll
  for (int j = 0; j < SL; ++j) sb[j] = a.sbias ? a.sbias[min(l32 + 32 * j, a.E - 1)] : 0.f;
}

// scores, selection, weights and blend coefficients of token t from its loaded logits and
// this lane's selection biases.
// coherent: the ids, weights and blend coefficients are stored at device scope (written
// through to the point every XCD reads from), for a workgroup on another XCD to read without
// a cache write-back and invalidate.
template <int SL>
MOE_DEV void topk_half_select(const TopkArgs &a, int t, int l32, const float (&lg)[SL], float2 cp,
                              const float (&sb)[SL], int *el, float *esc, int32_t *sidx, bool coherent) {
  const bool live = t < a.T;
  if (a.logits_out && live) {
#pragma unroll
    for (int j = 0; j < SL; ++j)
      if (l32 + 32 * j < a.E) a.logits_out[(int64_t)t * a.E + l32 + 32 * j] = lg[j];
  }
  float sc[SL];
  if (a.scoring == 1) {  // softmax over experts, max-subtracted, fp32
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < SL; ++j)
      if (l32 + 32 * j < a.E) m = fmaxf(m, lg[j]);
    const float mx = half_max_f32(m);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      sc[j] = (l32 + 32 * j < a.E) ? expf(lg[j] - mx) : 0.f;
      sum += sc[j];
    }
    const float inv = 1.0f / half_sum_f32(sum);
#pragma unroll
    for (int j = 0; j < SL; ++j) sc[j] *= inv;
  } else {  // sigmoid
#pragma unroll
    for (int j = 0; j < SL; ++j) sc[j] = 1.0f / (1.0f + expf(-lg[j]));
  }
  // selection keys: the order-preserving u32 of score + bias (0, below every key, for absent
  // or retired experts).  Each round takes the half-wave maximum key, then the lowest expert
  // id holding it (each lane offers its lowest slot with its own maximum), and the owner
  // retires that slot.
  uint32_t key[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) key[j] = (l32 + 32 * j < a.E) ? ord_key(sc[j] + sb[j]) : 0u;
  uint32_t bv;
  int bj;
  auto local_best = [&]() {
    bv = key[0];
    bj = 0;
#pragma unroll
    for (int j = 1; j < SL; ++j)
      if (key[j] > bv) {
        bv = key[j];
        bj = j;
      }
  };
  local_best();
  for (int k = 0; k < a.K; ++k) {
    const uint32_t m = half_max_u32(bv);
    const int be = (int)half_min_u32(bv == m ? (uint32_t)(32 * bj + l32) : 0xFFFFFFFFu);
    if ((be & 31) == l32) {  // the owner retires the winner and records its score
      float ws = 0.f;
#pragma unroll
      for (int j = 0; j < SL; ++j)
        if (j == bj) {
          ws = sc[j];
          key[j] = 0u;
        }
      esc[k] = ws;
      el[k] = be;
      local_best();
    }
  }
  // the chosen ids in ascending order and the weight sum
  const int my_e = l32 < a.K ? el[l32] : 0x7fffffff;
  const float my_s = l32 < a.K ? esc[l32] : 0.f;
  const float wsum = half_sum_f32(my_s);
  if (live && l32 < a.K) {
    int rank = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int4 v = *(const int4 *)(el + 4 * q);
      rank += (4 * q + 0 < a.K && v.x < my_e) + (4 * q + 1 < a.K && v.y < my_e) +
              (4 * q + 2 < a.K && v.z < my_e) + (4 * q + 3 < a.K && v.w < my_e);
    }
    float w = a.norm ? my_s / wsum : my_s;
    w *= a.rscale;
    if (coherent) {
      __hip_atomic_store(a.idx + (int64_t)t * a.K + rank, my_e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      st_dev(a.w + (int64_t)t * a.K + rank, w);
    } else {
      a.idx[(int64_t)t * a.K + rank] = my_e;
      a.w[(int64_t)t * a.K + rank] = w;
    }
    if (sidx) sidx[t * a.K + rank] = my_e;
  }
  if (a.clog) {
    const float c0 = half_sum_f32(cp.x), c1 = half_sum_f32(cp.y);
    if (live && l32 == 0) {
      const float m = fmaxf(c0, c1);
      const float x0 = expf(c0 - m), x1 = expf(c1 - m);
      if (coherent) {
        st_dev(a.coef + 2 * t, x0 / (x0 + x1));
        st_dev(a.coef + 2 * t + 1, x1 / (x0 + x1));
      } else {
        a.coef[2 * t] = x0 / (x0 + x1);
        a.coef[2 * t + 1] = x1 / (x0 + x1);
      }
    }
  }
}

// token t on a half-wave (32 lanes, lane l32): topk_half_load then topk_half_select
template <int SL, bool COH_IN = false>
MOE_DEV void topk_half(const TopkArgs &a, int t, int l32, int *el, float *esc, int32_t *sidx, bool coherent = false) {
  float lg[SL], sb[SL];
  float2 cp;
  topk_half_load<SL, COH_IN>(a, t, l32, lg, cp);
  topk_half_sbias<SL>(a, l32, sb);
  topk_half_select<SL>(a, t, l32, lg, cp, sb, el, esc, sidx, coherent);
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// The permutation of a decode-sized batch (T <= MOE_ROUTE_SMALL_T) by one workgroup of NT
// threads, from the selections stored in idx [T][K] (read with device-scope loads: they may
// come from other workgroups of the same launch): per-expert slot counts and token masks,
// one scan over the experts of the packed (slot count, tile count) pairs (T*K <= 1024, so
// both fit 16 bits), then each slot's rank among the earlier tokens of its expert.  COH:
// sorted_slot, the tile list and its count are stored with device scope (read by other
// workgroups of the same launch).
// ---------------------------------------------------------------------------
template <int NT>
struct DecodePermSmem {
  int cnt[MOE_MAX_EXPERTS], offs[MOE_MAX_EXPERTS];
  uint32_t tmask[MOE_MAX_EXPERTS][MOE_ROUTE_SMALL_T / 32];
  int wtot[NT / 64];
};

// IDX_LDS: idx is the workgroup's own copy in LDS (else global memory, read at device scope).
// Returns the number of m-tiles (in every thread).
template <int NT, bool COH, bool IDX_LDS = false>
MOE_DEV int decode_permute(const int32_t *idx, int T, int K, int E, int32_t *__restrict__ counts,
                            int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
                            int32_t *__restrict__ slot_pos, int4 *tiles, int *tile_count, int mt,
                            DecodePermSmem<NT> &sm) {
  constexpr int NTW = MOE_ROUTE_SMALL_T / 32;  // token mask words per expert
  constexpr int EPT = (MOE_MAX_EXPERTS + NT - 1) / NT;  // experts per thread in the scan
  static_assert(NT % 64 == 0 && EPT * NT >= MOE_MAX_EXPERTS, "scan layout");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int TK = T * K;
  auto st = [](int32_t *p, int v) {
    if constexpr (COH)
      __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *p = v;
  };
  for (int e = tid; e < E; e += NT) {
    sm.cnt[e] = 0;
#pragma unroll
    for (int w = 0; w < NTW; ++w) sm.tmask[e][w] = 0u;
  }
  __syncthreads();
  // slot p = t*K + j: per-expert counts and per-expert token masks
  auto ld_id = [&](int p) {
    if constexpr (IDX_LDS)
      return idx[p];
    else
      return __hip_atomic_load(idx + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  constexpr int MAXP = (MOE_ROUTE_SMALL_T * 16 + NT - 1) / NT;  // slots per thread (K <= 16)
  int epv[MAXP];  // the thread's slots' experts, read once
#pragma unroll
  for (int q = 0; q < MAXP; ++q) {
    const int p = tid + q * NT;
    epv[q] = p < TK ? ld_id(p) : 0;
  }
#pragma unroll
  for (int q = 0; q < MAXP; ++q) {
    const int p = tid + q * NT;
    if (p < TK) {
      const int ep = epv[q], tp = p / K;
      atomicAdd(&sm.cnt[ep], 1);
      atomicOr(&sm.tmask[ep][tp >> 5], 1u << (tp & 31));
    }
  }
  __syncthreads();
  // exclusive scan over experts of (count | tiles << 16), experts EPT tid .. EPT tid + EPT-1
  int c[EPT], nt[EPT], pk[EPT];
  int local = 0;
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int e = EPT * tid + q;
    c[q] = e < E ? sm.cnt[e] : 0;
    nt[q] = (c[q] + mt - 1) / mt;
    pk[q] = c[q] | (nt[q] << 16);
    local += pk[q];
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sm.wtot[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int v = sm.wtot[w];
    base += (w < wave) ? v : 0;
    total += v;
  }
  int ex = base + incl - local;
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int e = EPT * tid + q;
    if (e < E) {
      const int off = ex & 0xFFFF, tb = ex >> 16;
      sm.offs[e] = off;
      counts[e] = c[q];
      offsets[e] = off;
      if (tiles)
        for (int i = 0; i < nt[q]; ++i) {
          int32_t *tp = (int32_t *)(tiles + tb + i);
          st(tp + 0, e);
          st(tp + 1, off + i * mt);
          st(tp + 2, min(mt, c[q] - i * mt));
          st(tp + 3, 0);
        }
    }
    ex += pk[q];
  }
  if (tid == 0) {
    offsets[E] = total & 0xFFFF;
    if (tiles) st(tile_count, total >> 16);
  }
  __syncthreads();
  // rank of slot p among the slots of its expert: earlier tokens that chose the same expert
#pragma unroll
  for (int q = 0; q < MAXP; ++q) {
    const int p = tid + q * NT;
    if (p >= TK) continue;
    const int ep = epv[q], tp = p / K;
    int rank = __popc(sm.tmask[ep][tp >> 5] & ((1u << (tp & 31)) - 1u));
    for (int w = 0; w < (tp >> 5); ++w) rank += __popc(sm.tmask[ep][w]);
    const int pos = sm.offs[ep] + rank;
    st(sorted_slot + pos, p);
    slot_pos[p] = pos;
  }
  return total >> 16;
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// One tile of the decode router: logits of tokens 16 tt .. 16 tt + 15 for rows 16 rt ..
// 16 rt + 15 of [W_r; coef head], bf16 x and W_r, MFMA 16x16x32 with the reduction split over
// the 8 waves of a 512-thread workgroup and summed in a fixed order.  Rows 0..E-1 are the
// experts (+ logit_bias); with a blend head, rows E and E+1 are its two rows (+ coef_b),
// written to clog [T][2].  Every wave issues the loads of up to DEPTH of its reduction steps
// before the first MFMA (the sum runs over the steps in the same order for every DEPTH).  red: 8*16*17 floats of LDS.  COH: the logits are stored at device
// scope (read by other workgroups of the same launch).
// ---------------------------------------------------------------------------
template <bool COH, int DEPTH = 8>
MOE_DEV void router_tile_bf16(const uint16_t *__restrict__ x, const uint16_t *__restrict__ W,
                              const float *__restrict__ lbias, float *__restrict__ logits, int T, int H, int E,
                              const uint16_t *__restrict__ cw, const float *__restrict__ cb,
                              float *__restrict__ clog, int tt, int rt, float (*red)[16][17]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = tt * 16, e0 = rt * 16;
  const int r = lane & 15, kb = lane >> 4;
  const int trow = min(t0 + r, T - 1), er = e0 + r;
  const uint16_t *wrow = er < E ? W + (int64_t)er * H
                                : ((cw && er < E + 2) ? cw + (int64_t)(er - E) * H : W + (int64_t)(E - 1) * H);
  const u32x4_t *xa = (const u32x4_t *)(x + (int64_t)trow * H + kb * 8);
  const u32x4_t *wb = (const u32x4_t *)(wrow + kb * 8);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = H >> 5;
  for (int s0 = wave; s0 < nsteps; s0 += 8 * DEPTH) {
    u32x4_t av[DEPTH], bv[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      const int st = min(s0 + 8 * i, nsteps - 1);
      av[i] = xa[st * 4];
      bv[i] = wb[st * 4];
    }
#pragma unroll
    for (int i = 0; i < DEPTH; ++i)
      if (s0 + 8 * i < nsteps)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[i]),
                                                      __builtin_bit_cast(bf16x8_t, bv[i]), acc, 0, 0, 0);
  }
  // acc[i] holds row (token) 4*kb+i, column r of the 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * kb + i][r] = acc[i];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, n = threadIdx.x & 15;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) v += red[w][m][n];
    const int t = t0 + m, e = e0 + n;
    if (t < T) {
      float *dst = nullptr;
      float val = 0.f;
      if (e < E) {
        dst = logits + (int64_t)t * E + e;
        val = v + (lbias ? lbias[e] : 0.f);
      } else if (cw && e < E + 2) {
        dst = clog + 2 * t + (e - E);
        val = v + cb[e - E];
      }
      if (dst) {
        if constexpr (COH)
          st_dev(dst, val);
        else
          *dst = val;
      }
    }
  }
}

}  // namespace
