// moe_mfma.h - operand helpers of the grouped GEMMs: the 16x16x32 MFMA, 4-bit and FP4
// weight conversion to the MFMA's 16-bit types, and explicit vector-memory waits.
#pragma once

#include "moe_kernels.h"

namespace {

// 16x16x32 MFMA: lane l holds A[m = l%16][k = 8*(l/16) .. +8), B[k = 8*(l/16) .. +8][n = l%16]
// and D[m = 4*(l/16) + i][n = l%16], i = 0..3.
template <int AT>
MOE_DEV f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (AT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// Unit schedule of the grouped GEMMs: workgroup g takes at most one unit per round of G
// units (round r: units r*G .. r*G + G - 1; only the last round may be partial) and -1 when
// it has none.  Workgroups reach the 8 XCDs round-robin (XCD g % 8), and a round's units are
// cut into 8 equal runs of consecutive units, one per XCD: the column blocks of one m-tile
// (consecutive units, which read the same activation rows) share that XCD's L2, and a partial
// round still spreads over every XCD (each XCD's path to memory carries only its share of
// the bandwidth).
MOE_DEV int sched_unit(int g, int r, int G, int U) {
  const int base = r * G, n = min(G, U - base);
  if (n <= 0) return -1;
  if (G % 8) return g < n ? base + g : -1;
  const int per = (n + 7) >> 3, slot = g >> 3, pos = (g & 7) * per + slot;
  return (slot < per && pos < n) ? base + pos : -1;
}

// a constant the compiler must keep in a VGPR (so that mask-and-or with two constants is one v_and_or_b32)
MOE_DEV uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// 8 nibbles in pair order (nibble position i in bits 4i..4i+3) -> 4 words holding the
// 16-bit values (mag + nibble i, mag + nibble i+4), i = 0..3: elements (2i, 2i+1)
MOE_DEV u32x4_t magic_pairs(uint32_t w, uint32_t msk, uint32_t mag) {
  u32x4_t r;
  r[0] = (w & msk) | mag;
  r[1] = ((w >> 4) & msk) | mag;
  r[2] = ((w >> 8) & msk) | mag;
  r[3] = ((w >> 12) & msk) | mag;
  return r;
}

MOE_DEV float f16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
MOE_DEV float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// 8 nibbles in pair order -> 4 words of dequantised element pairs (2j, 2j+1) in the MFMA
// type.  The nibbles at bits 0-3 (of either half-word) become the exact f16 value 1024 + q
// under the magic 0x6400, those at bits 4-7 the exact 64 + q under 0x5400 (the mantissa's
// bit 4 weighs 1 at that exponent), so one shift by 8 serves the other two positions.  Each
// weight is then one fp32 FMA, sc * (1024 + q) + c0 or sc * (64 + q) + c1 with
// c0 = qbias - 1024 sc, c1 = qbias - 64 sc (both exact), i.e. sc*q + qbias rounded once to
// fp32, then rounded to 16 bits.
template <int AT>
MOE_DEV u32x4_t deq_affine(uint32_t w, uint32_t m0, uint32_t m1, uint32_t g0, uint32_t g1, float sc, float c0,
                           float c1) {
  const uint32_t w8 = w >> 8;
  const uint32_t m[4] = {(w & m0) | g0, (w & m1) | g1, (w8 & m0) | g0, (w8 & m1) | g1};
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float c = (j & 1) ? c1 : c0;
    const float lo = fmaf(f16lo(m[j]), sc, c), hi = fmaf(f16hi(m[j]), sc, c);
    if constexpr (AT == DT_BF16) {
      const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
      r[j] = __builtin_bit_cast(uint32_t, v);
    } else {
      const f16x2_t v = {(_Float16)lo, (_Float16)hi};  // one v_cvt_pk_f16_f32
      r[j] = __builtin_bit_cast(uint32_t, v);
    }
  }
  return r;
}

// The f16 form of deq_affine in packed half-precision arithmetic: the magic words hold the
// exact pairs (1024 + q, 1024 + q') or (64 + q, 64 + q'); one packed add takes the magic off
// (exact: q and the result are small integers) and one packed FMA gives sc*q + qbias rounded
// once to f16 -- the same single rounding as the fp32 form, with half the instructions.
// s2 = (sc, sc) and qb2 = (qbias, qbias) in f16: bf16 values convert to f16 exactly inside
// f16's normal range (a bf16 mantissa fits in f16's).
MOE_DEV u32x4_t deq_affine_h16(uint32_t w, uint32_t m0, uint32_t m1, uint32_t g0, uint32_t g1, f16x2_t s2,
                               f16x2_t qb2) {
  const uint32_t w8 = w >> 8;
  const uint32_t m[4] = {(w & m0) | g0, (w & m1) | g1, (w8 & m0) | g0, (w8 & m1) | g1};
  const f16x2_t o0 = {(_Float16)-1024.0f, (_Float16)-1024.0f}, o1 = {(_Float16)-64.0f, (_Float16)-64.0f};
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f16x2_t q = __builtin_bit_cast(f16x2_t, m[j]) + ((j & 1) ? o1 : o0);
    r[j] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, qb2));
  }
  return r;
}

// (v, v) in f16
MOE_DEV f16x2_t h16_pair(float v) {
  const f16x2_t r = {(_Float16)v, (_Float16)v};  // one v_cvt_pk_f16_f32
  return r;
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

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0 and 15:14;
// expcnt and lgkmcnt left at their maxima)
template <int N>
MOE_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// vector-memory instructions of one chunk's loads: 4 weight pieces, the scale words, SIT
// activation blocks
template <int WF, int GQ, int SIT>
constexpr int LOADS_PER_CHUNK() {
  return 4 + (WF == WF_AFFINE4 ? (pk_nu(WF, GQ) == 8 ? 4 : 2) : (WF == WF_MXFP4 ? 2 : 0)) + SIT;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// workgroup barrier without the compiler's release fence (which would drain every
// outstanding load, prefetched ones included); callers wait for their own global loads
// first.  LDS accesses are drained here (lgkmcnt 0, vmcnt and expcnt untouched), so LDS
// written before the barrier is visible after it and no wave's direct loads can overwrite
// LDS that another wave is still reading.
MOE_DEV void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// uniform values through the scalar data cache, so that reading them does not wait on the
// vector loads in flight; each load is waited for in its own asm block
MOE_DEV int4 load_uniform_int4(const int4 *ptr) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  i32x4 v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr));
  return make_int4(v[0], v[1], v[2], v[3]);
}
MOE_DEV int load_uniform_int(const int *ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr));
  return v;
}
// a uniform int and a uniform int4 read together (one wait)
MOE_DEV void load_uniform_int_int4(const int *a, const int4 *b, int &x, int4 &y) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  i32x4 v;
  int s;
  asm volatile("s_load_dword %0, %2, 0x0\n\ts_load_dwordx4 %1, %3, 0x0\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(s), "=&s"(v)
               : "s"(a), "s"(b));
  x = s;
  y = make_int4(v[0], v[1], v[2], v[3]);
}
// four uniform ints read together (one wait)
MOE_DEV void load_uniform_ints4(const int *a, const int *b, const int *c, const int *d, int (&v)[4]) {
  asm volatile(
      "s_load_dword %0, %4, 0x0\n\ts_load_dword %1, %5, 0x0\n\ts_load_dword %2, %6, 0x0\n\t"
      "s_load_dword %3, %7, 0x0\n\ts_waitcnt lgkmcnt(0)"
      : "=&s"(v[0]), "=&s"(v[1]), "=&s"(v[2]), "=&s"(v[3])
      : "s"(a), "s"(b), "s"(c), "s"(d));
}

// the scale operand of the scaled FP4 conversions for an E8M0 byte: the byte in the f32
// exponent field.  The conversion reads that field as the E8M0 value itself (0 -> 2^-127,
// 255 -> NaN): measured on gfx950 for every exponent 0..255 and every code at every nibble
// position, identical to passing the decoded 2^(e-127) (with 2^-127 and NaN at the ends), in
// both f16 and bf16.
MOE_DEV float e8m0_scale(uint32_t e) { return __uint_as_float(e << 23); }

template <int AT>
MOE_DEV u32x4_t cvt_dense(u32x4_t w) {
  if constexpr (AT == DT_BF16) {
    return w;
  } else {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2_t v = {(_Float16)__uint_as_float(w[i] << 16), (_Float16)__uint_as_float(w[i] & 0xFFFF0000u)};
      r[i] = __builtin_bit_cast(uint32_t, v);
    }
    return r;
  }
}

}  // namespace
