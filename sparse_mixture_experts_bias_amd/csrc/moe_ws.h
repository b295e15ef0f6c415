// moe_ws.h - stage layout of the loader-wave decode GEMMs (moe_gemm_ws.hip, moe_decode.hip).
#pragma once

#include "moe_mfma.h"

namespace {

template <int WF, int GQ>
struct WsCfg {
  static constexpr bool AFF = WF == WF_AFFINE4, MX = WF == WF_MXFP4;
  static_assert(AFF || MX, "4-bit formats");
  static constexpr int KC = pk_kc(WF);                     // reduction elements per record
  static constexpr int UE = pk_ue(WF, GQ);                 // elements per unit (group)
  static constexpr int SPU = UE / 32;                      // MFMA steps per unit
  static constexpr int QE = UE / 4;                        // elements per lane quarter per unit
  static constexpr int LPU = pk_lb(WF, GQ) / 4;            // weight words per lane, unit and half
  static constexpr int NU = pk_nu(WF, GQ);                 // units per record
  static constexpr int RB = pk_record_bytes(WF, GQ);       // bytes per record
  static constexpr int SB = RB - 4096;                     // scale bytes per record
  static constexpr int NSD = SB == 1024 ? 1 : SB / 256;    // scale loads: one 16-byte-lane or 4-byte-lane ones
  static_assert(NSD == 1 || NSD == 2, "one or two scale loads");
  static constexpr int SW = 4 * RB;                        // weight bytes of a stage (4 row blocks)
  static constexpr int SA = 16 * KC * 2;                   // activation bytes of a stage (16 rows)
  static constexpr int STAGE = SW + SA;
  static constexpr int NBUF = 2;                           // stage buffers (one stage in flight)
  static constexpr int WGS_PER_CU = (160 * 1024) / (NBUF * STAGE) < 3 ? 2 : 3;
  static constexpr int NDMA = 4 + NSD + 2;                 // direct loads per stage and loader wave
  static_assert(2 * NU * LPU == 16, "64 weight bytes per lane per record");
  static_assert(SB == 1024 || SB % 256 == 0, "scale block layout");
};

// direct load of SIZE bytes per lane: lane i writes LDS at lds + OFF + SIZE * i, reading
// rsrc at voff + soff + OFF (SIZE and OFF literal constants)
#define WS_DMA(SIZE, OFF, rsrc, lds, voff, soff) \
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(lds), SIZE, voff, soff, OFF, 0)

}  // namespace
