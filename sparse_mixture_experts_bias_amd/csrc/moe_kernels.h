// moe_kernels.h - kernel argument structs and kernel declarations (device + host side).
#pragma once

#include "moe_device.h"

#define MOE_MAX_EXPERTS 512  // router top-k keeps 8 experts per lane of a wave64
#define MOE_MAX_TOPK 32      // chosen experts live one per lane (K <= 32)
#define MOE_MT_MIN 16        // smallest m-tile (rows of one segment per work unit) of the grouped GEMM
#define MOE_KC 256           // reduction elements per chunk for 4-bit weights (128 B per row)
#define MOE_GEMM_THREADS 256 // 4 waves
#define MOE_ROUTE_SMALL_T 64 // tokens (K <= 16) up to which selection and permutation share one launch

struct TopkArgs {
  const float *logits;  // [slices][T][E]: partial sums of the router's reduction slices, added in order
  int slices;
  float *logits_out;    // the summed logits [T][E], or nullptr
  int T, E, K, scoring, norm;
  float rscale;
  const float *sbias;
  int32_t *idx;
  float *w;
  const float *clog;    // blend head logits [slices][T][2], or nullptr
  float *coef;          // blend coefficients [T][2]
};

// ---- packed weight stream (written by moe_pack_weights, read by the grouped GEMM) ----
// Per matrix: row blocks of 32 tile rows (GATEUP: 16 gate rows then the 16 up rows of the
// same outputs; LINEAR: 32 consecutive rows, zero-padded), each a run of chunk records, one
// per PK_KC reduction elements (zero-padded past cols).  A record is 4096 bytes of weights
// in MFMA lane order, piece (i, lane) at i*1024 + lane*16 holding words 4i..4i+3 of the
// lane's 16-word sequence q = (unit*2 + half)*LPU + w (see pk_word_source), followed by the
// chunk's scales: AFFINE4 [half][lane%16][unit] words (scale | qbias << 16), MXFP4
// [half][lane%16][8] E8M0 bytes.  AFFINE4 weight words keep their 8 codes in pair order:
// element 2j at bits 4j..4j+3, element 2j+1 at bits 16+4j..19+4j.
// WF_MXS (MXFP4 for the block-scaled 16x16x128 FP4 x FP8 MFMA): the record's 256 elements are
// two stages of 128; piece i = 2*stage + half holds, at lane l, the 16 stored bytes (32 codes,
// low nibble first) of tile row 16*half + l%16 at elements 128*stage + 32*(l/16) .. +32 -- the
// MFMA's FP4 operand order -- and the 256 scale bytes are one word per lane, byte 2*stage + half
// the E8M0 scale of those 32 elements.
__host__ __device__ constexpr int pk_kc(int wf) { return wf == WF_DENSE ? 64 : 256; }
__host__ __device__ constexpr int pk_ue(int wf, int gq) {
  return wf == WF_AFFINE4 ? gq : (wf == WF_MXFP4 ? 64 : (wf == WF_MXS ? 128 : 32));
}
__host__ __device__ constexpr int pk_lb(int wf, int gq) {  // weight bytes per lane, unit and half
  return wf == WF_DENSE ? 2 * (pk_ue(wf, gq) / 4) : pk_ue(wf, gq) / 8;
}
__host__ __device__ constexpr int pk_nu(int wf, int gq) { return pk_kc(wf) / pk_ue(wf, gq); }
__host__ __device__ constexpr int pk_scale_bytes(int wf, int gq) {
  return wf == WF_AFFINE4 ? 32 * pk_nu(wf, gq) * 4 : (wf == WF_MXFP4 || wf == WF_MXS ? 32 * 8 : 0);
}
__host__ __device__ constexpr int pk_record_bytes(int wf, int gq) { return 4096 + pk_scale_bytes(wf, gq); }

// one stacked weight operand [n][rows][cols] (see moe_linear)
struct WMat {
  const void *w;        // natural layout (f32 path)
  const void *scales;
  const void *qbias;
  const void *bias;     // output bias [n][rows], bf16 (or nullptr)
  int64_t w_stride;     // bytes between matrices
  int64_t s_stride;     // elements between matrices of scales/qbias
  int64_t ldw;          // bytes per row of w
  int lds;              // elements per row of scales/qbias
  int rows, cols;
  const char *pk;       // packed stream (GATEUP: gate and up together, in w0)
  int64_t pk_mat;       // bytes per matrix of the packed stream
  int pk_nblk;          // row blocks per matrix
  int pk_nch;           // chunk records per row block
};

// activation rows feeding a segment set: sorted row r reads A row
// gather ? gather[r] / gdiv : r - row_sub
struct AOp {
  const void *a;
  int64_t lda;          // elements
  const int32_t *gather;
  int gdiv;
  int row_sub;
  int64_t rows;         // rows of a (bounds of the byte offsets the tall kernel uses)
  const uint16_t *as;   // WF_MXS: the split activations' scale pairs [rows][ldas] (see split_fp8)
  int64_t ldas;
};

struct SegSet {
  AOp A;
  WMat w0, w1;          // GATEUP: gate, up;  LINEAR: w0 only
  float limit;          // GATEUP clamp (<= 0: none)
  int K;                // reduction length
  int nblk;             // column blocks of the output
};

struct GemmParams {
  SegSet seg[2];        // [0] routed experts (m-tiles from the tile list), [1] shared expert / plain rows
  const int4 *tiles;    // routed m-tiles (expert, first sorted row, rows), or nullptr
  const int *tile_count;// [0]: routed m-tiles in the list
  int max_tiles;        // entries allocated in tiles (loads are clamped into them)
  int sh_row0, sh_rows; // segment 1: first row (in the sorted-row numbering of out) and row count
  int sh_mt;            // segment 1's m-tile rows in the prefill kernel (0: its full 128; 64 for
                        // plain GEMMs with too few 128-row units to fill the CUs)
  int E;
  void *out;
  int64_t ldo;
  const float *resid;   // LINEAR: optional f32 [rows][ldr] added before the store
  int64_t ldr;
};

#define MOE_CNT_STRIDE 32  // ints between the counters of the one-launch decode path (128 bytes)
constexpr int kCntStride = MOE_CNT_STRIDE;
// the counter block of the one-launch decode path (ints, cleared by the router launch):
// Counter block of the decode launches (kCounterInts ints, every counter at the start of its
// own 128-byte line; zero when the routing launch starts, and left so): [kTileDone] router
// tiles done (one token block), [kSelCnt] tokens selected and [kTtCnt0 + kCntStride tt] router
// tiles of token block tt done (several blocks), all cleared by the routing launch once
// used, then the experts launch's m-tile counters (gate/up waves done) from kTileCnt0
// (cleared by the routing launch before it).
// The single-launch path (up to 16 tokens) uses two more blocks of the same layout, one per call
// in turn (each call clears the other for the next): [kTileDone] router tiles done, the m-tile
// counters from kTileCnt0, from kColCnt0 the down waves done per 32-column block of the
// output, and from kFlag0 the routing flag (1 once the routing is stored).
constexpr int kTileDone = 0, kSelCnt = kCntStride, kTtCnt0 = 2 * kCntStride;
constexpr int kTileCnt0 = kTtCnt0 + (MOE_ROUTE_SMALL_T / 16) * kCntStride;
constexpr int kMaxTileCnt = 584;  // shared + routed m-tiles
constexpr int kColCnt0 = kTileCnt0 + kMaxTileCnt * kCntStride;
constexpr int kMaxColCnt = 256;   // 32-column blocks of the output (hidden <= 8192)
// the routing flag in kFlagCopies lines (workgroup g polls copy g mod kFlagCopies)
constexpr int kFlag0 = kColCnt0 + kMaxColCnt * kCntStride, kFlagCopies = 32;
constexpr int kCounterInts = kFlag0 + kFlagCopies * kCntStride;

struct FusedParams {
  // router: logits [T][E] = x W_r^T (+ logit_bias), blend head logits clog [T][2]
  const uint16_t *x, *Wr, *cw;  // x [T][H] bf16, W_r [E][H] bf16, blend head [2][H] bf16 or nullptr
  const float *lbias, *cb;      // logit_bias [E] or nullptr, blend head bias [2]
  int H;
  TopkArgs ta;                // selection of every token (ta.logits: the router's output, one slice)
  int32_t *counts, *offsets, *slot_pos;  // permutation outputs (sorted_slot: gu.seg[0].A.gather)
  GemmParams gu;              // gate/up: seg[0] routed, seg[1] shared; out = h (bf16), ldo = its row stride
  GemmParams dn;              // down: seg[0] routed, seg[1] shared; out = o in token order (rows t*K + j,
                              // then T*K + t for the shared expert), ldo = Dout
  int Dout;
  int *cnt;                   // the counter block
  int n_tile_cnt;             // m-tile counters the experts launch uses
  int *status;                // 1 when a bounded wait gave up
  // the single launch (up to 16 tokens) only:
  int *cnt_next;              // the counter block of the next call, cleared by this one
  int nr_ub;                  // routed m-tiles at most
  void *y;                    // the block's output [T][ldy], ydt (DT_F32 or DT_BF16)
  int ldy, ydt;
  int mode;                   // 0 routed sum, 2 + shared, 3 blend with the shared expert
};

struct F32GemmParams {   // f32 activations with DENSE F32 weights (one thread per output)
  const float *a_routed; int64_t lda_r;   // rows gathered through sorted_slot / K
  const float *a_shared; int64_t lda_s;   // rows r - TK
  const int32_t *sorted_slot;
  const int32_t *topk_idx;
  int K, TK, Tsh;
  WMat r0, r1, s0, s1;
  float limit;
  float *out; int64_t ldo;
  int ncols_r, ncols_s;
  int gateup;
};

struct CombineArgs {
  const void *o; int64_t ldo;        // per-slot expert outputs (sorted rows, or token order), ODT
  const int32_t *slot_pos;           // row of slot t*K + j in o; nullptr: o is in token order
  const float *topk_w;
  int K, TK, T, D;
  void *y; int64_t ldy;              // YDT
  const float *coef;                 // blend coefficients [T][2]
  const float *norm_w; float eps;    // rms norm
  int mode;                          // 0 routed sum, 1 rms-norm, 2 + shared, 3 blend with shared
};

// ---- kernels ----
// router kernels: zero[0 .. zero_n) (optional) is cleared by the launch (the status word, the
// counter of route_decode and the counters of the one-launch decode experts)
__global__ void router_logits_bf16(const uint16_t *x, const uint16_t *W, const float *lbias, float *logits,
                                   int T, int H, int E, const uint16_t *cw, const float *cb, float *clog, int *zero,
                                   int zero_n);
__global__ void router_gemm_bf16(const uint16_t *x, const uint16_t *W, const float *lbias, float *logits, int T,
                                 int H, int E, const uint16_t *cw, const float *cb, float *clog, int *zero, int zero_n,
                                 int ks);
#define MOE_ROUTER_GEMM_T 256  // tokens from which the router runs as a tiled GEMM
__global__ void router_logits_f32(const float *x, const float *W, const float *lbias, float *logits, int T,
                                  int H, int E, const float *cw, const float *cb, float *clog, int *zero, int zero_n);
__global__ void topk_kernel(TopkArgs a);
template <int SL> __global__ void topk_half_kernel(TopkArgs a);
template <int SL>
__global__ void route_decode(TopkArgs a, int32_t *counts, int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos,
                             int4 *tiles, int *tile_count, int mt, int *done);
__global__ void perm_count(const int32_t *idx, int T, int K, int E, int32_t *chunk_counts);
__global__ void perm_scan(int32_t *chunk_counts, int nchunks, int E, int TK, int32_t *counts, int32_t *offsets,
                          int4 *tiles, int *tile_count, int mt);
__global__ void perm_scatter(const int32_t *idx, int T, int K, int E, const int32_t *chunk_base,
                             int32_t *sorted_slot, int32_t *slot_pos);
__global__ void perm_small(const int32_t *idx, int T, int K, int E, int32_t *counts, int32_t *offsets,
                           int32_t *sorted_slot, int32_t *slot_pos, int4 *tiles, int *tile_count, int mt);
__global__ void build_tiles(const int32_t *offsets, int E, int4 *tiles, int *tile_count, int mt);
constexpr int kPermFusedChunks = 256;  // chunks of 256 tokens of the single-launch permutation
__global__ void perm_fused(const int32_t *idx, int T, int K, int E, int32_t *chunk_counts, int32_t *counts,
                           int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos, int4 *tiles, int *tile_count,
                           int mt, int *done, int *status);

// host-side launchers (moe_gemm.hip, moe_combine.hip)
hipError_t launch_expert_gemm(int adt, int wfmt, int group, bool gateup, int odt, int mb, const GemmParams &p,
                              int grid, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
// decode-sized segments with 4-bit weights: loader waves stream the records through LDS
// (moe_gemm_ws.hip); same units as launch_expert_gemm with mb == 1
hipError_t launch_expert_gemm_ws(int adt, int wfmt, int group, bool gateup, int odt, const GemmParams &p, int grid,
                                 hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
int ws_wgs_per_cu(int wfmt, int group);  // resident workgroups per CU (LDS)
// prefill-sized segments: 128-row m-tiles, 8-wave workgroups (moe_gemm_tall.hip)
hipError_t launch_expert_gemm_tall(int adt, int wfmt, int group, bool gateup, int odt, const GemmParams &p,
                                   int grid, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
hipError_t launch_f32_gemm(const F32GemmParams &p, int rows, hipStream_t s);
// units_ub: an upper bound of the launch's units (grid = min(units_ub, resident capacity));
// idt: storage type of h and o (the activations' type)
// the routing launch of a decode batch (bf16 x and router, E <= 256): router logits, selection,
// permutation and m-tile list; clears the experts launch's counters
hipError_t launch_decode_route(const FusedParams &p, hipStream_t s);
// the experts launch: grid min(units_ub, what the device holds at once)
hipError_t launch_decode_one(int wfmt, int group, int idt, const FusedParams &p, int units_ub, hipStream_t s,
                             hipEvent_t e0, hipEvent_t e1);
hipError_t launch_decode_fused(int wfmt, int group, int idt, const FusedParams &p, int units_ub, hipStream_t s,
                               hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
// packed stream of one matrix stack (b: the up stack of a gate/up pair, or nullptr)
struct PackArgs {
  int wf, gq, n, rows, cols, gateup, dense_f32;
  const void *a_w, *a_s, *a_q;   // gate (or the only) stack, natural layout
  const void *b_w, *b_s, *b_q;   // up stack (gateup) or nullptr
  uint32_t *out;
  int nblk, nch;
};
hipError_t launch_pack(const PackArgs &a, hipStream_t s);
hipError_t launch_bf16_to_f16(const void *in, void *out, int64_t n, hipStream_t s);
hipError_t launch_split_fp8(const void *in, int64_t ldi, int rows, int cols, void *hl, uint16_t *hs, hipStream_t s);
hipError_t launch_combine(int odt, int ydt, const CombineArgs &a, hipStream_t s);
