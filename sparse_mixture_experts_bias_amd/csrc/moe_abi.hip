// moe_abi.hip - the C ABI of include/moe.h: argument validation, workspace
// layout and launch sequencing.  No entry point allocates device memory; every
// argument is checked before the first launch and errors come back as status
// codes (the load-time validation of mlxcel PR #1044 "Other guards" and of
// mlxcel issue #974 "Acceptance Criteria": zero checks before divisibility
// checks, top-k in 1..num_experts, full expert stacks, quantisation parameters
// bounded before use, nothing that can abort the process later).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "moe_kernels.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

#define CHECK(cond, st, ...) \
  do {                       \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)
#define TRY(expr)                      \
  do {                                 \
    moe_status _s = (expr);            \
    if (_s != MOE_OK) return _s;       \
  } while (0)
#define HIPCHK(expr)                                                                  \
  do {                                                                                \
    hipError_t _e = (expr);                                                           \
    if (_e != hipSuccess) return fail(MOE_ERR_DEVICE, "%s: %s", #expr, hipGetErrorString(_e)); \
  } while (0)

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int dt_size(int dt) { return dt == MOE_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// validation
// ---------------------------------------------------------------------------

// how a descriptor is used: as the source of moe_pack_weights, or by a forward pass (the
// BF16/F16 GEMM reads the packed stream; the up stack of a gate/up pair has none of its own)
enum { USE_SOURCE = 0, USE_GEMM = 1, USE_GEMM_PAIRED = 2 };

// act_dt: dtype of the activations this linear is applied to
moe_status check_linear(const moe_linear *L, const char *name, int n, int rows, int cols, int act_dt, int use) {
  CHECK(L != nullptr, MOE_ERR_ARG, "%s: descriptor is NULL", name);
  CHECK(L->n > 0 && L->rows > 0 && L->cols > 0, MOE_ERR_SHAPE, "%s: zero or negative dimension (n=%d rows=%d cols=%d)",
        name, L->n, L->rows, L->cols);
  CHECK(L->n == n, MOE_ERR_SHAPE, "%s: stack holds %d matrices, expected %d", name, L->n, n);
  CHECK(L->rows == rows && L->cols == cols, MOE_ERR_SHAPE, "%s: shape [%d, %d], expected [%d, %d]", name, L->rows,
        L->cols, rows, cols);
  const bool natural = use == USE_SOURCE || act_dt == MOE_F32;  // the natural-layout pointers are read
  if (natural) {
    CHECK(L->w != nullptr, MOE_ERR_ARG, "%s: weight pointer is NULL", name);
    CHECK(aligned(L->w, 16), MOE_ERR_ARG, "%s: weight pointer not 16-byte aligned", name);
  } else if (use == USE_GEMM) {
    CHECK(L->packed != nullptr, MOE_ERR_ARG, "%s: packed stream is NULL (write it with moe_pack_weights)", name);
    CHECK(aligned(L->packed, 256), MOE_ERR_ARG, "%s: packed stream not 256-byte aligned", name);
  }
  CHECK(L->bias == nullptr || aligned(L->bias, 4), MOE_ERR_ARG, "%s: bias pointer misaligned", name);
  CHECK(L->packed_scaled == nullptr || L->fmt == MOE_W_MXFP4, MOE_ERR_ARG,
        "%s: packed_scaled is for MXFP4 weights only", name);
  CHECK(L->packed_scaled == nullptr || aligned(L->packed_scaled, 256), MOE_ERR_ARG,
        "%s: packed_scaled stream not 256-byte aligned", name);
  switch (L->fmt) {
    case MOE_W_DENSE:
      CHECK(L->dense_dtype == MOE_F32 || L->dense_dtype == MOE_BF16, MOE_ERR_ARG, "%s: dense dtype %d not F32/BF16",
            name, L->dense_dtype);
      if (L->dense_dtype == MOE_F32) {
        CHECK(act_dt == MOE_F32, MOE_ERR_UNSUPPORTED, "%s: F32 weights need F32 activations", name);
      } else {
        CHECK(act_dt != MOE_F32, MOE_ERR_UNSUPPORTED, "%s: BF16 weights need BF16/F16 activations", name);
      }
      break;
    case MOE_W_AFFINE4:
      CHECK(L->bits == 4, MOE_ERR_QUANT, "%s: affine bits %d (only 4 is supported)", name, L->bits);
      CHECK(L->group_size == 32 || L->group_size == 64 || L->group_size == 128, MOE_ERR_QUANT,
            "%s: affine group_size %d (32, 64 or 128)", name, L->group_size);
      CHECK(cols % L->group_size == 0, MOE_ERR_SHAPE, "%s: cols %d not a multiple of group_size %d", name, cols,
            L->group_size);
      if (natural) {
        CHECK(L->scales != nullptr && L->qbias != nullptr, MOE_ERR_ARG, "%s: affine scales/qbias missing", name);
        CHECK(aligned(L->scales, 2) && aligned(L->qbias, 2), MOE_ERR_ARG, "%s: scales/qbias misaligned", name);
      }
      CHECK(act_dt != MOE_F32, MOE_ERR_UNSUPPORTED, "%s: quantized weights need BF16/F16 activations", name);
      break;
    case MOE_W_MXFP4:
      CHECK(L->bits == 4, MOE_ERR_QUANT, "%s: mxfp4 bits %d (must be 4)", name, L->bits);
      CHECK(L->group_size == 32, MOE_ERR_QUANT, "%s: mxfp4 group_size %d (must be 32)", name, L->group_size);
      CHECK(cols % 64 == 0, MOE_ERR_SHAPE, "%s: mxfp4 cols %d not a multiple of 64", name, cols);
      if (natural) CHECK(L->scales != nullptr, MOE_ERR_ARG, "%s: mxfp4 scales missing", name);
      CHECK(act_dt != MOE_F32, MOE_ERR_UNSUPPORTED, "%s: quantized weights need BF16/F16 activations", name);
      break;
    default:
      return fail(MOE_ERR_ARG, "%s: weight format %d out of range", name, L->fmt);
  }
  if (act_dt != MOE_F32) {
    CHECK(rows % 16 == 0, MOE_ERR_SHAPE, "%s: rows %d not a multiple of 16", name, rows);
    CHECK(cols % 32 == 0, MOE_ERR_SHAPE, "%s: cols %d not a multiple of 32", name, cols);
  }
  return MOE_OK;
}

moe_status check_mlp(const moe_mlp *m, const char *name, int n, int I, int D, int act_in, int act_mid) {
  char nm[64];
  snprintf(nm, sizeof nm, "%s.gate", name);
  TRY(check_linear(&m->gate, nm, n, I, D, act_in, USE_GEMM));
  snprintf(nm, sizeof nm, "%s.up", name);
  TRY(check_linear(&m->up, nm, n, I, D, act_in, USE_GEMM_PAIRED));
  CHECK(m->up.fmt == m->gate.fmt && m->up.group_size == m->gate.group_size && m->up.dense_dtype == m->gate.dense_dtype,
        MOE_ERR_UNSUPPORTED, "%s: gate and up stacks must share one format", name);
  snprintf(nm, sizeof nm, "%s.down", name);
  TRY(check_linear(&m->down, nm, n, D, I, act_mid, USE_GEMM));
  CHECK(std::isfinite(m->swiglu_limit), MOE_ERR_ARG, "%s: swiglu_limit not finite", name);
  return MOE_OK;
}

moe_status check_router(const moe_router *r, int H, int x_dt) {
  CHECK(r != nullptr, MOE_ERR_ARG, "router descriptor is NULL");
  CHECK(r->num_experts > 0, MOE_ERR_SHAPE, "num_experts %d must be positive", r->num_experts);
  CHECK(r->num_experts <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "num_experts %d above %d", r->num_experts,
        MOE_MAX_EXPERTS);
  CHECK(r->top_k >= 1 && r->top_k <= r->num_experts, MOE_ERR_SHAPE, "top_k %d outside 1..num_experts (%d)", r->top_k,
        r->num_experts);
  CHECK(r->top_k <= MOE_MAX_TOPK, MOE_ERR_SHAPE, "top_k %d above %d", r->top_k, MOE_MAX_TOPK);
  CHECK(r->scoring == MOE_SIGMOID || r->scoring == MOE_SOFTMAX, MOE_ERR_ARG, "scoring %d out of range", r->scoring);
  CHECK(r->norm_topk == 0 || r->norm_topk == 1, MOE_ERR_ARG, "norm_topk %d must be 0 or 1", r->norm_topk);
  CHECK(std::isfinite(r->routed_scale), MOE_ERR_ARG, "routed_scale not finite");
  CHECK(r->w != nullptr, MOE_ERR_ARG, "router weight is NULL");
  CHECK(aligned(r->w, 16), MOE_ERR_ARG, "router weight not 16-byte aligned");
  CHECK(x_dt == MOE_F32 || H % 32 == 0, MOE_ERR_SHAPE, "hidden %d not a multiple of 32", H);
  return MOE_OK;
}

moe_status check_tokens(int64_t T, int K) {
  CHECK(T >= 0, MOE_ERR_SHAPE, "token count %lld negative", (long long)T);
  CHECK(T <= (int64_t)(INT32_MAX / 2) / (K > 0 ? K : 1), MOE_ERR_SHAPE, "T*K overflows (T=%lld, K=%d)", (long long)T,
        K);
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
struct Plan {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  }
};

moe_status check_ws(void *ws, size_t *ws_bytes, size_t need, bool *query) {
  CHECK(ws_bytes != nullptr, MOE_ERR_ARG, "ws_bytes is NULL");
  if (ws == nullptr) {
    *ws_bytes = need;
    *query = true;
    return MOE_OK;
  }
  *query = false;
  CHECK(*ws_bytes >= need, MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", *ws_bytes, need);
  CHECK(need == 0 || aligned(ws, 256), MOE_ERR_WORKSPACE, "workspace not 256-byte aligned");
  return MOE_OK;
}

template <typename T>
T *at(void *ws, size_t off) {
  return (T *)((char *)ws + off);
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

WMat wmat(const moe_linear &L, bool gateup = false) {
  WMat m;
  const int wf = L.fmt == MOE_W_DENSE ? WF_DENSE : (L.fmt == MOE_W_AFFINE4 ? WF_AFFINE4 : WF_MXFP4);
  m.pk = (const char *)L.packed;
  m.pk_nblk = gateup ? (L.rows + 15) / 16 : (L.rows + 31) / 32;
  m.pk_nch = (L.cols + pk_kc(wf) - 1) / pk_kc(wf);
  m.pk_mat = (int64_t)m.pk_nblk * m.pk_nch * pk_record_bytes(wf, L.group_size);
  m.w = L.w;
  m.scales = L.scales;
  m.qbias = L.qbias;
  m.bias = L.bias;
  m.rows = L.rows;
  m.cols = L.cols;
  int64_t ldw;
  if (L.fmt == MOE_W_DENSE)
    ldw = (int64_t)L.cols * (L.dense_dtype == MOE_F32 ? 4 : 2);
  else
    ldw = L.cols / 2;
  m.ldw = ldw;
  m.w_stride = ldw * L.rows;
  m.lds = (L.fmt == MOE_W_AFFINE4) ? L.cols / L.group_size : (L.fmt == MOE_W_MXFP4 ? L.cols / 32 : 0);
  m.s_stride = (int64_t)m.lds * L.rows;
  return m;
}

int wf_of(const moe_linear &L) { return L.fmt == MOE_W_DENSE ? WF_DENSE : (L.fmt == MOE_W_AFFINE4 ? WF_AFFINE4 : WF_MXFP4); }

// moe_set_decode_fusion: 1 (default) three launches; 2 one launch up to 16 tokens (three
// above); 0 the separate launches
int g_decode_fusion = 1;

// ---------------------------------------------------------------------------
// optional live timing of one kernel class (moe_timing_enable / moe_timing_read)
// ---------------------------------------------------------------------------
enum { TK_OFF = 0, TK_GATEUP = 1, TK_DOWN = 2, TK_ROUTER = 3, TK_TOPK = 4, TK_PERM = 5, TK_COMBINE = 6, TK_PLAIN = 7,
       TK_FUSED = 8 };
constexpr int kTimingPairs = 8192;
struct Timing {
  int kind = TK_OFF;
  hipEvent_t ev[2 * kTimingPairs];
  bool created = false;
  int used = 0;
} g_timing;

// Times one launch of a class when that class is being timed.  By default the launch is
// bracketed with event records on its stream; with `in_dispatch` the caller hands start()
// and stop() to hipExtLaunchKernelGGL, which stamps them at the kernel's own start and end
// (what a kernel-trace profiler reports), without the cost of the records themselves.
struct Timed {
  int slot = -1;
  bool ext;
  hipStream_t s;
  Timed(int kind, hipStream_t st, bool in_dispatch = false) : ext(in_dispatch), s(st) {
    if (g_timing.kind == kind && g_timing.used < kTimingPairs) {
      slot = g_timing.used++;
      if (!ext) (void)hipEventRecord(g_timing.ev[2 * slot], s);
    }
  }
  hipEvent_t start() const { return slot >= 0 ? g_timing.ev[2 * slot] : nullptr; }
  hipEvent_t stop() const { return slot >= 0 ? g_timing.ev[2 * slot + 1] : nullptr; }
  ~Timed() {
    if (slot >= 0 && !ext) (void)hipEventRecord(g_timing.ev[2 * slot + 1], s);
  }
};

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
// slices of the tiled router's reduction (1 when it does not apply): enough 128x64 tiles x
// slices for ~1.5 workgroups per CU, slices of whole 64-element chunks.  The slice length
// depends on the experts, not on the blend head's two extra rows, so that moe_route and
// moe_block_forward sum alike.
bool router_tiled(int x_dt, int T, int H, int E) {
  return x_dt == MOE_BF16 && T >= MOE_ROUTER_GEMM_T && E % 8 == 0 && (int64_t)T * H * 2 <= INT32_MAX &&
         (int64_t)E * H * 2 <= INT32_MAX;
}
// The slice count is a function of (T, H, E) alone (sized for MI355X's 256 CUs, not read from
// the device), so the summation order of the logits, and with it the selection at near-ties,
// is the same on every device and partition.
constexpr int kRouterSliceCUs = 256;
int router_slice_len(int T, int H, int E) {
  const int tiles = ((T + 127) / 128) * ((E + 63) / 64);
  int S = (3 * kRouterSliceCUs / 2 + tiles - 1) / tiles;
  S = S < 1 ? 1 : (S > 16 ? 16 : S);
  return (((H + S - 1) / S) + 63) / 64 * 64;
}
int router_slices(int x_dt, int T, int H, int E, bool split) {
  if (!split || !router_tiled(x_dt, T, H, E)) return 1;
  const int ks = router_slice_len(T, H, E);
  return (H + ks - 1) / ks;
}

// router logits (+ the blend head's two logits into clog when coef_w is given).  split: the
// tiled router may write `slices` partial sums (logits + z*T*E, clog + z*2T), added in order by
// the selection.
moe_status launch_router(const void *x, int x_dt, int T, int H, const moe_router *r, const void *coef_w,
                         const float *coef_b, float *logits, float *clog, hipStream_t s, int *zero = nullptr,
                         bool split = false, int zero_n = 1) {
  const int E = r->num_experts;
  const int R = E + (coef_w ? 2 : 0);
  Timed tm(TK_ROUTER, s);
  if (router_tiled(x_dt, T, H, E)) {
    const int ks = split ? router_slice_len(T, H, E) : ((H + 63) / 64) * 64;
    const int S = (H + ks - 1) / ks;
    hipLaunchKernelGGL(router_gemm_bf16, dim3((T + 127) / 128, (R + 63) / 64, S), dim3(256), 0, s,
                       (const uint16_t *)x, (const uint16_t *)r->w, r->logit_bias, logits, T, H, E,
                       (const uint16_t *)coef_w, coef_b, clog, zero, zero_n, ks);
  } else if (x_dt == MOE_BF16) {
    hipLaunchKernelGGL(router_logits_bf16, dim3((T + 15) / 16, (R + 15) / 16), dim3(512), 0, s, (const uint16_t *)x,
                       (const uint16_t *)r->w, r->logit_bias, logits, T, H, E, (const uint16_t *)coef_w, coef_b,
                       clog, zero, zero_n);
  } else {
    const int64_t n = (int64_t)T * R;
    hipLaunchKernelGGL(router_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float *)x,
                       (const float *)r->w, r->logit_bias, logits, T, H, E, (const float *)coef_w, coef_b, clog,
                       zero, zero_n);
  }
  HIPCHK(hipGetLastError());
  return MOE_OK;
}

TopkArgs topk_args(int T, const moe_router *r, const float *logits, int32_t *idx, float *w, const float *clog,
                   float *coef, int slices = 1) {
  TopkArgs a;
  a.logits = logits;
  a.slices = slices;
  a.logits_out = nullptr;
  a.T = T;
  a.E = r->num_experts;
  a.K = r->top_k;
  a.scoring = r->scoring;
  a.norm = r->norm_topk;
  a.rscale = r->routed_scale;
  a.sbias = r->select_bias;
  a.idx = idx;
  a.w = w;
  a.clog = clog;
  a.coef = coef;
  return a;
}

// experts per lane of a 32-lane selection group (K <= 16), or 0 for the wave-per-token path
int topk_slots(int E, int K) {
  if (K > 16) return 0;
  return E <= 128 ? 4 : (E <= 256 ? 8 : 16);
}

moe_status launch_topk(const TopkArgs &a, hipStream_t s) {
  Timed tm(TK_TOPK, s);
  const dim3 g((a.T + 7) / 8);
  switch (topk_slots(a.E, a.K)) {
    case 4: hipLaunchKernelGGL(topk_half_kernel<4>, g, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(topk_half_kernel<8>, g, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL(topk_half_kernel<16>, g, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a); break;
  }
  HIPCHK(hipGetLastError());
  return MOE_OK;
}

// selection + permutation + tile list in one launch (T <= MOE_ROUTE_SMALL_T, K <= 16); done:
// a counter the router launch has set to zero
moe_status launch_route_decode(const TopkArgs &a, int32_t *counts, int32_t *offsets, int32_t *ss, int32_t *sp,
                               int4 *tiles, int *tc, int mt, int *done, hipStream_t s) {
  Timed tm(TK_TOPK, s);
  const dim3 g((a.T + 7) / 8), b(256);
  switch (topk_slots(a.E, a.K)) {
    case 4: hipLaunchKernelGGL(route_decode<4>, g, b, 0, s, a, counts, offsets, ss, sp, tiles, tc, mt, done); break;
    case 8: hipLaunchKernelGGL(route_decode<8>, g, b, 0, s, a, counts, offsets, ss, sp, tiles, tc, mt, done); break;
    case 16: hipLaunchKernelGGL(route_decode<16>, g, b, 0, s, a, counts, offsets, ss, sp, tiles, tc, mt, done); break;
    default: return fail(MOE_ERR_UNSUPPORTED, "route_decode needs top_k <= 16");
  }
  HIPCHK(hipGetLastError());
  return MOE_OK;
}

size_t perm_ws_bytes(int64_t T, int E) { return T <= 256 ? 0 : (size_t)((T + 255) / 256) * E * 4; }

// done / status: a counter that is zero when the launch starts and the status word (the
// block's router launch clears both): then more than 256 tokens take the single-launch
// permutation (up to kPermFusedChunks chunks of 256 tokens), else count, scan and scatter
moe_status launch_permute(const int32_t *idx, int T, int K, int E, int32_t *counts, int32_t *offsets, int32_t *ss,
                          int32_t *sp, int32_t *chunk_ws, int4 *tiles, int *tile_count, int mt, hipStream_t s,
                          int *done = nullptr, int *status = nullptr) {
  Timed tm(TK_PERM, s);
  if (T <= 256) {
    hipLaunchKernelGGL(perm_small, dim3(1), dim3(256), 0, s, idx, T, K, E, counts, offsets, ss, sp, tiles, tile_count,
                       mt);
    HIPCHK(hipGetLastError());
    return MOE_OK;
  }
  const int nch = (T + 255) / 256;
  if (done && status && nch <= kPermFusedChunks) {
    hipLaunchKernelGGL(perm_fused, dim3(nch), dim3(256), 0, s, idx, T, K, E, chunk_ws, counts, offsets, ss, sp, tiles,
                       tile_count, mt, done, status);
    HIPCHK(hipGetLastError());
    return MOE_OK;
  }
  hipLaunchKernelGGL(perm_count, dim3(nch), dim3(256), 0, s, idx, T, K, E, chunk_ws);
  HIPCHK(hipGetLastError());
  hipLaunchKernelGGL(perm_scan, dim3(1), dim3(1024), 0, s, chunk_ws, nch, E, T * K, counts, offsets, tiles,
                     tile_count, mt);
  HIPCHK(hipGetLastError());
  hipLaunchKernelGGL(perm_scatter, dim3(nch), dim3(256), 0, s, idx, T, K, E, chunk_ws, ss, sp);
  HIPCHK(hipGetLastError());
  return MOE_OK;
}

// routed m-tiles of at most mt rows: sum over experts of ceil(n_e / mt) <= TK / mt + min(E, TK)
int routed_tiles_ub(int TK, int E, int mt) { return TK / mt + (E < TK ? E : TK); }
int max_tiles(int TK, int E) { return routed_tiles_ub(TK, E, MOE_MT_MIN) + 1; }

// m-blocks (16 rows each) per m-tile: 1 for decode-sized segments (the HBM-streaming
// kernels), 8 otherwise (the 128-row MFMA kernel of moe_gemm_tall.hip).  Kernel codes: 0 and
// 1 the decode kernels of moe_gemm.hip (0: SHORT), MB_WS the loader-wave decode kernel of
// moe_gemm_ws.hip (4-bit weights; same units as 1), MB_TALL the prefill kernel.
constexpr int MB_WS = 2;
constexpr int MB_TALL = 8;
int pick_mb(double avg_rows) { return avg_rows <= 16.0 ? 1 : MB_TALL; }
int mb_for_routing(int TK, int E) { return pick_mb((double)TK / (E < TK ? E : (TK > 0 ? TK : 1))); }

// kmb: a kernel code (see above); per_cu: resident workgroups per CU
int gemm_grid(int units_ub, int kmb, int per_cu = 0) {
  if (per_cu <= 0) per_cu = kmb == 0 ? 4 : (kmb == 1 ? 3 : 1);
  const int cap = per_cu * device_cus();
  return units_ub < cap ? units_ub : cap;
}

// output column blocks of a segment: the decode kernel's 4 waves cover 64 gate/up outputs or
// 128 rows, the tall kernel's 8 waves twice that
int col_blocks(const SegSet &sg, bool gateup, int mb) {
  const int w = (gateup ? 64 : 128) * (mb == MB_TALL ? 2 : 1);
  return (sg.w0.rows + w - 1) / w;
}

hipError_t launch_gemm_kernel(int adt, const moe_linear &fmt_of, bool gateup, int odt, int kmb, const GemmParams &p,
                              int units_ub, hipStream_t s, hipEvent_t e0, hipEvent_t e1, bool scaled = false) {
  const int adt_k = adt == MOE_BF16 ? DT_BF16 : DT_F16;
  const int odt_k = odt == MOE_F32 ? DT_F32 : (odt == MOE_BF16 ? DT_BF16 : DT_F16);
  if (kmb == MB_WS)
    return launch_expert_gemm_ws(adt_k, wf_of(fmt_of), fmt_of.group_size, gateup, odt_k, p,
                                 gemm_grid(units_ub, kmb, ws_wgs_per_cu(wf_of(fmt_of), fmt_of.group_size)), s, e0,
                                 e1);
  if (kmb == MB_TALL)
    return launch_expert_gemm_tall(adt_k, scaled ? WF_MXS : wf_of(fmt_of), fmt_of.group_size, gateup, odt_k, p,
                                   gemm_grid(units_ub, kmb), s, e0, e1);
  return launch_expert_gemm(adt_k, wf_of(fmt_of), fmt_of.group_size, gateup, odt_k, kmb, p, gemm_grid(units_ub, kmb),
                            s, e0, e1);
}

// decode launches of 4-bit weights use the loader-wave kernel (also for short reductions, where
// it measured faster than the SHORT variant); DENSE decode LINEAR launches whose longest
// reduction spans at most three chunks use the SHORT variant
int kernel_mb(int mb, bool gateup, const moe_linear &w, int kmax) {
  if (mb != 1) return mb;
  if (w.fmt != MOE_W_DENSE) return MB_WS;
  const int kc = 64;
  return (!gateup && (kmax + kc - 1) / kc <= 3) ? 0 : mb;
}

AOp aop(const void *a, int64_t lda, const int32_t *gather, int gdiv, int row_sub, int64_t rows) {
  AOp o;
  o.a = a;
  o.lda = lda;
  o.gather = gather;
  o.gdiv = gdiv;
  o.row_sub = row_sub;
  o.rows = rows;
  o.as = nullptr;
  o.ldas = 0;
  return o;
}

// the tall kernel addresses its activation rows with 32-bit byte offsets, the loader-wave
// kernel with 31-bit ones (and the packed matrices likewise)
bool offsets_fit(const GemmParams &p, int64_t lim) {
  for (int i = 0; i < 2; ++i)
    if (p.seg[i].nblk > 0 && (p.seg[i].A.rows * p.seg[i].A.lda * 2 > lim || p.seg[i].w0.pk_mat > lim)) return false;
  return true;
}
bool tall_offsets_fit(const GemmParams &p) { return offsets_fit(p, (int64_t)UINT32_MAX); }

SegSet segset(AOp A, const moe_linear &w0, const moe_linear *w1, float limit, bool gateup) {
  SegSet s;
  s.A = A;
  s.w0 = wmat(w0, gateup);
  s.w1 = w1 ? wmat(*w1, gateup) : s.w0;
  s.limit = limit;
  s.K = w0.cols;
  s.nblk = 0;  // set by the launch (col_blocks) for the kernel it picks
  return s;
}

// routed experts (m-tiles of 16*mb rows from the tile list) + optional segment-1 rows
// [sh_row0, sh_row0 + sh_rows) (the shared expert) in the same launch
GemmParams gemm_params(bool gateup, int mb, const SegSet &routed, const SegSet *shared, int sh_row0, int sh_rows,
                       const int4 *tiles, const int *tile_count, int ntiles_alloc, int E, void *out, int64_t ldo,
                       const float *resid, int64_t ldr) {
  GemmParams p;
  memset(&p, 0, sizeof p);
  p.seg[0] = routed;
  p.seg[0].nblk = col_blocks(routed, gateup, mb);
  p.seg[1] = shared ? *shared : routed;
  p.seg[1].nblk = shared ? col_blocks(*shared, gateup, mb) : 0;
  p.tiles = tiles;
  p.tile_count = tile_count;
  p.max_tiles = ntiles_alloc;
  p.sh_row0 = sh_row0;
  p.sh_rows = shared ? sh_rows : 0;
  p.E = E;
  p.out = out;
  p.ldo = ldo;
  p.resid = resid;
  p.ldr = ldr;
  return p;
}

// scaled: the prefill kernel on the block-scaled MFMA (routed.A: split FP8 activations with
// their scale pairs; routed.w0.pk: the moe_pack_weights_scaled stream)
moe_status run_gemm(int adt, const moe_linear &fmt_of, bool gateup, int odt, int mb, const SegSet &routed,
                    const SegSet *shared, int sh_row0, int sh_rows, const int4 *tiles, const int *tile_count,
                    int ntiles_alloc, int TK, int E, void *out, int64_t ldo, const float *resid, int64_t ldr,
                    hipStream_t s, bool scaled = false) {
  const int mt = 16 * mb;
  const GemmParams p = gemm_params(gateup, mb, routed, shared, sh_row0, sh_rows, tiles, tile_count, ntiles_alloc, E,
                                   out, ldo, resid, ldr);
  if (!shared) sh_rows = 0;
  const int units_ub = routed_tiles_ub(TK, E, mt) * p.seg[0].nblk + ((sh_rows + mt - 1) / mt) * p.seg[1].nblk;
  int kmb = kernel_mb(mb, gateup, fmt_of, shared && shared->K > routed.K ? shared->K : routed.K);
  if (kmb == MB_WS && !offsets_fit(p, INT32_MAX)) kmb = 1;
  CHECK(kmb != MB_TALL || tall_offsets_fit(p), MOE_ERR_SHAPE, "activation operand of over 4 GiB");
  Timed tm(gateup ? TK_GATEUP : TK_DOWN, s, true);
  CHECK(!scaled || kmb == MB_TALL, MOE_ERR_UNSUPPORTED, "the block-scaled MFMA runs on the prefill kernel only");
  HIPCHK(launch_gemm_kernel(adt, fmt_of, gateup, odt, kmb, p, units_ub, s, tm.start(), tm.stop(), scaled));
  return MOE_OK;
}

// a plain GEMM over `rows` rows (no routing): out[r] = W a[r] (+ resid)
moe_status run_plain(int adt, const moe_linear &W, const moe_linear *W1, float limit, bool gateup, int odt,
                     const void *a, int64_t lda, int rows, void *out, int64_t ldo, const float *resid, int64_t ldr,
                     hipStream_t s) {
  const int mb = pick_mb(rows);
  const int mt = 16 * mb;
  SegSet sg = segset(aop(a, lda, nullptr, 1, 0, rows), W, W1, limit, gateup);
  sg.nblk = col_blocks(sg, gateup, mb);
  SegSet none = sg;
  none.nblk = 0;
  // plain mode: every m-tile is a segment-1 tile; the routed set has no units
  GemmParams p;
  memset(&p, 0, sizeof p);
  p.seg[0] = none;
  p.seg[1] = sg;
  p.tiles = nullptr;
  p.tile_count = nullptr;
  p.max_tiles = 0;
  p.sh_row0 = 0;
  p.sh_rows = rows;
  p.E = 0;
  p.out = out;
  p.ldo = ldo;
  p.resid = resid;
  p.ldr = ldr;
  int units = ((rows + mt - 1) / mt) * sg.nblk;
  int kmb = kernel_mb(mb, gateup, W, W.cols);
  if (kmb == MB_WS && !offsets_fit(p, INT32_MAX)) kmb = 1;
  CHECK(kmb != MB_TALL || tall_offsets_fit(p), MOE_ERR_SHAPE, "activation operand of over 4 GiB");
  // prefill kernel: 64-row m-tiles when 128-row ones leave over a quarter of the CUs idle
  if (kmb == MB_TALL && rows > 64 && 4 * units < 3 * device_cus()) {
    p.sh_mt = 64;
    units = ((rows + 63) / 64) * sg.nblk;
  }
  Timed tm(TK_PLAIN, s, true);
  HIPCHK(launch_gemm_kernel(adt, W, gateup, odt, kmb, p, units, s, tm.start(), tm.stop()));
  return MOE_OK;
}

moe_status combine(int odt, int ydt, const void *o, int64_t ldo, const int32_t *slot_pos, const float *topk_w, int K,
                   int TK, int T, int D, void *y, int64_t ldy, const float *coef, const float *norm_w, float eps,
                   int mode, hipStream_t s) {
  CombineArgs a;
  a.o = o;
  a.ldo = ldo;
  a.slot_pos = slot_pos;
  a.topk_w = topk_w;
  a.K = K;
  a.TK = TK;
  a.T = T;
  a.D = D;
  a.y = y;
  a.ldy = ldy;
  a.coef = coef;
  a.norm_w = norm_w;
  a.eps = eps;
  a.mode = mode;
  auto k = [](int dt) { return dt == MOE_F32 ? DT_F32 : (dt == MOE_BF16 ? DT_BF16 : DT_F16); };
  Timed tm(TK_COMBINE, s);
  HIPCHK(launch_combine(k(odt), k(ydt), a, s));
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// counters of the decode launches: one block per stream that runs them (up to kCounterSlots
// streams per device), in the code object: zero when it loads, and each call's routing launch
// leaves the counters it used zero and clears the ones the experts launch uses.  Calls on one
// stream are ordered, so no two use a block at the same time.  As with `scratch` below, host
// code uses only the device address looked up for each GPU.  A graph captured on one stream
// may be replayed on another, beside calls on the first, so a capturing stream takes the
// separate launches.
// ---------------------------------------------------------------------------
// Each slot holds three blocks: [0] the three-launch path's, [1] and [2] the single launch's,
// used in turn (each call clears the other one for the next call).
constexpr int kCounterSlots = 16;
static __device__ __align__(256) int fused_counters[kCounterSlots][3][kCounterInts];

constexpr int kCounterDevices = 64;
std::mutex g_counter_mu;
int *g_counter_ptr[kCounterDevices] = {};
hipStream_t g_counter_stream[kCounterDevices][kCounterSlots];
int g_counter_used[kCounterDevices] = {};
int g_counter_turn[kCounterDevices][kCounterSlots] = {};  // the single launch's next block (0 or 1)

// the counter blocks of stream s (on the calling thread's current device), or nullptr: s is
// capturing or on another device, or every slot already belongs to another stream.  *turn
// (when given) is the slot's single-launch turn, which the caller flips after a launch.
int *counters_for(hipStream_t s, int **turn = nullptr) {
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kCounterDevices) return nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamGetDevice(s, &sdev) != hipSuccess || sdev != dev || hipStreamIsCapturing(s, &cap) != hipSuccess ||
      cap != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_counter_mu);
  if (g_counter_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(fused_counters)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_counter_ptr[dev] = (int *)ptr;
  }
  int i = 0;
  while (i < g_counter_used[dev] && g_counter_stream[dev][i] != s) ++i;
  if (i == g_counter_used[dev]) {
    if (i == kCounterSlots) return nullptr;
    g_counter_stream[dev][i] = s;
    ++g_counter_used[dev];
  }
  if (turn) *turn = &g_counter_turn[dev][i];
  return g_counter_ptr[dev] + (size_t)i * 3 * kCounterInts;
}

// ---------------------------------------------------------------------------
// scratch memory of moe_block_forward_noalloc: one array per GPU, in the code object, held
// until the process ends.  Host code never uses the array's name as an address (on the host
// it is only a stand-in for the symbol): the device address of each GPU's copy is looked up
// once, with that GPU current, and kept here.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// the device address of `scratch` on device dev (the calling thread's current device)
moe_status scratch_on(int dev, void **out) {
  CHECK(dev >= 0 && dev < kMaxDevices, MOE_ERR_DEVICE, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    HIPCHK(hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)));
    CHECK(ptr != nullptr, MOE_ERR_DEVICE, "hipGetSymbolAddress returned NULL for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

// ===========================================================================
// entry points
// ===========================================================================
extern "C" {

const char *moe_status_str(int32_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
    case MOE_ERR_QUANT: return "MOE_ERR_QUANT";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char *moe_last_error(void) { return g_err; }

int32_t moe_abi_version(void) { return (3 << 16) | 0; }

static moe_status pack_stream(const moe_linear *a, const moe_linear *b, void *out, size_t *out_bytes, void *stream,
                              bool scaled) {
  CHECK(out_bytes != nullptr, MOE_ERR_ARG, "out_bytes is NULL");
  CHECK(a != nullptr, MOE_ERR_ARG, "weight descriptor is NULL");
  CHECK(a->fmt == MOE_W_AFFINE4 || a->fmt == MOE_W_MXFP4 || (a->fmt == MOE_W_DENSE && a->dense_dtype == MOE_BF16),
        MOE_ERR_UNSUPPORTED, "packing needs AFFINE4, MXFP4 or DENSE BF16 weights (fmt %d)", a->fmt);
  TRY(check_linear(a, b ? "gate" : "weights", a->n, a->rows, a->cols, MOE_BF16, USE_SOURCE));
  if (b) {
    TRY(check_linear(b, "up", a->n, a->rows, a->cols, MOE_BF16, USE_SOURCE));
    CHECK(b->fmt == a->fmt && b->group_size == a->group_size && b->dense_dtype == a->dense_dtype,
          MOE_ERR_UNSUPPORTED, "gate and up stacks must share one format");
  }
  const WMat m = wmat(*a, b != nullptr);
  const size_t need = (size_t)a->n * (size_t)m.pk_mat;
  if (out == nullptr) {
    *out_bytes = need;
    return MOE_OK;
  }
  CHECK(*out_bytes >= need, MOE_ERR_WORKSPACE, "packed buffer %zu bytes, need %zu", *out_bytes, need);
  CHECK(aligned(out, 256), MOE_ERR_ARG, "packed buffer not 256-byte aligned");
  PackArgs pa;
  pa.wf = scaled ? WF_MXS : wf_of(*a);
  pa.gq = a->fmt == MOE_W_AFFINE4 ? a->group_size : (a->fmt == MOE_W_MXFP4 ? 32 : 0);
  pa.n = a->n;
  pa.rows = a->rows;
  pa.cols = a->cols;
  pa.gateup = b != nullptr;
  pa.dense_f32 = 0;
  pa.a_w = a->w;
  pa.a_s = a->scales;
  pa.a_q = a->qbias;
  pa.b_w = b ? b->w : nullptr;
  pa.b_s = b ? b->scales : nullptr;
  pa.b_q = b ? b->qbias : nullptr;
  pa.out = (uint32_t *)out;
  pa.nblk = m.pk_nblk;
  pa.nch = m.pk_nch;
  HIPCHK(launch_pack(pa, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_pack_weights(const moe_linear *a, const moe_linear *b, void *out, size_t *out_bytes, void *stream) {
  g_err[0] = 0;
  return pack_stream(a, b, out, out_bytes, stream, false);
}

moe_status moe_pack_weights_scaled(const moe_linear *a, const moe_linear *b, void *out, size_t *out_bytes,
                                   void *stream) {
  g_err[0] = 0;
  CHECK(a != nullptr, MOE_ERR_ARG, "weight descriptor is NULL");
  CHECK(a->fmt == MOE_W_MXFP4, MOE_ERR_UNSUPPORTED, "the block-scaled stream needs MXFP4 weights (fmt %d)", a->fmt);
  return pack_stream(a, b, out, out_bytes, stream, true);
}

moe_status moe_set_decode_fusion(int32_t enabled) {
  g_err[0] = 0;
  CHECK(enabled >= 0 && enabled <= 2, MOE_ERR_ARG, "the decode launch mode must be 0, 1 or 2 (got %d)", enabled);
  g_decode_fusion = enabled;
  return MOE_OK;
}

moe_status moe_timing_enable(int32_t kind) {
  g_err[0] = 0;
  CHECK(kind >= TK_OFF && kind <= TK_FUSED, MOE_ERR_ARG, "timing kind %d out of range", kind);
  if (kind != TK_OFF && !g_timing.created) {
    for (int i = 0; i < 2 * kTimingPairs; ++i) HIPCHK(hipEventCreate(&g_timing.ev[i]));
    g_timing.created = true;
  }
  g_timing.kind = kind;
  return MOE_OK;
}

moe_status moe_timing_read(int32_t *launches, double *total_ms) {
  g_err[0] = 0;
  CHECK(launches != nullptr && total_ms != nullptr, MOE_ERR_ARG, "output pointers must be non-NULL");
  double tot = 0.0;
  for (int i = 0; i < g_timing.used; ++i) {
    HIPCHK(hipEventSynchronize(g_timing.ev[2 * i + 1]));
    float ms = 0.f;
    HIPCHK(hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]));
    tot += ms;
  }
  *launches = g_timing.used;
  *total_ms = tot;
  g_timing.used = 0;
  return MOE_OK;
}

moe_status moe_route(const void *x, int32_t x_dtype, int64_t T, int32_t H, const moe_router *r, int32_t *topk_idx,
                     float *topk_w, float *logits, void *ws, size_t *ws_bytes, void *stream) {
  g_err[0] = 0;
  CHECK(x_dtype == MOE_F32 || x_dtype == MOE_BF16, MOE_ERR_ARG, "x dtype %d not F32/BF16", x_dtype);
  CHECK(H > 0, MOE_ERR_SHAPE, "hidden %d must be positive", H);
  TRY(check_router(r, H, x_dtype));
  TRY(check_tokens(T, r->top_k));
  Plan pl;
  // the router's slices as in moe_block_forward (same sums, same selection); the summed logits
  // go to `logits` when given
  const int rs = T > INT32_MAX ? 1 : router_slices(x_dtype, (int)T, H, r->num_experts, true);
  const size_t o_logits = pl.take((size_t)rs * T * r->num_experts * 4);
  bool query;
  TRY(check_ws(ws, ws_bytes, pl.off, &query));
  if (query || T == 0) return MOE_OK;
  CHECK(x && topk_idx && topk_w, MOE_ERR_ARG, "x, topk_idx and topk_w must be non-NULL");
  CHECK(aligned(x, 16), MOE_ERR_ARG, "x not 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  float *lg = at<float>(ws, o_logits);
  TRY(launch_router(x, x_dtype, (int)T, H, r, nullptr, nullptr, lg, nullptr, s, nullptr, true));
  TopkArgs ta = topk_args((int)T, r, lg, topk_idx, topk_w, nullptr, nullptr, rs);
  ta.logits_out = logits;
  TRY(launch_topk(ta, s));
  return MOE_OK;
}

moe_status moe_permute(const int32_t *topk_idx, int64_t T, int32_t K, int32_t E, int32_t *counts, int32_t *offsets,
                       int32_t *sorted_slot, int32_t *slot_pos, void *ws, size_t *ws_bytes, void *stream) {
  g_err[0] = 0;
  CHECK(E > 0 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "num_experts %d outside 1..%d", E, MOE_MAX_EXPERTS);
  CHECK(K >= 1 && K <= E && K <= MOE_MAX_TOPK, MOE_ERR_SHAPE, "top_k %d outside 1..min(E, %d)", K, MOE_MAX_TOPK);
  TRY(check_tokens(T, K));
  Plan pl;
  const size_t o_chunk = pl.take(perm_ws_bytes(T, E));
  bool query;
  TRY(check_ws(ws, ws_bytes, pl.off, &query));
  if (query || T == 0) return MOE_OK;
  CHECK(topk_idx && counts && offsets && sorted_slot && slot_pos, MOE_ERR_ARG,
        "topk_idx, counts, offsets, sorted_slot and slot_pos must be non-NULL");
  TRY(launch_permute(topk_idx, (int)T, K, E, counts, offsets, sorted_slot, slot_pos, at<int32_t>(ws, o_chunk), nullptr,
                     nullptr, MOE_MT_MIN, (hipStream_t)stream));
  return MOE_OK;
}

moe_status moe_experts_forward(const void *z, int32_t z_dtype, int64_t T, int32_t D, const moe_mlp *ex, int32_t E,
                               int32_t K, const int32_t *topk_idx, const float *topk_w, const int32_t *offsets,
                               const int32_t *sorted_slot, const int32_t *slot_pos, int32_t inter_dtype,
                               float *y_routed, void *ws, size_t *ws_bytes, void *stream) {
  g_err[0] = 0;
  CHECK(z_dtype == MOE_F32 || z_dtype == MOE_BF16 || z_dtype == MOE_F16, MOE_ERR_ARG, "z dtype %d out of range",
        z_dtype);
  CHECK(D > 0, MOE_ERR_SHAPE, "expert_dim %d must be positive", D);
  CHECK(E > 0 && E <= MOE_MAX_EXPERTS, MOE_ERR_SHAPE, "num_experts %d outside 1..%d", E, MOE_MAX_EXPERTS);
  CHECK(K >= 1 && K <= E && K <= MOE_MAX_TOPK, MOE_ERR_SHAPE, "top_k %d outside 1..min(E, %d)", K, MOE_MAX_TOPK);
  TRY(check_tokens(T, K));
  CHECK(ex != nullptr, MOE_ERR_ARG, "expert descriptor is NULL");
  if (z_dtype == MOE_F32) {
    CHECK(inter_dtype == MOE_F32, MOE_ERR_UNSUPPORTED, "f32 activations need inter_dtype F32");
  } else {
    CHECK(inter_dtype == MOE_BF16 || inter_dtype == MOE_F16, MOE_ERR_ARG, "inter_dtype %d not BF16/F16", inter_dtype);
  }
  const int I = ex->gate.rows;
  CHECK(I > 0, MOE_ERR_SHAPE, "expert intermediate %d must be positive", I);
  TRY(check_mlp(ex, "experts", E, I, D, z_dtype, inter_dtype));
  CHECK(z_dtype != MOE_F32 || D % 8 == 0, MOE_ERR_SHAPE, "expert_dim %d not a multiple of 8", D);
  const int TK = (int)(T * K);
  const int isz = dt_size(inter_dtype);
  Plan pl;
  const bool mf = z_dtype != MOE_F32;
  const int ntile = max_tiles(TK, E);
  const size_t o_tiles = mf ? pl.take((size_t)ntile * 16) : 0;
  const size_t o_tcount = mf ? pl.take(16) : 0;
  const size_t o_h = pl.take((size_t)TK * I * isz);
  const size_t o_o = pl.take((size_t)TK * D * isz);
  bool query;
  TRY(check_ws(ws, ws_bytes, pl.off, &query));
  if (query || T == 0) return MOE_OK;
  CHECK(z && topk_idx && topk_w && offsets && sorted_slot && slot_pos && y_routed, MOE_ERR_ARG,
        "a required pointer is NULL");
  CHECK(aligned(z, 16) && aligned(y_routed, 16), MOE_ERR_ARG, "z / y_routed not 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  void *h = at<char>(ws, o_h);
  void *o = at<char>(ws, o_o);
  if (mf) {
    int4 *tiles = at<int4>(ws, o_tiles);
    int *tc = at<int>(ws, o_tcount);
    const int mb = mb_for_routing(TK, E);
    hipLaunchKernelGGL(build_tiles, dim3(1), dim3(256), 0, s, offsets, E, tiles, tc, 16 * mb);
    HIPCHK(hipGetLastError());
    SegSet gu = segset(aop(z, D, sorted_slot, K, 0, T), ex->gate, &ex->up, ex->swiglu_limit, true);
    TRY(run_gemm(z_dtype, ex->gate, true, inter_dtype, mb, gu, nullptr, 0, 0, tiles, tc, ntile, TK, E, h, I, nullptr,
                 0, s));
    SegSet dn = segset(aop(h, I, nullptr, 1, 0, TK), ex->down, nullptr, 0.f, false);
    TRY(run_gemm(inter_dtype, ex->down, false, inter_dtype, mb, dn, nullptr, 0, 0, tiles, tc, ntile, TK, E, o, D,
                 nullptr, 0, s));
  } else {
    F32GemmParams p;
    memset(&p, 0, sizeof p);
    p.a_routed = (const float *)z;
    p.lda_r = D;
    p.sorted_slot = sorted_slot;
    p.topk_idx = topk_idx;
    p.K = K;
    p.TK = TK;
    p.Tsh = 0;
    p.r0 = wmat(ex->gate);
    p.r1 = wmat(ex->up);
    p.limit = ex->swiglu_limit;
    p.out = (float *)h;
    p.ldo = I;
    p.ncols_r = I;
    p.gateup = 1;
    {
      Timed tm(TK_GATEUP, s);
      HIPCHK(launch_f32_gemm(p, TK, s));
    }
    p.a_routed = (const float *)h;
    p.lda_r = I;
    p.r0 = wmat(ex->down);
    p.out = (float *)o;
    p.ldo = D;
    p.ncols_r = D;
    p.gateup = 0;
    {
      Timed tm(TK_DOWN, s);
      HIPCHK(launch_f32_gemm(p, TK, s));
    }
  }
  TRY(combine(inter_dtype, MOE_F32, o, D, slot_pos, topk_w, K, TK, (int)T, D, y_routed, D, nullptr, nullptr, 0.f, 0,
              s));
  return MOE_OK;
}

moe_status moe_block_forward(const void *x, int32_t x_dtype, int64_t T, const moe_block *b, void *y, int32_t y_dtype,
                             int32_t *topk_idx, float *topk_w, void *ws, size_t *ws_bytes, void *stream) {
  g_err[0] = 0;
  CHECK(b != nullptr, MOE_ERR_ARG, "block descriptor is NULL");
  CHECK(x_dtype == MOE_F32 || x_dtype == MOE_BF16, MOE_ERR_ARG, "x dtype %d not F32/BF16", x_dtype);
  CHECK(y_dtype == MOE_F32 || y_dtype == MOE_BF16, MOE_ERR_ARG, "y dtype %d not F32/BF16", y_dtype);
  CHECK(x_dtype == MOE_BF16 || y_dtype == MOE_F32, MOE_ERR_UNSUPPORTED, "f32 input needs f32 output");
  const int H = b->hidden;
  CHECK(H > 0 && b->expert_dim > 0, MOE_ERR_SHAPE, "hidden %d / expert_dim %d must be positive", H, b->expert_dim);
  TRY(check_router(&b->router, H, x_dtype));
  const int E = b->router.num_experts, K = b->router.top_k;
  TRY(check_tokens(T, K));
  const bool latent = b->latent_down.w != nullptr;
  const int D = b->expert_dim;
  CHECK(latent || D == H, MOE_ERR_SHAPE, "expert_dim %d != hidden %d without a latent projection", D, H);
  const int inter = b->inter_dtype;
  if (x_dtype == MOE_F32) {
    CHECK(inter == MOE_F32, MOE_ERR_UNSUPPORTED, "f32 input needs inter_dtype F32");
    CHECK(!latent, MOE_ERR_UNSUPPORTED, "the latent projection needs BF16 input");
  } else {
    CHECK(inter == MOE_BF16 || inter == MOE_F16, MOE_ERR_ARG, "inter_dtype %d not BF16/F16", inter);
  }
  const int zdt = latent ? inter : x_dtype;
  const int I = b->experts.gate.rows;
  CHECK(I > 0, MOE_ERR_SHAPE, "expert intermediate %d must be positive", I);
  TRY(check_mlp(&b->experts, "experts", E, I, D, zdt, inter));
  CHECK(b->shared_mode >= MOE_SHARED_NONE && b->shared_mode <= MOE_SHARED_BLEND, MOE_ERR_ARG,
        "shared_mode %d out of range", b->shared_mode);
  const bool has_shared = b->shared_mode != MOE_SHARED_NONE;
  int Is = 0;
  if (has_shared) {
    Is = b->shared.gate.rows;
    CHECK(Is > 0, MOE_ERR_SHAPE, "shared intermediate %d must be positive", Is);
    TRY(check_mlp(&b->shared, "shared", 1, Is, H, x_dtype, inter));
  }
  if (b->shared_mode == MOE_SHARED_BLEND) {
    CHECK(b->coef_w != nullptr && b->coef_b != nullptr, MOE_ERR_ARG,
          "blend needs the coefficient head (coef_w [2, H] and coef_b [2])");
    CHECK(!latent, MOE_ERR_UNSUPPORTED, "blend with the latent projection is not supported");
    CHECK(aligned(b->coef_w, 16), MOE_ERR_ARG, "coef_w not 16-byte aligned");
  }
  if (latent) {
    TRY(check_linear(&b->latent_down, "latent_down", 1, D, H, x_dtype, USE_GEMM));
    TRY(check_linear(&b->latent_up, "latent_up", 1, H, D, inter, USE_GEMM));
    CHECK(b->latent_down.fmt == MOE_W_DENSE && b->latent_up.fmt == MOE_W_DENSE, MOE_ERR_UNSUPPORTED,
          "latent projections must be DENSE BF16");
    if (b->latent_norm_w) {
      CHECK(std::isfinite(b->norm_eps) && b->norm_eps > 0.f, MOE_ERR_ARG, "norm_eps must be finite and > 0");
      CHECK(D <= 8192, MOE_ERR_SHAPE, "latent width %d above 8192 with the norm", D);
    }
  }
  CHECK(H % 8 == 0 && D % 8 == 0, MOE_ERR_SHAPE, "hidden/expert_dim must be multiples of 8");

  // ---- workspace
  const int TK = (int)(T * K);
  const int isz = dt_size(inter);
  const bool mf = x_dtype != MOE_F32;
  // shared expert inside the routed launches when it shares the routed format and input
  const bool fuse_shared = has_shared && !latent && mf && b->shared.gate.fmt == b->experts.gate.fmt &&
                           b->shared.gate.group_size == b->experts.gate.group_size &&
                           b->shared.down.fmt == b->experts.down.fmt &&
                           b->shared.down.group_size == b->experts.down.group_size;
  const int Tsh = (has_shared && !latent) ? (int)T : 0;  // shared rows appended to h / o
  const int ldh = I > Is ? I : Is;
  Plan pl;
  const bool blend = b->shared_mode == MOE_SHARED_BLEND;
  const int rs = (T > INT32_MAX) ? 1 : router_slices(x_dtype, (int)T, H, E, true);
  // the routing state and the status word first, at the offsets include/moe.h documents
  const int ntile = max_tiles(TK, E);
  const int mb = mb_for_routing(TK, E);
  const bool small = T <= MOE_ROUTE_SMALL_T && topk_slots(E, K) > 0;
  // the one-launch decode path: bf16 activations and intermediates, decode-sized segments,
  // 4-bit routed experts (and a shared expert of the same format, or none), the router's
  // logits in one tile pass
  const int ns_f = has_shared ? (int)((T + 15) / 16) : 0;
  bool fused = g_decode_fusion && mf && !latent && small && mb == 1 && x_dtype == MOE_BF16 && inter == MOE_BF16 &&
               b->experts.gate.fmt != MOE_W_DENSE && (!has_shared || fuse_shared) &&
               !router_tiled(x_dtype, (int)T, H, E) && E <= 256 && ns_f + ntile <= kMaxTileCnt;
  const size_t o_counts = pl.take((size_t)E * 4);
  const size_t o_offsets = pl.take((size_t)(E + 1) * 4);
  const size_t o_ss = pl.take((size_t)TK * 4);
  const size_t o_sp = pl.take((size_t)TK * 4);
  const size_t o_st = pl.take(2 * 4);  // [0] status, [1] route_decode's counter
  const size_t o_logits = pl.take((size_t)rs * T * E * 4);
  const size_t o_coef = pl.take((size_t)T * 2 * 4);
  const size_t o_clog = pl.take((size_t)rs * T * 2 * 4);
  const size_t o_idx = topk_idx ? 0 : pl.take((size_t)TK * 4);
  const size_t o_w = topk_w ? 0 : pl.take((size_t)TK * 4);
  const size_t o_chunk = pl.take(perm_ws_bytes(T, E));
  const size_t o_tiles = pl.take((size_t)ntile * 16);
  const size_t o_tc = pl.take(16);
  const size_t o_z = latent ? pl.take((size_t)T * D * isz) : 0;
  const size_t o_h = pl.take((size_t)(TK + Tsh) * ldh * isz);
  const size_t o_o = pl.take((size_t)(TK + Tsh) * D * isz);
  const size_t o_yn = latent ? pl.take((size_t)T * D * isz) : 0;
  const size_t o_hs = (latent && has_shared) ? pl.take((size_t)T * Is * isz) : 0;
  const size_t o_s = (latent && has_shared) ? pl.take((size_t)T * H * 4) : 0;
  // the routed experts of the latent layer on the block-scaled MFMA: both stacks carry the
  // scaled stream, prefill-sized segments, f16 intermediates, widths in whole 128-blocks
  const bool mxs = latent && b->experts.gate.packed_scaled != nullptr && b->experts.down.packed_scaled != nullptr &&
                   inter == MOE_F16 && mb == MB_TALL && D % 128 == 0 && I % 128 == 0;
  const size_t o_zhl = mxs ? pl.take((size_t)T * D * 2) : 0;
  const size_t o_zs = mxs ? pl.take((size_t)T * (D / 32) * 2) : 0;
  const size_t o_hhl = mxs ? pl.take((size_t)TK * I * 2) : 0;
  const size_t o_hsc = mxs ? pl.take((size_t)TK * (I / 32) * 2) : 0;
  // f16 intermediates on the prefill kernel: the gate/up launch reads an f16 copy of x, so
  // that its MFMAs and the dequantisation run in f16 (packed half-precision arithmetic)
  const bool x16 = !latent && mf && x_dtype == MOE_BF16 && inter == MOE_F16 && mb == MB_TALL;
  const size_t o_x16 = x16 ? pl.take((size_t)T * H * 2) : 0;
  bool query;
  TRY(check_ws(ws, ws_bytes, pl.off, &query));
  if (query || T == 0) return MOE_OK;
  CHECK(x && y, MOE_ERR_ARG, "x and y must be non-NULL");
  CHECK(aligned(x, 16) && aligned(y, 16), MOE_ERR_ARG, "x / y not 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  float *logits = at<float>(ws, o_logits);
  float *coef = at<float>(ws, o_coef);
  int32_t *idx = topk_idx ? topk_idx : at<int32_t>(ws, o_idx);
  float *wts = topk_w ? topk_w : at<float>(ws, o_w);
  int32_t *counts = at<int32_t>(ws, o_counts);
  int32_t *offsets = at<int32_t>(ws, o_offsets);
  int32_t *ss = at<int32_t>(ws, o_ss);
  int32_t *sp = at<int32_t>(ws, o_sp);
  int4 *tiles = at<int4>(ws, o_tiles);
  int *tc = at<int>(ws, o_tc);
  void *h = at<char>(ws, o_h);
  void *o = at<char>(ws, o_o);
  const int Ti = (int)T;

  // 1. router + selection (+ blend coefficients); the router launch clears the status word
  // and route_decode's counter (the decode launches have their own router)
  float *clog = at<float>(ws, o_clog);
  int *st = at<int>(ws, o_st);
  int *turn = nullptr;
  int *cnt = fused ? counters_for(s, &turn) : nullptr;
  fused = cnt != nullptr;  // (else separate launches)
  int *done = st + 1;
  if (!fused)
    TRY(launch_router(x, x_dtype, Ti, H, &b->router, blend ? b->coef_w : nullptr, blend ? b->coef_b : nullptr, logits,
                      clog, s, st, true, 2));
  const TopkArgs ta = topk_args(Ti, &b->router, logits, idx, wts, blend ? clog : nullptr, coef, rs);
  // 2. permutation + tile list (for a few tokens in the same workgroup as the selection; on
  // the one-launch decode path, inside that launch)
  if (fused) {
  } else if (small) {
    TRY(launch_route_decode(ta, counts, offsets, ss, sp, mf ? tiles : nullptr, mf ? tc : nullptr, 16 * mb, done, s));
  } else {
    TRY(launch_topk(ta, s));
    TRY(launch_permute(idx, Ti, K, E, counts, offsets, ss, sp, at<int32_t>(ws, o_chunk), mf ? tiles : nullptr,
                       mf ? tc : nullptr, 16 * mb, s, done, st));
  }

  if (!mf) {
    // ---- f32 path
    F32GemmParams p;
    memset(&p, 0, sizeof p);
    p.a_routed = (const float *)x;
    p.lda_r = H;
    p.a_shared = (const float *)x;
    p.lda_s = H;
    p.sorted_slot = ss;
    p.topk_idx = idx;
    p.K = K;
    p.TK = TK;
    p.Tsh = Tsh;
    p.r0 = wmat(b->experts.gate);
    p.r1 = wmat(b->experts.up);
    if (has_shared) {
      p.s0 = wmat(b->shared.gate);
      p.s1 = wmat(b->shared.up);
    }
    p.limit = b->experts.swiglu_limit;
    p.out = (float *)h;
    p.ldo = ldh;
    p.ncols_r = I;
    p.ncols_s = Is;
    p.gateup = 1;
    {
      Timed tm(TK_GATEUP, s);
      HIPCHK(launch_f32_gemm(p, TK + Tsh, s));
    }
    p.a_routed = (const float *)h;
    p.lda_r = ldh;
    p.a_shared = (const float *)h;
    p.lda_s = ldh;
    p.r0 = wmat(b->experts.down);
    if (has_shared) p.s0 = wmat(b->shared.down);
    p.out = (float *)o;
    p.ldo = D;
    p.ncols_r = D;
    p.ncols_s = has_shared ? D : 0;
    p.gateup = 0;
    {
      Timed tm(TK_DOWN, s);
      HIPCHK(launch_f32_gemm(p, TK + Tsh, s));
    }
    const int mode = !has_shared ? 0 : (blend ? 3 : 2);
    TRY(combine(MOE_F32, y_dtype, o, D, sp, wts, K, TK, Ti, D, y, H, coef, nullptr, 0.f, mode, s));
    return MOE_OK;
  }

  if (fused) {
    // 1-2. router, selection and permutation in one launch; 3-4. gate/up and down of every
    // slot (and the shared expert) in one persistent launch
    const SegSet gu = segset(aop(x, H, ss, K, 0, Ti), b->experts.gate, &b->experts.up, b->experts.swiglu_limit, true);
    SegSet gus, dns;
    if (has_shared) {
      gus = segset(aop(x, H, nullptr, 1, TK, Ti), b->shared.gate, &b->shared.up, b->shared.swiglu_limit, true);
      dns = segset(aop(h, ldh, nullptr, 1, 0, TK + Tsh), b->shared.down, nullptr, 0.f, false);
    }
    const SegSet dn = segset(aop(h, ldh, nullptr, 1, 0, TK + Tsh), b->experts.down, nullptr, 0.f, false);
    FusedParams fp;
    memset(&fp, 0, sizeof fp);
    // o: the per-slot outputs in token order (slot t*K + j; the shared expert's rows after)
    fp.gu = gemm_params(true, 1, gu, has_shared ? &gus : nullptr, TK, Tsh, tiles, tc, ntile, E, h, ldh, nullptr, 0);
    fp.dn = gemm_params(false, 1, dn, has_shared ? &dns : nullptr, TK, Tsh, tiles, tc, ntile, E, o, D, nullptr, 0);
    CHECK(offsets_fit(fp.gu, INT32_MAX) && offsets_fit(fp.dn, INT32_MAX), MOE_ERR_SHAPE,
          "operands of over 2 GiB on the decode path");
    fp.x = (const uint16_t *)x;
    fp.Wr = (const uint16_t *)b->router.w;
    fp.cw = blend ? (const uint16_t *)b->coef_w : nullptr;
    fp.lbias = b->router.logit_bias;
    fp.cb = blend ? b->coef_b : nullptr;
    fp.H = H;
    fp.ta = ta;
    fp.counts = counts;
    fp.offsets = offsets;
    fp.slot_pos = sp;
    fp.Dout = D;
    fp.cnt = cnt;
    fp.n_tile_cnt = ns_f + ntile;
    fp.status = st;
    const int tub = routed_tiles_ub(TK, E, 16);
    const int units_ub = tub * (fp.gu.seg[0].nblk + fp.dn.seg[0].nblk) + ns_f * (fp.gu.seg[1].nblk + fp.dn.seg[1].nblk);
    const int mode = !has_shared ? 0 : (blend ? 3 : 2);
    if (g_decode_fusion == 2 && T <= 16 && (y_dtype == MOE_F32 || y_dtype == MOE_BF16) && D % 32 == 0 &&
        D <= 32 * kMaxColCnt) {
      // up to 16 tokens: everything in one launch, the combine included
      fp.cnt = cnt + (size_t)(1 + *turn) * kCounterInts;
      fp.cnt_next = cnt + (size_t)(2 - *turn) * kCounterInts;
      fp.nr_ub = tub;
      fp.y = y;
      fp.ldy = H;
      fp.ydt = y_dtype == MOE_F32 ? DT_F32 : DT_BF16;
      fp.mode = mode;
      {
        Timed tm(TK_FUSED, s, true);
        HIPCHK(launch_decode_one(wf_of(b->experts.gate), b->experts.gate.group_size, DT_BF16, fp, units_ub, s,
                                 tm.start(), tm.stop()));
      }
      *turn ^= 1;
      return MOE_OK;
    }
    {
      Timed tm(TK_ROUTER, s);
      HIPCHK(launch_decode_route(fp, s));
    }
    {
      Timed tm(TK_FUSED, s, true);
      HIPCHK(launch_decode_fused(wf_of(b->experts.gate), b->experts.gate.group_size, DT_BF16, fp, units_ub, s,
                                 tm.start(), tm.stop()));
    }
    // 5. weighted combine + shared add/blend over the token-ordered rows
    TRY(combine(inter, y_dtype, o, D, nullptr, wts, K, TK, Ti, H, y, H, coef, nullptr, 0.f, mode, s));
    return MOE_OK;
  }

  if (!latent) {
    // 3. gate/up (+ SwiGLU) for every slot, shared rows appended
    const void *xa = x;
    int xdt = x_dtype;
    if (x16) {
      xa = at<char>(ws, o_x16);
      xdt = MOE_F16;
      HIPCHK(launch_bf16_to_f16(x, (void *)xa, T * H, s));
    }
    SegSet gu = segset(aop(xa, H, ss, K, 0, Ti), b->experts.gate, &b->experts.up, b->experts.swiglu_limit, true);
    SegSet gus;
    if (has_shared) gus = segset(aop(xa, H, nullptr, 1, TK, Ti), b->shared.gate, &b->shared.up, b->shared.swiglu_limit, true);
    TRY(run_gemm(xdt, b->experts.gate, true, inter, mb, gu, fuse_shared ? &gus : nullptr, TK, Tsh, tiles, tc,
                 ntile, TK, E, h, ldh, nullptr, 0, s));
    if (has_shared && !fuse_shared)
      TRY(run_plain(xdt, b->shared.gate, &b->shared.up, b->shared.swiglu_limit, true, inter, xa, H, Ti,
                    (char *)h + (size_t)TK * ldh * isz, ldh, nullptr, 0, s));
    // 4. down
    SegSet dn = segset(aop(h, ldh, nullptr, 1, 0, TK + Tsh), b->experts.down, nullptr, 0.f, false);
    SegSet dns;
    if (has_shared) dns = segset(aop(h, ldh, nullptr, 1, 0, TK + Tsh), b->shared.down, nullptr, 0.f, false);
    TRY(run_gemm(inter, b->experts.down, false, inter, mb, dn, fuse_shared ? &dns : nullptr, TK, Tsh, tiles, tc,
                 ntile, TK, E, o, D, nullptr, 0, s));
    if (has_shared && !fuse_shared)
      TRY(run_plain(inter, b->shared.down, nullptr, 0.f, false, inter, (char *)h + (size_t)TK * ldh * isz, ldh, Ti,
                    (char *)o + (size_t)TK * D * isz, D, nullptr, 0, s));
    // 5. weighted combine + shared add/blend
    const int mode = !has_shared ? 0 : (blend ? 3 : 2);
    TRY(combine(inter, y_dtype, o, D, sp, wts, K, TK, Ti, H, y, H, coef, nullptr, 0.f, mode, s));
    return MOE_OK;
  }

  // ---- latent flow: z = down_proj(x); experts in latent space; rms_norm; up_proj; + shared(x)
  void *z = at<char>(ws, o_z);
  void *yn = at<char>(ws, o_yn);
  TRY(run_plain(x_dtype, b->latent_down, nullptr, 0.f, false, inter, x, H, Ti, z, D, nullptr, 0, s));
  if (mxs) {
    // z and h split into FP8 pairs with E8M0 block scales; the MXFP4 weights go to the MFMA as
    // stored (libmir-metal ExpertLayout::Native)
    void *zhl = at<char>(ws, o_zhl), *hhl = at<char>(ws, o_hhl);
    uint16_t *zs = at<uint16_t>(ws, o_zs), *hsc = at<uint16_t>(ws, o_hsc);
    HIPCHK(launch_split_fp8(z, D, Ti, D, zhl, zs, s));
    SegSet gu = segset(aop(zhl, D, ss, K, 0, Ti), b->experts.gate, &b->experts.up, b->experts.swiglu_limit, true);
    gu.A.as = zs;
    gu.A.ldas = D / 32;
    gu.w0.pk = (const char *)b->experts.gate.packed_scaled;
    TRY(run_gemm(inter, b->experts.gate, true, inter, mb, gu, nullptr, 0, 0, tiles, tc, ntile, TK, E, h, ldh, nullptr,
                 0, s, true));
    HIPCHK(launch_split_fp8(h, ldh, TK, I, hhl, hsc, s));
    SegSet dn = segset(aop(hhl, I, nullptr, 1, 0, TK), b->experts.down, nullptr, 0.f, false);
    dn.A.as = hsc;
    dn.A.ldas = I / 32;
    dn.w0.pk = (const char *)b->experts.down.packed_scaled;
    TRY(run_gemm(inter, b->experts.down, false, inter, mb, dn, nullptr, 0, 0, tiles, tc, ntile, TK, E, o, D, nullptr,
                 0, s, true));
  } else {
    SegSet gu = segset(aop(z, D, ss, K, 0, Ti), b->experts.gate, &b->experts.up, b->experts.swiglu_limit, true);
    TRY(run_gemm(inter, b->experts.gate, true, inter, mb, gu, nullptr, 0, 0, tiles, tc, ntile, TK, E, h, ldh, nullptr,
                 0, s));
    SegSet dn = segset(aop(h, ldh, nullptr, 1, 0, TK), b->experts.down, nullptr, 0.f, false);
    TRY(run_gemm(inter, b->experts.down, false, inter, mb, dn, nullptr, 0, 0, tiles, tc, ntile, TK, E, o, D, nullptr,
                 0, s));
  }
  TRY(combine(inter, inter, o, D, sp, wts, K, TK, Ti, D, yn, D, nullptr, b->latent_norm_w, b->norm_eps,
              b->latent_norm_w ? 1 : 0, s));
  const float *resid = nullptr;
  if (has_shared) {
    void *hs = at<char>(ws, o_hs);
    float *sv = at<float>(ws, o_s);
    TRY(run_plain(x_dtype, b->shared.gate, &b->shared.up, b->shared.swiglu_limit, true, inter, x, H, Ti, hs, Is,
                  nullptr, 0, s));
    TRY(run_plain(inter, b->shared.down, nullptr, 0.f, false, MOE_F32, hs, Is, Ti, sv, H, nullptr, 0, s));
    resid = sv;
  }
  TRY(run_plain(inter, b->latent_up, nullptr, 0.f, false, y_dtype, yn, D, Ti, y, H, resid, H, s));
  return MOE_OK;
}

moe_status moe_block_forward_noalloc(const void *x, int32_t x_dtype, int64_t T, const moe_block *b, void *y,
                                     int32_t y_dtype, int32_t *topk_idx, float *topk_w, void *stream) {
  g_err[0] = 0;
  // the workspace this call needs (validates every argument; launches nothing)
  size_t need = 0;
  TRY(moe_block_forward(x, x_dtype, T, b, y, y_dtype, topk_idx, topk_w, nullptr, &need, nullptr));
  CHECK(need <= (size_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
        "moe_block_forward_noalloc: %lld tokens need %zu bytes of scratch, above its fixed %u bytes "
        "(use moe_block_forward with a workspace)", (long long)T, need, (unsigned)MOE_NOALLOC_SCRATCH_BYTES);
  if (T == 0) return MOE_OK;
  CHECK(x && y, MOE_ERR_ARG, "x and y must be non-NULL");
  int dev = -1, sdev = -1;
  HIPCHK(hipGetDevice(&dev));
  HIPCHK(hipStreamGetDevice((hipStream_t)stream, &sdev));
  CHECK(sdev == dev, MOE_ERR_ARG, "the stream belongs to device %d, the calling thread's current device is %d",
        sdev, dev);
  void *ws = nullptr;
  TRY(scratch_on(dev, &ws));
  size_t have = MOE_NOALLOC_SCRATCH_BYTES;
  return moe_block_forward(x, x_dtype, T, b, y, y_dtype, topk_idx, topk_w, ws, &have, stream);
}

}  // extern "C"
