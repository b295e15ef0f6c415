// moe_route.hip - router projection, scoring + top-k, token->expert permutation.
//
// Router and selection follow mlxcel PR #1044 point 3 (sigmoid scores in fp32,
// a per-expert bias added to a copy used only for ranking, weights gathered
// from the unbiased scores, optional renormalisation) and ferrox-models
// latent_moe.rs (route_top_k_sigmoid_with_bias(logits, bias, k, renormalize,
// scaling)).  Softmax scoring is the alternative that page contrasts with.
// Ties in the selection key go to the lower expert id; the K chosen ids of a
// token are written in ascending id order.
#include "moe_topk.h"

// ---------------------------------------------------------------------------
// router logits, bf16 x and W_r: MFMA 16x16x32, 16 tokens x 16 rows per workgroup,
// the reduction split over 8 waves and summed in a fixed order.  Rows 0..E-1 are the
// experts (W_r, + logit_bias); with a blend head, rows E and E+1 are its two rows
// (coef_w, + coef_b), written to clog [T][2].  Every wave issues the loads of up to 8
// of its reduction steps before the first MFMA.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void router_logits_bf16(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ W,
                                                          const float *__restrict__ lbias,
                                                          float *__restrict__ logits, int T, int H, int E,
                                                          const uint16_t *__restrict__ cw,
                                                          const float *__restrict__ cb, float *__restrict__ clog,
                                                          int *__restrict__ zero, int zero_n) {
  if (zero && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < zero_n; i += blockDim.x) zero[i] = 0;
  __shared__ float red[8][16][17];
  router_tile_bf16<false>(x, W, lbias, logits, T, H, E, cw, cb, clog, blockIdx.x, blockIdx.y, red);
}

// router logits for many tokens (bf16): a tiled MFMA GEMM with the reduction split over
// gridDim.z workgroups.  A 256-thread workgroup owns 128 tokens x 64 rows of [W_r; coef head]
// (4 waves of 64 x 32) and one slice of the reduction, in chunks of 64 elements through a
// 3-stage LDS ring filled two chunks ahead by 16-byte direct loads (buffer resources over x,
// W_r and the coef head, fixed per-lane offsets; rows past the matrices read as zero, token
// elements past the slice are zeroed in LDS).  Rows are 16-byte-block XOR-swizzled so that
// fragment reads spread over the banks.  Slice z writes its partial
// sums to logits + z*T*E and clog + z*2T (the bias with slice 0); the selection adds the
// slices in order.
__global__ __launch_bounds__(256) void router_gemm_bf16(const uint16_t *__restrict__ x,
                                                        const uint16_t *__restrict__ W,
                                                        const float *__restrict__ lbias,
                                                        float *__restrict__ logits, int T, int H, int E,
                                                        const uint16_t *__restrict__ cw,
                                                        const float *__restrict__ cb, float *__restrict__ clog,
                                                        int *__restrict__ zero, int zero_n, int ks) {
  if (zero && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < zero_n; i += blockDim.x) zero[i] = 0;
  constexpr int TM = 128, TN = 64, KC = 64;
  // one LDS variable per stage: reads of one stage then do not wait for direct loads into others
  __shared__ __attribute__((aligned(16))) uint16_t sX0[TM * KC], sX1[TM * KC], sX2[TM * KC];
  __shared__ __attribute__((aligned(16))) uint16_t sW0[TN * KC], sW1[TN * KC], sW2[TN * KC];
  uint16_t *const sX[3] = {sX0, sX1, sX2};
  uint16_t *const sW[3] = {sW0, sW1, sW2};
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, kq = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * TM, r0 = blockIdx.y * TN;
  const int R = E + (cw ? 2 : 0);
  const int kb = blockIdx.z * ks, ke = min(H, kb + ks);
  const int nk = (ke - kb + KC - 1) / KC;
  auto swz = [](int row) { return (row >> 1) & 7; };

  // token rows: direct load n (0..3) of wave w covers tile rows 8 (4 w + n) .. + 8, lane l row
  // 8 (4 w + n) + l / 8 and LDS slot l % 8, which holds block (l % 8) ^ swz(row)
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void *)x, (short)0, (int)((int64_t)T * H * 2), 0x00020000);
  uint32_t xo[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int row = 8 * (4 * wave + n) + (lane >> 3);
    xo[n] = (uint32_t)min(t0 + row, T - 1) * (uint32_t)H * 2u + (uint32_t)(((lane & 7) ^ swz(row)) << 4);
  }
  auto load_x = [&](int c, uint16_t *bx) {
#pragma unroll
    for (int n = 0; n < 4; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t *)&bx[(4 * wave + n) * 512], 16, xo[n],
                                               (kb + min(c, nk - 1) * KC) * 2, 0, 0);
  };
  // weight rows: direct load n (0..1) of wave w covers tile rows 8 (2 w + n) .. + 8 (the host
  // keeps E a multiple of 8, so each group comes from W_r or from the coef head only); rows past
  // the matrix read as zero
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc((void *)W, (short)0, (int)((int64_t)E * H * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc((void *)(cw ? cw : W), (short)0, cw ? 2 * H * 2 : 0, 0x00020000);
  uint32_t wo[2];
  bool wcoef[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int g0 = r0 + 8 * (2 * wave + n), row = 8 * (2 * wave + n) + (lane >> 3);
    wcoef[n] = g0 >= E;
    const int rr = r0 + row - (wcoef[n] ? E : 0);
    wo[n] = (uint32_t)rr * (uint32_t)H * 2u + (uint32_t)(((lane & 7) ^ swz(row)) << 4);
  }
  auto load_w = [&](int c, uint16_t *bw) {
    const int so = (kb + min(c, nk - 1) * KC) * 2;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      if (wcoef[n])
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, (lds_void_t *)&bw[(2 * wave + n) * 512], 16, wo[n], so, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void_t *)&bw[(2 * wave + n) * 512], 16, wo[n], so, 0, 0);
    }
  };

  f32x4_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int sw = (n16 >> 1) & 7;
  auto compute = [&](const uint16_t *bx, const uint16_t *bw) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int slot = ((4 * st + kq) ^ sw) << 3;
      u32x4_t af[4], bf[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) af[mb] = *(const u32x4_t *)&bx[(wm * 64 + 16 * mb + n16) * KC + slot];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bf[nb] = *(const u32x4_t *)&bw[(wn * 32 + 16 * nb + n16) * KC + slot];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[mb]),
                                                               __builtin_bit_cast(bf16x8_t, bf[nb]), acc[mb][nb], 0, 0,
                                                               0);
    }
  };
  // elements past the slice in the last chunk: the token blocks read there belong to the next
  // row (or past x); each wave zeroes those of its own direct loads, once they have landed
  auto zero_tail = [&](int c, uint16_t *bx) {
    const int kn = ke - (kb + c * KC);
    if (kn >= KC) return;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int row = 8 * (4 * wave + n) + (lane >> 3), slot = lane & 7, blk = slot ^ swz(row);
      if (blk * 8 >= kn) *(u32x4_t *)&bx[row * KC + (slot << 3)] = u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  load_x(0, sX[0]);
  load_w(0, sW[0]);
  load_x(1, sX[1]);
  load_w(1, sW[1]);
  // chunk c in buffer j = c % 3: loads of chunk c + 2 (clamped past the end) issued, chunk c
  // computed.  Whole groups of three chunks run branch-free (compile-time buffers), then the
  // remainder.
  auto chunk = [&](int c, int j) {
    load_x(c + 2, sX[(j + 2) % 3]);
    load_w(c + 2, sW[(j + 2) % 3]);
    wait_vmcnt<12>();  // chunk c has landed (the 6 loads of each of the two later chunks may not)
    if (c == nk - 1) zero_tail(c, sX[j]);
    stage_barrier();
    compute(sX[j], sW[j]);
    stage_barrier();  // every wave is done with chunk c before its buffer is loaded again
  };
  int c = 0;
  for (; c + 3 <= nk; c += 3) {
    chunk(c, 0);
    chunk(c + 1, 1);
    chunk(c + 2, 2);
  }
  if (c < nk) chunk(c, 0);
  if (c + 1 < nk) chunk(c + 1, 1);
  wait_vmcnt<0>();  // the loads past the end

  // acc[mb][nb][i]: token 64 wm + 16 mb + 4 kq + i, row 32 wn + 16 nb + n16
  float *lg = logits + (int64_t)blockIdx.z * T * E;
  float *cl = clog ? clog + (int64_t)blockIdx.z * 2 * T : nullptr;
  const bool first = blockIdx.z == 0;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int e = r0 + wn * 32 + 16 * nb + n16;
    const float add = !first ? 0.f : (e < E ? (lbias ? lbias[e] : 0.f) : (e < R ? cb[e - E] : 0.f));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + wm * 64 + 16 * mb + 4 * kq + i;
        if (t < T) {
          if (e < E)
            lg[(int64_t)t * E + e] = acc[mb][nb][i] + add;
          else if (e < R)
            cl[2 * t + (e - E)] = acc[mb][nb][i] + add;
        }
      }
  }
}

// router logits, f32 x and W_r: one thread per (token, row), sequential fp32 sum; rows as above.
__global__ void router_logits_f32(const float *__restrict__ x, const float *__restrict__ W,
                                  const float *__restrict__ lbias, float *__restrict__ logits, int T, int H,
                                  int E, const float *__restrict__ cw, const float *__restrict__ cb,
                                  float *__restrict__ clog, int *__restrict__ zero, int zero_n) {
  if (zero && blockIdx.x == 0)
    for (int i = threadIdx.x; i < zero_n; i += blockDim.x) zero[i] = 0;
  const int R = E + (cw ? 2 : 0);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * R) return;
  const int t = (int)(i / R), e = (int)(i % R);
  const float *xr = x + (int64_t)t * H, *wr = e < E ? W + (int64_t)e * H : cw + (int64_t)(e - E) * H;
  float v = 0.f;
  for (int h = 0; h < H; ++h) v = fmaf(xr[h], wr[h], v);
  if (e < E)
    logits[(int64_t)t * E + e] = v + (lbias ? lbias[e] : 0.f);
  else
    clog[2 * t + (e - E)] = v + cb[e - E];
}

// ---------------------------------------------------------------------------
// scores + top-k + weights (+ the blend coefficients): one wave per token.
// The selection key of expert e is (score + select_bias) mapped to an order-preserving
// u32 in the high word and ~e in the low word, so the largest key is the largest
// selection value with ties to the lower id.  Each of the K rounds takes the wave-wide
// maximum key (DPP within rows of 16 lanes, then the four row maxima) and retires it.
// ---------------------------------------------------------------------------

// one wave per token (K > 16)
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ float sl[4][MOE_MAX_EXPERTS];
  __shared__ int el[4][MOE_MAX_TOPK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.T) return;  // wave-uniform
  topk_token(a, t, lane, sl[wave], el[wave], nullptr);
}

// one half-wave per token (K <= 16), 8 tokens per workgroup
template <int SL>
__global__ __launch_bounds__(256) void topk_half_kernel(TopkArgs a) {
  __shared__ __attribute__((aligned(16))) int el[8][16];
  __shared__ float esc[8][16];
  const int lane = threadIdx.x & 63, half = threadIdx.x >> 5;
  topk_half<SL>(a, blockIdx.x * 8 + half, lane & 31, el[half], esc[half], nullptr);
}
template __global__ void topk_half_kernel<4>(TopkArgs);
template __global__ void topk_half_kernel<8>(TopkArgs);
template __global__ void topk_half_kernel<16>(TopkArgs);

// ---------------------------------------------------------------------------
// permutation: per-chunk expert histograms, a scan in expert-major order, and a
// deterministic scatter (rank inside a chunk from per-expert token bitmasks).
// ---------------------------------------------------------------------------

// exclusive scan of v[0..n) in place (shared memory, n <= 4*blockDim, blockDim a multiple
// of 64); returns the total.  Each thread owns consecutive elements; waves scan with
// shuffles and combine their totals through tmp (>= blockDim/64 ints).
static __device__ int block_exclusive_scan(int *v, int n, int *tmp) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
  const int per = (n + nt - 1) / nt;
  const int b = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < n) local += v[b + i];
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < nw; ++w) {
    const int c = tmp[w];
    base += (w < wave) ? c : 0;
    total += c;
  }
  int run = base + incl - local;
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      const int c = v[b + i];
      v[b + i] = run;
      run += c;
    }
  __syncthreads();
  return total;
}

// ids j0 .. j0+7 of token t, all loads in flight together (entries past K repeat id K-1
// and are never used)
constexpr int kIdBatch = 8;
static __device__ void load_ids(const int32_t *__restrict__ idx, int t, int K, int j0, int (&ids)[kIdBatch]) {
#pragma unroll
  for (int j = 0; j < kIdBatch; ++j) ids[j] = idx[(int64_t)t * K + min(j0 + j, K - 1)];
}

// m-tile list for the grouped expert GEMMs: every routed segment (expert e's slots, sorted
// rows offsets[e]..offsets[e+1]) cut into tiles of at most mt rows (mt <= 128).  A segment of
// n rows becomes t = ceil(n / mt) tiles: t - 1 of q rows, q = ceil(n / t) rounded up to whole
// 16-row blocks and capped at mt, and a last one with the rest (1..q rows), so that the
// fewest tiles hold ceil(n / 16) blocks in all.  The list is ordered by tile size, the most
// 16-row blocks first: the GEMMs deal units to workgroups round-robin, so every workgroup
// then gets a similar mix of large and small tiles.  Within one size the order is that of
// arrival at a shared counter (a segment's tiles of one size stay together); every tile's
// results are independent of its position.  offs: shared copy of offsets[0..E]; cls: 16
// shared ints.
static __device__ void emit_tiles(const int *offs, int E, int mt, int4 *tiles, int *tile_count, int *cls) {
  const int tid = threadIdx.x;
  int *tot = cls, *cur = cls + 8;  // tiles per size class (blocks - 1), then placement cursors
  auto shape = [&](int e, int &n, int &t, int &q, int &cq, int &cl) {
    n = offs[e + 1] - offs[e];
    t = (n + mt - 1) / mt;
    q = t ? min(mt, (((n + t - 1) / t) + 15) & ~15) : 16;
    cq = q / 16 - 1;                              // size class of the first t - 1 tiles
    cl = t ? (n - (t - 1) * q + 15) / 16 - 1 : 0;  // ... and of the last
  };
  if (tid < 16) cls[tid] = 0;
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    int n, t, q, cq, cl;
    shape(e, n, t, q, cq, cl);
    if (n == 0) continue;
    if (t > 1) atomicAdd(&tot[cq], t - 1);
    atomicAdd(&tot[cl], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int R = 0;
    for (int b = 7; b >= 0; --b) {
      cur[b] = R;
      R += tot[b];
    }
    tile_count[0] = R;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    int n, t, q, cq, cl;
    shape(e, n, t, q, cq, cl);
    if (n == 0) continue;
    if (t > 1) {
      const int pq = atomicAdd(&cur[cq], t - 1);
      for (int i = 0; i < t - 1; ++i) tiles[pq + i] = make_int4(e, offs[e] + i * q, q, 0);
    }
    tiles[atomicAdd(&cur[cl], 1)] = make_int4(e, offs[e] + (t - 1) * q, n - (t - 1) * q, 0);
  }
}

__global__ __launch_bounds__(256) void perm_count(const int32_t *__restrict__ idx, int T, int K, int E,
                                                  int32_t *__restrict__ chunk_counts) {
  __shared__ int cnt[MOE_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < T) {
    for (int j0 = 0; j0 < K; j0 += kIdBatch) {
      int ids[kIdBatch];
      load_ids(idx, t, K, j0, ids);
#pragma unroll
      for (int j = 0; j < kIdBatch; ++j)
        if (j0 + j < K) atomicAdd(&cnt[ids[j]], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// single workgroup: per-expert totals, offsets, per-(chunk, expert) bases, tiles.
__global__ __launch_bounds__(1024) void perm_scan(int32_t *__restrict__ chunk_counts, int nchunks, int E, int TK,
                                                  int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                  int4 *tiles, int *tile_count, int mt) {
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ int cls[16];
  __shared__ int tmp[16];
  // the chunk counts of expert e, eight independent loads per trip (clamped, masked)
  constexpr int B = 8;
  auto chunk_batch = [&](int e, int c0, int (&v)[B]) {
#pragma unroll
    for (int j = 0; j < B; ++j) v[j] = chunk_counts[(int64_t)min(c0 + j, nchunks - 1) * E + e];
#pragma unroll
    for (int j = 0; j < B; ++j) v[j] = c0 + j < nchunks ? v[j] : 0;
  };
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += B) {
      int v[B];
      chunk_batch(e, c0, v);
#pragma unroll
      for (int j = 0; j < B; ++j) run += v[j];
    }
    offs[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(offs, E, tmp);
  if (threadIdx.x == 0) offs[E] = total;
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = offs[e];
  // chunk c's base for expert e: offsets[e] + the counts of e in chunks 0 .. c - 1
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = offs[e];
    for (int c0 = 0; c0 < nchunks; c0 += B) {
      int v[B];
      chunk_batch(e, c0, v);
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (c0 + j < nchunks) chunk_counts[(int64_t)(c0 + j) * E + e] = run;
        run += v[j];
      }
    }
  }
  if (tiles) {
    __syncthreads();
    emit_tiles(offs, E, mt, tiles, tile_count, cls);
  }
}

// each slot of the chunk's tokens (mask: bit t of word t / 32 of its expert's row set for every
// token t of the chunk that chose that expert) placed at base[e] + its rank among them
static __device__ void chunk_scatter(const int32_t *__restrict__ idx, int T, int K, int chunk, const int *base,
                                     const uint32_t (*mask)[8], int32_t *__restrict__ sorted_slot,
                                     int32_t *__restrict__ slot_pos) {
  const int tid = threadIdx.x;
  const int t = chunk * 256 + tid;
  if (t >= T) return;
  const int wd = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
  for (int j0 = 0; j0 < K; j0 += kIdBatch) {
    int ids[kIdBatch];
    load_ids(idx, t, K, j0, ids);
#pragma unroll
    for (int j = 0; j < kIdBatch; ++j) {
      if (j0 + j < K) {
        const int e = ids[j];
        int rank = __popc(mask[e][wd] & below);
        for (int w = 0; w < wd; ++w) rank += __popc(mask[e][w]);
        const int pos = base[e] + rank;
        const int p = t * K + j0 + j;
        sorted_slot[pos] = p;
        slot_pos[p] = pos;
      }
    }
  }
}

// rank of each (token, slot) among the chunk's tokens that chose the same expert
static __device__ void scatter_chunk(const int32_t *__restrict__ idx, int T, int K, int E, int chunk,
                                     const int *base /* [E], absolute position of the chunk's first slot of e */,
                                     uint32_t (*mask)[8], int32_t *__restrict__ sorted_slot,
                                     int32_t *__restrict__ slot_pos) {
  const int tid = threadIdx.x;
  const int t = chunk * 256 + tid;
  for (int i = tid; i < E * 8; i += blockDim.x) mask[i >> 3][i & 7] = 0u;
  __syncthreads();
  if (t < T) {
    for (int j0 = 0; j0 < K; j0 += kIdBatch) {
      int ids[kIdBatch];
      load_ids(idx, t, K, j0, ids);
#pragma unroll
      for (int j = 0; j < kIdBatch; ++j)
        if (j0 + j < K) atomicOr(&mask[ids[j]][tid >> 5], 1u << (tid & 31));
    }
  }
  __syncthreads();
  chunk_scatter(idx, T, K, chunk, base, mask, sorted_slot, slot_pos);
}

__global__ __launch_bounds__(256) void perm_scatter(const int32_t *__restrict__ idx, int T, int K, int E,
                                                    const int32_t *__restrict__ chunk_base,
                                                    int32_t *__restrict__ sorted_slot,
                                                    int32_t *__restrict__ slot_pos) {
  __shared__ uint32_t mask[MOE_MAX_EXPERTS][8];
  __shared__ int base[MOE_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += 256) base[e] = chunk_base[(int64_t)blockIdx.x * E + e];
  scatter_chunk(idx, T, K, E, blockIdx.x, base, mask, sorted_slot, slot_pos);
}

// More than 256 tokens, at most kPermFusedChunks chunks of 256: count, scan and scatter in one
// launch of a workgroup per chunk (all resident at once).  Each counts its slots per expert
// and keeps the per-expert token masks in LDS, stores its counts at device scope, waits until
// its stores have completed and counts itself on *done (zero when the launch starts); once
// every chunk is in, each reads all the counts (device scope), sums them per expert, scans
// the totals into the offsets, adds the counts of the chunks before its own, and places its
// slots; workgroup 0 also writes counts, offsets and the m-tile list.  The same arithmetic and
// the same positions as perm_count + perm_scan + perm_scatter.  The wait is bounded: if it
// gives up (only possible when the chunks are not all resident) *status is set.
__global__ __launch_bounds__(256) void perm_fused(const int32_t *__restrict__ idx, int T, int K, int E,
                                                  int32_t *__restrict__ chunk_counts, int32_t *__restrict__ counts,
                                                  int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
                                                  int32_t *__restrict__ slot_pos, int4 *tiles, int *tile_count,
                                                  int mt, int *done, int *status) {
  __shared__ uint32_t mask[MOE_MAX_EXPERTS][8];
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ int base[MOE_MAX_EXPERTS];
  __shared__ int tmp[16];
  __shared__ int cls[16];
  const int tid = threadIdx.x, c = blockIdx.x, nch = gridDim.x;
  const int t = c * 256 + tid;
  for (int i = tid; i < E * 8; i += 256) mask[i >> 3][i & 7] = 0u;
  for (int e = tid; e < E; e += 256) offs[e] = 0;
  __syncthreads();
  constexpr int KC = 2 * kIdBatch;  // ids kept in registers for the scatter (top_k <= 16)
  int idc[KC];
  if (t < T) {
    for (int j0 = 0; j0 < K; j0 += kIdBatch) {
      int ids[kIdBatch];
      load_ids(idx, t, K, j0, ids);
#pragma unroll
      for (int j = 0; j < kIdBatch; ++j) {
        if (j0 + j < K) {
          atomicAdd(&offs[ids[j]], 1);
          atomicOr(&mask[ids[j]][tid >> 5], 1u << (tid & 31));
        }
        if (j0 == 0) idc[j] = ids[j];
        if (j0 == kIdBatch) idc[kIdBatch + j] = ids[j];
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256)
    __hip_atomic_store(chunk_counts + (int64_t)c * E + e, offs[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  wait_vmcnt<0>();  // this thread's count stores have completed
  __syncthreads();
  if (tid == 0) {
    __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int it = 0;
    for (; it < (1 << 19); ++it) {
      if (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= nch) break;
      __builtin_amdgcn_s_sleep(4);
    }
    if (it == (1 << 19)) __hip_atomic_store(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  // per expert: the total over every chunk and the part of the chunks before this one
  constexpr int B = 16;
  for (int e = tid; e < E; e += 256) {
    int run = 0, pre = 0;
    for (int c0 = 0; c0 < nch; c0 += B) {
      int v[B];
#pragma unroll
      for (int j = 0; j < B; ++j)
        v[j] = __hip_atomic_load(chunk_counts + (int64_t)min(c0 + j, nch - 1) * E + e, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (c0 + j == c) pre = run;
        run += c0 + j < nch ? v[j] : 0;
      }
    }
    offs[e] = run;
    base[e] = pre;
  }
  __syncthreads();
  const int total = block_exclusive_scan(offs, E, tmp);
  if (tid == 0) offs[E] = total;
  __syncthreads();
  for (int e = tid; e < E; e += 256) base[e] += offs[e];
  if (c == 0) {
    for (int e = tid; e <= E; e += 256) {
      offsets[e] = offs[e];
      if (e < E) counts[e] = offs[e + 1] - offs[e];
    }
    if (tiles) emit_tiles(offs, E, mt, tiles, tile_count, cls);
  }
  __syncthreads();
  if (K > KC) {
    chunk_scatter(idx, T, K, c, base, mask, sorted_slot, slot_pos);
    return;
  }
  if (t >= T) return;
  const int wd = tid >> 5;
  const uint32_t below = (1u << (tid & 31)) - 1u;
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    if (j < K) {
      const int e = idc[j];
      int rank = __popc(mask[e][wd] & below);
      for (int w = 0; w < wd; ++w) rank += __popc(mask[e][w]);
      const int pos = base[e] + rank;
      const int p = t * K + j;
      sorted_slot[pos] = p;
      slot_pos[p] = pos;
    }
  }
}

// T <= 256: the whole permutation (and the tile list) in one workgroup (blockDim >= 256).
// idx may point to global or shared memory.
struct PermSmem {
  uint32_t mask[MOE_MAX_EXPERTS][8];
  int offs[MOE_MAX_EXPERTS + 1];
  int cls[16];
  int tmp[16];
};

static __device__ void perm_block(const int32_t *idx, int T, int K, int E, int32_t *__restrict__ counts,
                                  int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
                                  int32_t *__restrict__ slot_pos, int4 *tiles, int *tile_count, int mt,
                                  PermSmem &sm) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) sm.offs[e] = 0;
  __syncthreads();
  if (tid < T) {
    for (int j0 = 0; j0 < K; j0 += kIdBatch) {
      int ids[kIdBatch];
      load_ids(idx, tid, K, j0, ids);
#pragma unroll
      for (int j = 0; j < kIdBatch; ++j)
        if (j0 + j < K) atomicAdd(&sm.offs[ids[j]], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) counts[e] = sm.offs[e];
  __syncthreads();
  const int total = block_exclusive_scan(sm.offs, E, sm.tmp);
  if (tid == 0) sm.offs[E] = total;
  __syncthreads();
  for (int e = tid; e <= E; e += blockDim.x) offsets[e] = sm.offs[e];
  scatter_chunk(idx, T, K, E, 0, sm.offs, sm.mask, sorted_slot, slot_pos);
  if (tiles) {
    __syncthreads();
    emit_tiles(sm.offs, E, mt, tiles, tile_count, sm.cls);
  }
}

__global__ __launch_bounds__(256) void perm_small(const int32_t *__restrict__ idx, int T, int K, int E,
                                                  int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                  int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_pos,
                                                  int4 *tiles, int *tile_count, int mt) {
  __shared__ PermSmem sm;
  perm_block(idx, T, K, E, counts, offsets, sorted_slot, slot_pos, tiles, tile_count, mt, sm);
}

// T <= MOE_ROUTE_SMALL_T, K <= 16: selection and permutation in one launch.  Each 256-thread
// workgroup selects for 8 tokens (one half-wave each), so that the selection, which is bound
// by dependent cross-lane steps, runs on several CUs; the last workgroup to finish (a counter
// that the router launch set to zero) builds the permutation and the tile list from the
// stored selections: per-expert counts and token masks, one scan over the experts of the
// packed (slot count, tile count) pairs (T*K <= 1024), then each slot's rank among the earlier
// tokens of its expert.
template <int SL>
__global__ __launch_bounds__(256) void route_decode(TopkArgs a, int32_t *__restrict__ counts,
                                                   int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_slot,
                                                   int32_t *__restrict__ slot_pos, int4 *tiles, int *tile_count,
                                                   int mt, int *done) {
  __shared__ __attribute__((aligned(16))) int el[8][16];
  __shared__ float esc[8][16];
  __shared__ DecodePermSmem<256> sm;
  __shared__ int last;
  const int tid = threadIdx.x, half = tid >> 5;
  // hand-over without cache maintenance: the ids are device-scope stores, complete (vmcnt 0)
  // before the workgroup is counted; the last workgroup reads them with device-scope loads
  topk_half<SL>(a, blockIdx.x * 8 + half, tid & 31, el[half], esc[half], nullptr, true);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): this thread's stores have completed
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  decode_permute<256, false>(a.idx, a.T, a.K, a.E, counts, offsets, sorted_slot, slot_pos, tiles, tile_count, mt, sm);
  if (tid == 0) *done = 0;
}
template __global__ void route_decode<4>(TopkArgs, int32_t *, int32_t *, int32_t *, int32_t *, int4 *, int *, int,
                                         int *);
template __global__ void route_decode<8>(TopkArgs, int32_t *, int32_t *, int32_t *, int32_t *, int4 *, int *, int,
                                         int *);
template __global__ void route_decode<16>(TopkArgs, int32_t *, int32_t *, int32_t *, int32_t *, int4 *, int *, int,
                                          int *);

// tile list from caller-provided offsets (moe_experts_forward)
__global__ __launch_bounds__(256) void build_tiles(const int32_t *__restrict__ offsets, int E, int4 *tiles,
                                                   int *tile_count, int mt) {
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ int cls[16];
  for (int e = threadIdx.x; e <= E; e += 256) offs[e] = offsets[e];
  __syncthreads();
  emit_tiles(offs, E, mt, tiles, tile_count, cls);
}
