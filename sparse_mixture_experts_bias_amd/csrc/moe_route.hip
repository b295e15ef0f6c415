// moe_route.hip - router projection, scoring + top-k, token->expert permutation.
//
// Router and selection follow mlxcel PR #1044 point 3 (sigmoid scores in fp32,
// a per-expert bias added to a copy used only for ranking, weights gathered
// from the unbiased scores, optional renormalisation) and ferrox-models
// latent_moe.rs (route_top_k_sigmoid_with_bias(logits, bias, k, renormalize,
// scaling)).  Softmax scoring is the alternative that page contrasts with.
// Ties in the selection key go to the lower expert id; the K chosen ids of a
// token are written in ascending id order.
#include "moe_kernels.h"

// ---------------------------------------------------------------------------
// router logits, bf16 x and W_r: MFMA 16x16x32, 16 tokens x 16 experts per
// workgroup, the reduction split over 8 waves and summed in a fixed order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void router_logits_bf16(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ W,
                                                          const float *__restrict__ lbias,
                                                          float *__restrict__ logits, int T, int H, int E) {
  __shared__ float red[8][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16;
  const int r = lane & 15, kb = lane >> 4;
  const int trow = min(t0 + r, T - 1), erow = min(e0 + r, E - 1);
  const u32x4_t *xa = (const u32x4_t *)(x + (int64_t)trow * H + kb * 8);
  const u32x4_t *wb = (const u32x4_t *)(W + (int64_t)erow * H + kb * 8);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = H >> 5;
  int s = wave;
  for (; s + 8 < nsteps; s += 16) {
    u32x4_t a0 = xa[s * 4], b0 = wb[s * 4];
    u32x4_t a1 = xa[(s + 8) * 4], b1 = wb[(s + 8) * 4];
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                  __builtin_bit_cast(bf16x8_t, b0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                  __builtin_bit_cast(bf16x8_t, b1), acc, 0, 0, 0);
  }
  for (; s < nsteps; s += 8) {
    u32x4_t a0 = xa[s * 4], b0 = wb[s * 4];
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                  __builtin_bit_cast(bf16x8_t, b0), acc, 0, 0, 0);
  }
  // acc[i] holds row (token) 4*kb+i, column (expert) r of the 16x16 tile
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * kb + i][r] = acc[i];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, n = threadIdx.x & 15;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) v += red[w][m][n];
    const int t = t0 + m, e = e0 + n;
    if (t < T && e < E) logits[(int64_t)t * E + e] = v + (lbias ? lbias[e] : 0.f);
  }
}

// router logits, f32 x and W_r: one thread per (token, expert), sequential fp32 sum.
__global__ void router_logits_f32(const float *__restrict__ x, const float *__restrict__ W,
                                  const float *__restrict__ lbias, float *__restrict__ logits, int T, int H,
                                  int E) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float *xr = x + (int64_t)t * H, *wr = W + (int64_t)e * H;
  float v = 0.f;
  for (int h = 0; h < H; ++h) v = fmaf(xr[h], wr[h], v);
  logits[i] = v + (lbias ? lbias[e] : 0.f);
}

// ---------------------------------------------------------------------------
// scores + top-k + weights (+ the blend coefficient head): one wave per token.
// ---------------------------------------------------------------------------
template <int XDT>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  constexpr int EPL = MOE_MAX_EXPERTS / 64;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const float *lrow = a.logits + (int64_t)t * a.E;
  float s[EPL], sel[EPL];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    s[j] = (e < a.E) ? lrow[e] : -INFINITY;
    mx = fmaxf(mx, s[j]);
  }
  if (a.scoring == 1) {  // softmax over experts, max-subtracted, fp32
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
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    sel[j] = s[j] + ((a.sbias && e < a.E) ? a.sbias[e] : 0.f);
  }
  uint32_t taken = 0;
  int my_e = 0x7fffffff;
  float my_s = 0.f;
  for (int k = 0; k < a.K; ++k) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
    float bs = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      const bool ok = (e < a.E) && !((taken >> j) & 1u);
      if (ok && (be == 0x7fffffff || sel[j] > bv || (sel[j] == bv && e < be))) {
        bv = sel[j];
        be = e;
        bs = s[j];
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      const float os = __shfl_xor(bs, o, 64);
      const bool take = (oe != 0x7fffffff) &&
                        (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (take) {
        bv = ov;
        be = oe;
        bs = os;
      }
    }
    if (lane == k) {
      my_e = be;
      my_s = bs;
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
  }
  // ascending-id order and the weight sum (over the K chosen, fixed order)
  int rank = 0;
  float wsum = 0.f;
  for (int i = 0; i < a.K; ++i) {
    const int ei = __shfl(my_e, i, 64);
    wsum += __shfl(my_s, i, 64);
    rank += (ei < my_e) ? 1 : 0;
  }
  if (lane < a.K) {
    float w = a.norm ? my_s / wsum : my_s;
    w *= a.rscale;
    a.idx[(int64_t)t * a.K + rank] = my_e;
    a.w[(int64_t)t * a.K + rank] = w;
  }
  // blend coefficients: softmax over the 2-way head, fp32
  if (a.coef_w) {
    float c0 = 0.f, c1 = 0.f;
    if constexpr (XDT == DT_F32) {
      const float *xr = (const float *)a.x + (int64_t)t * a.H;
      const float *w0 = (const float *)a.coef_w, *w1 = w0 + a.H;
      for (int h = lane; h < a.H; h += 64) {
        c0 = fmaf(xr[h], w0[h], c0);
        c1 = fmaf(xr[h], w1[h], c1);
      }
    } else {
      const uint16_t *xr = (const uint16_t *)a.x + (int64_t)t * a.H;
      const uint16_t *w0 = (const uint16_t *)a.coef_w, *w1 = w0 + a.H;
      for (int h = lane * 8; h < a.H; h += 512) {
        float xf[8], af[8], bf[8];
        unpack8<DT_BF16>(*(const u32x4_t *)(xr + h), xf);
        unpack8<DT_BF16>(*(const u32x4_t *)(w0 + h), af);
        unpack8<DT_BF16>(*(const u32x4_t *)(w1 + h), bf);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          c0 = fmaf(xf[q], af[q], c0);
          c1 = fmaf(xf[q], bf[q], c1);
        }
      }
    }
    c0 = wave_sum(c0) + a.coef_b[0];
    c1 = wave_sum(c1) + a.coef_b[1];
    const float m = fmaxf(c0, c1);
    const float x0 = expf(c0 - m), x1 = expf(c1 - m);
    if (lane == 0) {
      a.coef[2 * t] = x0 / (x0 + x1);
      a.coef[2 * t + 1] = x1 / (x0 + x1);
    }
  }
}

template __global__ void topk_kernel<DT_F32>(TopkArgs);
template __global__ void topk_kernel<DT_BF16>(TopkArgs);

// ---------------------------------------------------------------------------
// permutation: per-chunk expert histograms, a scan in expert-major order, and a
// deterministic scatter (rank inside a chunk from per-expert token bitmasks).
// ---------------------------------------------------------------------------

// exclusive scan of v[0..n) in place (shared memory, n <= 4*blockDim); returns the total.
static __device__ int block_exclusive_scan(int *v, int n, int *tmp /* >= blockDim ints */) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int b = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (b + i < n) local += v[b + i];
  tmp[tid] = local;
  __syncthreads();
  for (int off = 1; off < nt; off <<= 1) {
    const int add = (tid >= off) ? tmp[tid - off] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  const int total = tmp[nt - 1];
  int run = tmp[tid] - local;
  __syncthreads();
  for (int i = 0; i < per; ++i)
    if (b + i < n) {
      const int c = v[b + i];
      v[b + i] = run;
      run += c;
    }
  __syncthreads();
  return total;
}

// m-tile list for the grouped expert GEMMs: every routed segment (expert e's slots,
// sorted rows offsets[e]..offsets[e+1]) cut into tiles of mt rows, in expert order.
// offs: shared-memory copy of offsets[0..E].
static __device__ void emit_tiles(const int *offs, int E, int mt, int4 *tiles, int *tile_count,
                                  int *nmc /* shared, E ints */, int *tmp) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) nmc[e] = (offs[e + 1] - offs[e] + mt - 1) / mt;
  __syncthreads();
  const int R = block_exclusive_scan(nmc, E, tmp);
  for (int e = tid; e < E; e += blockDim.x) {
    const int n = offs[e + 1] - offs[e];
    for (int i = 0, base = nmc[e]; i * mt < n; ++i)
      tiles[base + i] = make_int4(e, offs[e] + i * mt, min(mt, n - i * mt), 0);
  }
  if (tid == 0) tile_count[0] = R;
}

__global__ __launch_bounds__(256) void perm_count(const int32_t *__restrict__ idx, int T, int K, int E,
                                                  int32_t *__restrict__ chunk_counts) {
  __shared__ int cnt[MOE_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < T)
    for (int j = 0; j < K; ++j) atomicAdd(&cnt[idx[(int64_t)t * K + j]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// single workgroup: per-expert totals, offsets, per-(chunk, expert) bases, tiles.
__global__ __launch_bounds__(1024) void perm_scan(int32_t *__restrict__ chunk_counts, int nchunks, int E, int TK,
                                                  int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                  int4 *tiles, int *tile_count, int mt) {
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ int nmc[MOE_MAX_EXPERTS];
  __shared__ int tmp[1024];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int run = 0;
    for (int c = 0; c < nchunks; ++c) {
      const int v = chunk_counts[(int64_t)c * E + e];
      chunk_counts[(int64_t)c * E + e] = run;
      run += v;
    }
    offs[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan(offs, E, tmp);
  if (threadIdx.x == 0) offs[E] = total;
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = offs[e];
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    for (int c = 0; c < nchunks; ++c) chunk_counts[(int64_t)c * E + e] += offs[e];
  if (tiles) {
    __syncthreads();
    emit_tiles(offs, E, mt, tiles, tile_count, nmc, tmp);
  }
}

// rank of each (token, slot) among the chunk's tokens that chose the same expert
static __device__ void scatter_chunk(const int32_t *__restrict__ idx, int T, int K, int E, int chunk,
                                     const int *base /* [E], absolute position of the chunk's first slot of e */,
                                     uint32_t (*mask)[8], int32_t *__restrict__ sorted_slot,
                                     int32_t *__restrict__ slot_pos) {
  const int tid = threadIdx.x;
  for (int i = tid; i < E * 8; i += blockDim.x) mask[i >> 3][i & 7] = 0u;
  __syncthreads();
  const int t = chunk * 256 + tid;
  if (t < T)
    for (int j = 0; j < K; ++j) atomicOr(&mask[idx[(int64_t)t * K + j]][tid >> 5], 1u << (tid & 31));
  __syncthreads();
  if (t < T) {
    const int wd = tid >> 5;
    const uint32_t below = (1u << (tid & 31)) - 1u;
    for (int j = 0; j < K; ++j) {
      const int e = idx[(int64_t)t * K + j];
      int rank = __popc(mask[e][wd] & below);
      for (int w = 0; w < wd; ++w) rank += __popc(mask[e][w]);
      const int pos = base[e] + rank;
      const int p = t * K + j;
      sorted_slot[pos] = p;
      slot_pos[p] = pos;
    }
  }
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

// T <= 256: the whole permutation (and the tile list) in one workgroup.
__global__ __launch_bounds__(256) void perm_small(const int32_t *__restrict__ idx, int T, int K, int E,
                                                  int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                  int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_pos,
                                                  int4 *tiles, int *tile_count, int mt) {
  __shared__ uint32_t mask[MOE_MAX_EXPERTS][8];
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ int nmc[MOE_MAX_EXPERTS];
  __shared__ int tmp[256];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) offs[e] = 0;
  __syncthreads();
  if (tid < T)
    for (int j = 0; j < K; ++j) atomicAdd(&offs[idx[(int64_t)tid * K + j]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) counts[e] = offs[e];
  __syncthreads();
  const int total = block_exclusive_scan(offs, E, tmp);
  if (tid == 0) offs[E] = total;
  __syncthreads();
  for (int e = tid; e <= E; e += 256) offsets[e] = offs[e];
  scatter_chunk(idx, T, K, E, 0, offs, mask, sorted_slot, slot_pos);
  if (tiles) {
    __syncthreads();
    emit_tiles(offs, E, mt, tiles, tile_count, nmc, tmp);
  }
}

// tile list from caller-provided offsets (moe_experts_forward)
__global__ __launch_bounds__(256) void build_tiles(const int32_t *__restrict__ offsets, int E, int4 *tiles,
                                                   int *tile_count, int mt) {
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ int nmc[MOE_MAX_EXPERTS];
  __shared__ int tmp[256];
  for (int e = threadIdx.x; e <= E; e += 256) offs[e] = offsets[e];
  __syncthreads();
  emit_tiles(offs, E, mt, tiles, tile_count, nmc, tmp);
}
