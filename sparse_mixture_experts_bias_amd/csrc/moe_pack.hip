// moe_pack.hip - the packed weight stream of the grouped GEMM (layout in moe_kernels.h).
//
// A pure permutation of the natural layout (mlxcel issue #974's SwitchLinear::Quantized
// words, scales and biases; libmir-metal ExpertLayout blocks/scales): every output word is
// gathered from one source word (scales: one scale and one qbias, or four E8M0 bytes), and
// positions past the matrix's rows or columns are zero.  Weight and group parameters are
// never converted, so a GEMM over the packed stream sees exactly the stored values.
#include "moe_kernels.h"

// AFFINE4 word of 8 codes (element j in bits 4j..4j+3) -> even elements in the low
// half-word, odd ones in the high half-word (element 2j at bits 4j, element 2j+1 at bits
// 16+4j), so that (w >> 4j) & 0x000F000F is the adjacent pair (2j, 2j+1)
static __device__ uint32_t pair_order(uint32_t v) {
  uint32_t r = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r |= ((v >> (8 * j)) & 0xFu) << (4 * j);
    r |= ((v >> (8 * j + 4)) & 0xFu) << (16 + 4 * j);
  }
  return r;
}

__global__ __launch_bounds__(256) void pack_kernel(const PackArgs a) {
  const int kc_len = pk_kc(a.wf), ue = pk_ue(a.wf, a.gq), qe = ue / 4, lpu = pk_lb(a.wf, a.gq) / 4;
  const int nu = pk_nu(a.wf, a.gq), rw = pk_record_bytes(a.wf, a.gq) / 4;
  const int64_t total = (int64_t)a.n * a.nblk * a.nch * rw;
  const int wpr = a.wf == WF_DENSE ? a.cols / 2 : a.cols / 8;  // 32-bit words per natural row
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int o = (int)(idx % rw);
    int64_t rest = idx / rw;
    const int c = (int)(rest % a.nch);
    rest /= a.nch;
    const int b = (int)(rest % a.nblk);
    const int m = (int)(rest / a.nblk);
    const int kc = c * kc_len;
    // tile row (half h, lane row n16) -> (source stack, matrix row)
    auto src_row = [&](int h, int n16, bool &upper) {
      upper = a.gateup && h == 1;
      return a.gateup ? 16 * b + n16 : 32 * b + 16 * h + n16;
    };
    uint32_t v = 0u;
    if (a.wf == WF_MXS) {
      // piece i = 2 * stage + half: lane l's 16 stored bytes of tile row (half, l % 16) at
      // elements kc + 128 * stage + 32 * (l / 16); the scale word of lane l: byte 2 * stage +
      // half is the E8M0 scale of those 32 elements
      const int lane = o < 1024 ? (o >> 2) & 63 : o - 1024, n16 = lane & 15, kq = lane >> 4;
      const int NB = a.cols / 32;
      if (o < 1024) {
        const int i = o >> 8, st = i >> 1, h = i & 1;
        bool upper;
        const int row = src_row(h, n16, upper);
        const int e0 = kc + 128 * st + 32 * kq;
        if (row < a.rows && e0 < a.cols) {
          const uint32_t *w = (const uint32_t *)(upper ? a.b_w : a.a_w);
          v = w[((int64_t)m * a.rows + row) * wpr + e0 / 8 + (o & 3)];
        }
      } else {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int st = bb >> 1, h = bb & 1;
          bool upper;
          const int row = src_row(h, n16, upper);
          const int g = kc / 32 + 4 * st + kq;
          if (row < a.rows && g < NB) {
            const uint8_t *sc = (const uint8_t *)(upper ? a.b_s : a.a_s);
            v |= (uint32_t)sc[((int64_t)m * a.rows + row) * NB + g] << (8 * bb);
          }
        }
      }
    } else if (o < 1024) {  // weights: piece i = o / 256, lane = (o / 4) % 64, word j = o % 4
      const int i = o >> 8, lane = (o >> 2) & 63, j = o & 3;
      const int q = 4 * i + j;
      const int uu = q / (2 * lpu), h = (q / lpu) & 1, wi = q % lpu;
      const int n16 = lane & 15, kq = lane >> 4;
      bool upper;
      const int row = src_row(h, n16, upper);
      const int e0 = kc + uu * ue + kq * qe;
      if (row < a.rows && e0 < a.cols) {
        const uint32_t *w = (const uint32_t *)(upper ? a.b_w : a.a_w);
        const int word = a.wf == WF_DENSE ? e0 / 2 + wi : e0 / 8 + wi;
        v = w[((int64_t)m * a.rows + row) * wpr + word];
        if (a.wf == WF_AFFINE4) v = pair_order(v);
      }
    } else if (a.wf == WF_AFFINE4) {  // [half][n16][unit]: scale | qbias << 16
      const int ent = o - 1024;
      const int h = ent / (16 * nu), n16 = (ent / nu) % 16, un = ent % nu;
      bool upper;
      const int row = src_row(h, n16, upper);
      const int G = a.cols / a.gq, g = kc / a.gq + un;
      if (row < a.rows && g < G) {
        const uint16_t *sc = (const uint16_t *)(upper ? a.b_s : a.a_s);
        const uint16_t *qb = (const uint16_t *)(upper ? a.b_q : a.a_q);
        const int64_t si = ((int64_t)m * a.rows + row) * G + g;
        v = (uint32_t)sc[si] | ((uint32_t)qb[si] << 16);
      }
    } else {  // MXFP4: [half][n16][8] E8M0 bytes, four per word
      const int NB = a.cols / 32;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int by = 4 * (o - 1024) + bb;
        const int h = by / 128, n16 = (by / 8) % 16, jj = by % 8;
        bool upper;
        const int row = src_row(h, n16, upper);
        const int g = kc / 32 + jj;
        if (row < a.rows && g < NB) {
          const uint8_t *sc = (const uint8_t *)(upper ? a.b_s : a.a_s);
          v |= (uint32_t)sc[((int64_t)m * a.rows + row) * NB + g] << (8 * bb);
        }
      }
    }
    a.out[idx] = v;
  }
}

hipError_t launch_pack(const PackArgs &a, hipStream_t s) {
  const int64_t total = (int64_t)a.n * a.nblk * a.nch * (pk_record_bytes(a.wf, a.gq) / 4);
  if (total <= 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}
