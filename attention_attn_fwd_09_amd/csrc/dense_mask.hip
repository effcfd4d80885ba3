// Dense element mask preparation for gfx950.
//
// The generic mask of the fused multi-head attention operator write-up (zwxr.cn), section 3.3,
// is one byte per (query, key) pair: 0 sends the score to minus infinity. The attention kernels
// cannot afford a byte load per score, and should not visit 64x64 blocks the mask hides
// entirely (the write-up advises skipping blocks with no work in them). One pass over the byte mask
// therefore produces, per distinct (batch element, query head) of the mask:
//   * row bits: bit k % 32 of word k / 32 of query row q (the forward and the dQ pass read the
//     32 keys of one half-tile with one word per lane);
//   * column bits: bit q % 32 of word q / 32 of key column k (the dK/dV pass holds one key per
//     lane and 16 consecutive queries);
//   * a block layout: one byte per 64x64 block, 1 if the block keeps any pair, which the planner
//     and the kernels use exactly like a block-sparse layout.
// One workgroup per 64x64 block: the block's bytes go to LDS once; rows and columns are packed
// from there.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

__global__ __launch_bounds__(256) void dense_pack_kernel(DensePackParams p) {
  __shared__ uint8_t tile[64][64 + 4];
  const int t = threadIdx.x;
  const int bi = (int)(blockIdx.x / (uint32_t)p.nb_k), bj = (int)(blockIdx.x % (uint32_t)p.nb_k);
  const int bh = (int)blockIdx.y;                       // b_m * heads_m + h_m
  const int b_m = bh / p.heads_m, h_m = bh % p.heads_m;
  const uint8_t* src = p.mask + b_m * p.stride_b + h_m * p.stride_h;

  // thread t: row r = t / 4 of the block, keys c0 .. c0 + 15
  const int r = t >> 2, c0 = (t & 3) * 16;
  const int q = bi * 64 + r;
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int k = bj * 64 + c0 + e;
    const uint8_t v = (q < p.seq_q && k < p.seq_k) ? src[(size_t)q * p.seq_k + k] : (uint8_t)0;
    tile[r][c0 + e] = v;
    bits |= (uint32_t)(v != 0) << e;
  }
  // row bits: 16-bit halves of the row's words
  const int word = bj * 2 + (c0 >> 5);
  if (q < p.seq_q && word < p.row_words) {
    uint16_t* row = (uint16_t*)(p.row_bits + ((size_t)bh * p.seq_q + q) * p.row_words);
    row[word * 2 + ((c0 >> 4) & 1)] = (uint16_t)bits;
  }
  const int any = __syncthreads_or(bits != 0);
  if (t == 0) p.layout[((size_t)bh * p.nb_q + bi) * p.nb_k + bj] = any ? 1 : 0;
  // column bits: thread t < 128 packs key column t / 2, queries (t % 2) * 32 .. + 31
  if (p.col_bits != nullptr && t < 128) {
    const int c = t >> 1, qh = t & 1;
    const int k = bj * 64 + c;
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) w |= (uint32_t)(tile[qh * 32 + e][c] != 0) << e;
    const int cw = bi * 2 + qh;
    if (k < p.seq_k && cw < p.col_words) p.col_bits[((size_t)bh * p.seq_k + k) * p.col_words + cw] = w;
  }
}

}  // namespace

hipError_t launch_dense_pack(const DensePackParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(dense_pack_kernel, dim3((uint32_t)p.nb_q * (uint32_t)p.nb_k, (uint32_t)(p.batch_m * p.heads_m)),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn
