// Work decomposition shared by the forward kernels (bf16 and fp8 inputs): which key tiles one
// query tile visits under each mask kind, and which of them need no element mask.
#pragma once

#include "common.h"
#include "params.h"

namespace attn {

// Key tiles of one (batch, head, query tile) item: the sequence the item walks, in order.
//  * NONE: every tile of the keys; CAUSAL: tiles up to the item's last query;
//  * PADDING: tiles of the batch element's valid length (none for a fully padded query tile);
//  * BLOCK / DENSE: the kept tiles of the layout rows the item covers (a dense mask through its
//    derived layout; for 128-row tiles the two rows tile_row names), listed by wave 0 into `list`
//    with one bit per covered 64-row layout row (bits << 16 | key tile); list[max_list] holds the
//    count.
// kv_len / q_len: keys at or beyond kv_len are hidden; queries at or beyond q_len see nothing.
// Every thread of the workgroup must call this (the list is published with a barrier).
template <int MASK, int BM, int BN>
__device__ __forceinline__ int fwd_key_tiles(const FwdParams& p, int b, int h, int q0, int wave, int lane,
                                             uint32_t* list, int max_list, int& kv_len, int& q_len) {
  kv_len = p.seq_k;
  q_len = p.seq_q;
  if constexpr (MASK == MASK_PADDING) {
    kv_len = clamp_len(p.lengths[b], p.seq_k);
    q_len = clamp_len(p.lengths[b], p.seq_q);
    return (q0 < q_len) ? (kv_len + BN - 1) / BN : 0;
  } else if constexpr (MASK == MASK_CAUSAL) {
    const int last_q = min(q0 + BM, p.seq_q) - 1;
    return min((p.seq_k + BN - 1) / BN, last_q / BN + 1);
  } else if constexpr (MASK == MASK_BLOCK || MASK == MASK_DENSE) {
    constexpr int ROWS = BM / 64 > 0 ? BM / 64 : 1;
    const uint8_t* lay = p.layout + b * p.layout_stride_b + h * p.layout_stride_h;
    const int r0 = q0 / 64;
    if (wave == 0) {
      int count = 0;
      for (int j0 = 0; j0 < p.nb_k; j0 += 64) {
        const int j = j0 + lane;
        uint32_t bits = 0;
        if (j < p.nb_k) {
#pragma unroll
          for (int r = 0; r < ROWS; ++r) {
            const int row = ROWS == 2 ? tile_row(p.row_pairs, r0 / 2, r) : r0 + r;
            if (row < p.nb_q && lay[(size_t)row * p.nb_k + j] != 0) bits |= 1u << r;
          }
        }
        const uint64_t ball = __ballot(bits != 0);
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(ball >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ball, 0));
        if (bits != 0) list[count + before] = (uint32_t)j | (bits << 16);
        count += __popcll(ball);
      }
      if (lane == 0) list[max_list] = (uint32_t)count;
    }
    lds_barrier();   // the Q loads issued before the list stay in flight
    return (int)list[max_list];
  } else {
    return (p.seq_k + BN - 1) / BN;
  }
}

// Tiles [0, n_free) of the walk need no element mask for any wave of the workgroup; the rest
// (causal diagonal, ragged tail, padded query rows, every tile of a dense mask) do.
// last_tile: key tile index of the walk's last entry (listed masks only).
template <int MASK, int BM, int BN>
__device__ __forceinline__ int fwd_free_tiles(const FwdParams& p, int q0, int kv_len, int q_len, int n_tiles,
                                              int last_tile) {
  int n_free;
  if constexpr (MASK == MASK_CAUSAL) {
    n_free = min(q0 / BN, p.seq_k / BN);
  } else if constexpr (MASK == MASK_PADDING) {
    n_free = (q0 + BM <= q_len) ? kv_len / BN : 0;
  } else if constexpr (MASK == MASK_BLOCK) {
    n_free = (n_tiles > 0 && last_tile * BN + BN > p.seq_k) ? n_tiles - 1 : n_tiles;
  } else if constexpr (MASK == MASK_DENSE) {
    n_free = 0;
  } else {
    n_free = p.seq_k / BN;
  }
  return min(n_free, n_tiles);
}

// Split-KV: workgroup `split` of an item visits tiles [t0, t1) of its walk, an equal share.
__device__ __forceinline__ void fwd_split_range(const FwdParams& p, int split, int n_tiles, int& t0, int& t1) {
  t0 = 0;
  t1 = n_tiles;
  if (p.kv_splits > 1) {
    const int chunk = (n_tiles + p.kv_splits - 1) / p.kv_splits;
    t0 = min(split * chunk, n_tiles);
    t1 = min(t0 + chunk, n_tiles);
  }
}

}  // namespace attn
