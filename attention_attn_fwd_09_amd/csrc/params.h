// Plain parameter blocks passed by value from the C ABI to the kernels (no device code here).
#pragma once

#include <stdint.h>

namespace attn {

// Mask kinds, same values as the C ABI.
enum MaskKind : int { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_PADDING = 2, MASK_BLOCK = 3, MASK_DENSE = 4 };

// A dense element mask packed to bits (built from the caller's byte mask by the pack kernel).
// Kernels of the dense kind walk the kept 64x64 blocks of the derived block layout (in the
// layout fields of the parameter blocks) and test every pair against these bits.
struct DenseBits {
  const uint32_t* rows;         // bit (k % 32) of word k / 32 of query row q: [.., seq_q][row_words]
  const uint32_t* cols;         // bit (q % 32) of word q / 32 of key column k: [.., seq_k][col_words]
  int32_t row_words, col_words; // ceil(seq_k / 32), ceil(seq_q / 32)
  int64_t rows_stride_b, rows_stride_h;   // words per batch element / query head (0 = shared)
  int64_t cols_stride_b, cols_stride_h;
};

// Everything a kernel needs to know about one call, passed by value.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* lengths;       // PADDING
  const uint8_t* layout;        // BLOCK
  int64_t layout_stride_b, layout_stride_h;
  const uint32_t* items;        // planner output (PADDING/BLOCK), else null
  const uint16_t* row_pairs;    // planner output: the two layout rows of each 128-row query tile, or
                                //   null for rows 2t, 2t + 1
  int32_t batch, heads_q, heads_kv, seq_q, seq_k;
  int32_t group;                // heads_q / heads_kv
  int32_t n_qtiles;             // ceil(seq_q / BM)
  int32_t n_items;              // batch * heads_q * n_qtiles
  int32_t nb_q, nb_k;           // BLOCK layout dims (64 x 64 tiles)
  float scale;                  // softmax scale
  float scale_log2;             // scale * log2(e)
  DenseBits dense;              // MASK_DENSE (bf16 kernels)
  const uint8_t* dense_bytes;   // MASK_DENSE (fp32 kernel): the caller's byte mask
  int64_t dense_stride_b, dense_stride_h;
  int32_t kv_splits;            // workgroups sharing one item's key range (1 = no split)
  int32_t n_xcd;                // XCDs the dispatcher deals workgroups to, round robin (1 = no grouping)
  float* o_part;                // kv_splits > 1: per-split O (normalised over the split), fp32
                                //   [kv_splits][batch * heads_q * seq_q][head_dim]
  float* lse_part;              // kv_splits > 1: per-split log2-sum-exp, fp32 [kv_splits][rows]
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;                 // workspace: -rowsum(dO * O) (negated Delta), fp32 [B, Hq, Sq]
  float* lse2;                  // workspace: LSE * log2(e), +inf for empty rows, fp32 [B, Hq, Sq]
  float* sseed;                 // workspace (two-pass mode): -LSE / scale, -inf for empty rows, fp32
                                //   [B, Hq, Sq]: the start value of the dK/dV pass's score accumulator
  DenseBits dense;              // MASK_DENSE
  float* dq_acc;                // single-pass mode: dQ / scale accumulated with fp32 atomics,
                                //   [B, Hq, Sq, D]; zeroed by the preprocess; null otherwise
  const int32_t* lengths;
  const uint8_t* layout;
  int64_t layout_stride_b, layout_stride_h;
  const uint32_t* items_kv;     // planner output for the dK/dV pass
  const uint32_t* items_q;      // planner output for the dQ pass
  const uint16_t* row_pairs;    // planner output: the two layout rows of each dQ query tile, or null
  int32_t batch, heads_q, heads_kv, seq_q, seq_k;
  int32_t group;
  int32_t n_qtiles, n_ktiles;
  int32_t nb_q, nb_k;
  float scale, scale_log2;
  float inv_scale_log2;         // 1 / scale_log2
};

}  // namespace attn
