// Internal interface between the C ABI (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "params.h"

namespace attn {

enum PlanMode : int { PLAN_FWD_Q = 0, PLAN_BWD_KV = 1 };

// Input of the tile-list scheduler. Items are numbered (b * heads + h) * n_tiles + t.
struct PlanParams {
  int32_t mode;          // PlanMode
  int32_t mask;          // mask kind
  int32_t heads;         // heads_q for PLAN_FWD_Q, heads_kv for PLAN_BWD_KV
  int32_t group;         // heads_q / heads_kv
  int32_t seq_q, seq_k;
  int32_t n_tiles;       // tiles per (b, h)
  int32_t tile;          // rows per tile (BM for query tiles, BN for key tiles)
  int32_t n_items;
  int32_t nb_q, nb_k;
  const int32_t* lengths;
  const uint8_t* layout;
  int64_t layout_stride_b, layout_stride_h;
  int32_t n_xcd;         // XCDs workgroups are dealt to round robin (at most kMaxXcd; 1 = no grouping)
  uint32_t* items;       // output: item ids, longest first
  uint16_t* row_pairs;   // output (query tiles of two layout rows, when plan_pairs_rows holds): the two
                         //   rows of tile t are row_pairs[2t], row_pairs[2t + 1]; nb_q = no row. Else null
};

constexpr int kMaxXcd = 8;   // XCDs the planner can group items for

// Whether a query-tile list pairs its layout rows by shared kept tiles instead of taking rows 2t
// and 2t + 1: a block layout shared by every (batch, head), of at most 64 rows and 64 key tiles
// per row, with 128-row query tiles (two layout rows each). Host and device decide alike.
__host__ __device__ inline bool plan_pairs_rows(int mask, int64_t layout_stride_b, int64_t layout_stride_h, int tile,
                                                int n_tiles, int nb_q, int nb_k) {
  return mask == MASK_BLOCK && layout_stride_b == 0 && layout_stride_h == 0 && tile == 128 && nb_k <= 64 &&
         nb_q <= 64 && n_tiles == (nb_q + 1) / 2;
}

// Dense element mask -> row bits, column bits (optional) and a 64x64 block layout.
struct DensePackParams {
  const uint8_t* mask;          // caller's byte mask, [.., seq_q, seq_k]
  int64_t stride_b, stride_h;   // elements between batch elements / query heads of the mask
  int32_t batch_m, heads_m;     // distinct batch elements / heads of the mask (1 when shared)
  int32_t seq_q, seq_k, nb_q, nb_k;
  uint32_t* row_bits;           // [batch_m * heads_m][seq_q][row_words]
  uint32_t* col_bits;           // [batch_m * heads_m][seq_k][col_words], or null
  int32_t row_words, col_words;
  uint8_t* layout;              // [batch_m * heads_m][nb_q][nb_k]
};
hipError_t launch_dense_pack(const DensePackParams& p, hipStream_t stream);

hipError_t launch_plan(const PlanParams& p, hipStream_t stream);
hipError_t launch_plan_pair(const PlanParams& a, const PlanParams& b, hipStream_t stream);
hipError_t launch_plan_triple(const PlanParams& a, const PlanParams& b, const PlanParams& c, hipStream_t stream);

int fwd_bf16_block_m(int head_dim, int mask);
hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, int mask, hipStream_t stream);
hipError_t launch_fwd_merge(const FwdParams& p, int head_dim, hipStream_t stream);
int fwd_fp8_block_m();
hipError_t launch_fwd_fp8(const FwdParams& p, int head_dim, int mask, hipStream_t stream);

int fwd_f32_block_m();
hipError_t launch_fwd_f32(const FwdParams& p, int head_dim, int mask, hipStream_t stream);

// Backward: tile sizes and launchers.
int bwd_block_q(int head_dim, int mask);
// dK/dV kernel of a backward call: one wave per 32 keys (single-pass mode, and layouts with more
// listed steps than the wave-pair kernel holds), or wave pairs in 64-key workgroups.
enum { DKDV_ONE_WAVE = 0, DKDV_PAIR = 1 };
int bwd_dkdv_variant(int mask, int flags, int group, int nb_q);
int bwd_block_k(int head_dim, int mask, int variant);
int bwd_max_steps();  // (query head, query tile) pairs one dK/dV workgroup can list for a block mask
hipError_t launch_bwd_preprocess(const BwdParams& p, int head_dim, hipStream_t stream);
hipError_t launch_bwd_dkdv(const BwdParams& p, int head_dim, int mask, int n_items, hipStream_t stream);
hipError_t launch_bwd_dkdv_pair(const BwdParams& p, int head_dim, int mask, int n_items, hipStream_t stream);
hipError_t launch_bwd_dq_convert(const BwdParams& p, int head_dim, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdParams& p, int head_dim, int mask, int n_items, hipStream_t stream);

}  // namespace attn
