// Fused attention forward, bf16 in / fp32 accumulate, for gfx950 (CDNA4).
//
// Method: the FlashAttention-style forward of the "fused multi-head attention operator" write-up
// (zwxr.cn), sections 3.1-3.3: one workgroup owns a tile of BM query rows, streams the key/value
// rows tile by tile (64 keys at a time), computes the scores and an online softmax on chip
// (running row maximum and sum with a correction factor), accumulates P V in registers, and writes
// O and the per-row log-sum-exp once at the end. The seq x seq score matrix never reaches HBM.
//
// gfx950 mapping:
//  * every wave owns 32 query rows; BM = 32 * NW.
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: lane (c, h) of
//    the 32x32 result holds query c and 16 consecutive keys (h selects the half), so the row max
//    and sum reduce inside the lane plus one permlane32 swap with lane c+32.
//  * Q lives in registers for the whole item (B operand of the score product).
//  * K and V tiles are copied global -> LDS by the buffer-load-to-LDS path (no VGPR staging,
//    hardware zero-fill past the end of the sequence), double-buffered: the copy of tile j+1 is in
//    flight while tile j is computed.
//  * P is converted to bf16 in registers and used directly as the B operand of O^T += V^T P^T; the
//    V^T operand comes from LDS through the transposing ds_read_b64_tr_b16.
//  * the running maximum is re-based only when it grows by more than 2^8 (exact: numerator and
//    denominator always share the same reference), which skips most accumulator rescales.
#include <type_traits>

#include "common.h"
#include "fwd_shared.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int BN = 64;           // keys per tile
constexpr float RESCALE_SLACK = 8.0f;  // log2 headroom before the reference maximum is re-based
constexpr int K_LEAD = 4;        // k-steps of K fragment reads in flight ahead of the score MFMAs

template <int D>
struct FwdLds {
  static constexpr int TILE_BYTES = BN * D * 2;              // one K or V tile
  static constexpr int MAX_LIST = 1024;                      // kept key tiles per query tile
};

// MINW: waves per SIMD the register allocation must allow (2 lets two workgroups share a CU).
template <int D, int NW, int MASK, int MINW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(MINW))) void fwd_bf16_kernel(FwdParams p) {
  constexpr int BM = NW * 32;
  constexpr int KS = D / 16;   // k-steps of the score product
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int RB = D * 2;    // bytes per tile row
  using L = FwdLds<D>;
  // Four separately named tiles (K and V of stage 0 and 1): the compiler can then prove that the
  // buffer-to-LDS copy into one stage does not alias the reads of the other, and issues no
  // vmcnt wait before those reads.
  __shared__ __attribute__((aligned(16))) char k_st0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_st0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char k_st1[L::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_st1[L::TILE_BYTES];
  // block and dense masks walk a list of kept key tiles (a dense mask through its derived layout)
  constexpr bool LISTED = MASK == MASK_BLOCK || MASK == MASK_DENSE;
  // Structured masks issue the copy of the next tile after the score MFMAs, so that its LDS writes
  // land while the softmax runs instead of during the burst of K reads that opens every tile (the
  // listed masks, whose kept tiles are farther apart in memory, keep the copy at the step's start).
  constexpr bool LATE = !LISTED;
  __shared__ uint32_t list[LISTED ? L::MAX_LIST + 1 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hh = lane >> 5;
  const int i16 = lane & 15, dsub = ((lane >> 4) & 1) * 16;

  // ---- which tile of which (batch, head), and which part of its key range (split-KV) ----
  int item_idx, split;
  split_item(blockIdx.x, p.n_items, p.kv_splits, p.n_xcd, item_idx, split);
  Item it;
  if constexpr (MASK == MASK_NONE || MASK == MASK_CAUSAL) {
    it = closed_form_item(item_idx, p.batch, p.heads_q, p.heads_kv, p.n_qtiles, MASK == MASK_CAUSAL, p.n_xcd);
  } else {
    it = decode_item(p.items[item_idx], p.heads_q, p.n_qtiles);
  }
  const int b = it.b, h = it.h, kvh = h / p.group;
  const int q0 = it.t * BM;
  // the 32 query rows of this wave: waves 0-1 cover the tile's first layout row, 2-3 its second
  // (under a block layout, the two rows the planner paired for the tile)
  const int qw0 = (MASK == MASK_BLOCK && BM == 128) ? tile_row(p.row_pairs, it.t, wave >> 1) * 64 + (wave & 1) * 32
                                                    : q0 + wave * 32;
  const int my_q = qw0 + c;
  // dense mask: this query's row of bits (only read when MASK_DENSE)
  const uint32_t* dense_row = MASK == MASK_DENSE
      ? p.dense.rows + b * p.dense.rows_stride_b + h * p.dense.rows_stride_h + (int64_t)my_q * p.dense.row_words
      : nullptr;

  const size_t q_off = ((size_t)(b * p.heads_q + h) * p.seq_q) * D;
  const size_t kv_off = ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const bf16*)p.q + q_off, (uint32_t)p.seq_q * RB);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const bf16*)p.k + kv_off, (uint32_t)p.seq_k * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16*)p.v + kv_off, (uint32_t)p.seq_k * RB);

  // ---- Q fragments: B operand of S^T = K Q^T; lane (c, hh) holds Q[my_q][16 ks + 8 hh .. +7] ----
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const i32x4 raw = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
        rq, (uint32_t)my_q * RB + (uint32_t)(ks * 32 + hh * 16), 0, 0));
    qf[ks] = __builtin_bit_cast(bf16x8, raw);
  }

  // ---- key tiles this item walks ----
  int kv_len, q_len;
  const int n_tiles = fwd_key_tiles<MASK, BM, BN>(p, b, h, q0, wave, lane, list, L::MAX_LIST, kv_len, q_len);

  // ---- per-lane LDS byte offsets inside a tile; everything else in an address is a constant ----
  // K row fragment for k-step ks of key block kb: koff[ks] + kb * 32 rows.
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int row = sigma32(c);
    koff[ks] = row * RB + (((2 * ks + hh) ^ swz<D>(row)) * 16);
  }
  // transposed V fragment for column block db, rows +0..3 (half 0) or +4..7 (half 1) of the
  // 8-key chunk: voff[db][half] + (chunk base row) rows.
  int voff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = hh * 16 + half * 4 + (i16 >> 2);
      const int d = db * 32 + dsub + 4 * (i16 & 3);
      voff[db][half] = row * RB + (((d >> 3) ^ swz<D>(row)) * 16) + (d & 7) * 2;
    }
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;   // reference maximum, log2 domain (scores times scale*log2(e))
  float l_run = 0.0f;        // this lane's partial denominators (its 16 keys of the first and of
  float l_run2 = 0.0f;       // the second 32-key block of every tile)
  const float cs = p.scale_log2;

  auto tile_index = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (LISTED) return (int)(list[j] & 0xffffu);
    return j;
  };
  auto issue_tile = [&](auto stage_tag, int kt) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    issue_rows<D, NW>(ST == 0 ? k_st0 : k_st1, rk, kt * BN, wave, lane);
    issue_rows<D, NW>(ST == 0 ? v_st0 : v_st1, rv, kt * BN, wave, lane);
  };

  // One 64-key tile for this wave's 32 queries, read from LDS stage ST; after_scores() runs once
  // the score MFMAs are issued (the late copy of the next tile, or nothing). The instruction order is
  // pinned with sched_group_barrier (masks: 0x008 MFMA, 0x100 LDS read, 0x002 VALU) so that LDS
  // reads run K_LEAD k-steps ahead of the MFMAs that consume them, and the first V fragments are in
  // flight while the softmax runs on the vector ALU.
  auto tile = [&](auto stage_tag, auto masked_tag, int k0, auto&& after_scores) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* kl = ST == 0 ? k_st0 : k_st1;
    const char* vl = ST == 0 ? v_st0 : v_st1;

    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    bf16x8 ka[KS], kb1[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ka[ks] = *(const bf16x8*)(kl + koff[ks]);
      kb1[ks] = *(const bf16x8*)(kl + koff[ks] + 32 * RB);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma32(ka[ks], qf[ks], s0);
      s1 = mfma32(kb1[ks], qf[ks], s1);
    }
    constexpr int KL = K_LEAD < KS ? K_LEAD : KS;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KL, 0);
#pragma unroll
    for (int ks = 0; ks < KS - KL; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * KL, 0);
    if constexpr (LATE) __builtin_amdgcn_sched_barrier(0);
    after_scores();
    if constexpr (LATE) __builtin_amdgcn_sched_barrier(0);

    // ---- mask (boundary tiles only): hidden scores become -inf ----
    uint32_t dw0 = 0, dw1 = 0;   // dense mask: the query's bits for keys k0 .. k0+31, k0+32 .. k0+63
    if constexpr (MASK == MASK_DENSE) {
      if (my_q < p.seq_q) {
        const int w = k0 >> 5;
        dw0 = dense_row[w];
        if (w + 1 < p.dense.row_words) dw1 = dense_row[w + 1];
      }
    }
    if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key0 = k0 + hh * 16 + i, key1 = key0 + 32;
        bool v0 = key0 < kv_len, v1 = key1 < kv_len;
        if constexpr (MASK == MASK_CAUSAL) {
          v0 = v0 && key0 <= my_q;
          v1 = v1 && key1 <= my_q;
        }
        if constexpr (MASK == MASK_PADDING) {
          v0 = v0 && my_q < q_len;
          v1 = v1 && my_q < q_len;
        }
        if constexpr (MASK == MASK_DENSE) {
          v0 = v0 && ((dw0 >> (hh * 16 + i)) & 1u);
          v1 = v1 && ((dw1 >> (hh * 16 + i)) & 1u);
        }
        s0[i] = v0 ? s0[i] : -INFINITY;
        s1[i] = v1 ? s1[i] : -INFINITY;
      }
    }

    // ---- online softmax on this lane's 32 scores (keys k0 + kb*32 + hh*16 + i) ----
    // two chains of three-input maxima (one per key block), then their maximum
    float ma = vmax(s0[0], s0[1]), mb = vmax(s1[0], s1[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      ma = vmax3(ma, s0[i], s0[i + 1]);
      mb = vmax3(mb, s1[i], s1[i + 1]);
    }
    float mx = partner_max(vmax(ma, mb)) * cs;   // cs > 0, so max(s) * cs = max(s * cs); -inf stays -inf
    if (__builtin_expect(__ballot(mx > m_run + RESCALE_SLACK) != 0, 0)) {
      const float m_new = vmax(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      l_run2 *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float msub = (m_run == -INFINITY) ? 0.0f : m_run;

    // first V fragments go out before the exponentials
    bf16x8 va[4][DB];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int rows = ((kc >> 1) * 32 + (kc & 1) * 8) * RB;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vl + voff[db][0] + rows));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vl + voff[db][1] + rows));
        va[kc][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
    bf16x8 pb[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e0 = fast_exp2(fmaf(s0[i], cs, -msub));
      const float e1 = fast_exp2(fmaf(s1[i], cs, -msub));
      pb[i >> 3][i & 7] = (bf16)e0;
      pb[2 + (i >> 3)][i & 7] = (bf16)e1;
    }
    // the denominator sums the same bf16-rounded probabilities that enter P V
    l_run = sum_bf16x8(pb[0], sum_bf16x8(pb[1], l_run));
    l_run2 = sum_bf16x8(pb[2], sum_bf16x8(pb[3], l_run2));
    // O^T += V^T P^T; chunk kc holds keys kb*32 + hh*16 + hc*8 + 0..7 for lane half hh
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = mfma32(va[kc][db], pb[kc], acc[db]);
    }
    constexpr int PV = 4 * DB;                 // PV MFMAs, two transposed reads each
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 200, 0);
#pragma unroll
    for (int m = 0; m < PV - 4; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // Tile j lives in LDS stage j % 2; the copy of tile j+1 into the other stage is in flight while
  // tile j is computed. Tiles [0, n_free) need no masking for any wave of the workgroup and run a
  // body without mask code; the rest (causal diagonal, ragged tail, padded query rows) check per
  // wave whether they see the tile at all and apply the element mask.
  const int n_free =
      fwd_free_tiles<MASK, BM, BN>(p, q0, kv_len, q_len, n_tiles, n_tiles > 0 ? tile_index(n_tiles - 1) : 0);
  int t0, t1;
  fwd_split_range(p, split, n_tiles, t0, t1);
  const int t_free = min(max(n_free, t0), t1);

  auto step = [&](auto stage_tag, auto masked_tag, int j) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    wait_vmem();
    __syncthreads();  // tile j is in LDS; every wave is done with the stage tile j+1 will overwrite
    auto issue_next = [&]() __attribute__((always_inline)) {
      if (j + 1 < t1) issue_tile(std::integral_constant<int, 1 - ST>{}, tile_index(j + 1));
    };
    if constexpr (!LATE) issue_next();
    const int k0 = tile_index(j) * BN;
    // wave-uniform: does this wave see any key of the tile?
    bool active = true;
    if constexpr (LISTED && (MASKED || BM > 64)) active = ((list[j] >> 16) >> ((wave * 32) / 64)) & 1u;
    if constexpr (MASKED && !LISTED) {
      active = k0 < kv_len;
      if constexpr (MASK == MASK_CAUSAL) active = active && k0 <= qw0 + 31;
      if constexpr (MASK == MASK_PADDING) active = active && qw0 < q_len;
    }
    if constexpr (LATE) {
      if (active) tile(stage_tag, masked_tag, k0, issue_next);
      else issue_next();
    } else if (active) {
      tile(stage_tag, masked_tag, k0, [] {});
    }
  };
  auto run = [&](auto masked_tag, int j0, int j1) __attribute__((always_inline)) {
    int j = j0;
    if (j < j1 && (j & 1)) step(std::integral_constant<int, 1>{}, masked_tag, j++);
    for (; j + 1 < j1; j += 2) {
      step(std::integral_constant<int, 0>{}, masked_tag, j);
      step(std::integral_constant<int, 1>{}, masked_tag, j + 1);
    }
    if (j < j1) step(std::integral_constant<int, 0>{}, masked_tag, j);
  };

  // tile j lives in stage j % 2
  if (t0 < t1) {
    if (t0 & 1) issue_tile(std::integral_constant<int, 1>{}, tile_index(t0));
    else issue_tile(std::integral_constant<int, 0>{}, tile_index(t0));
  }
  run(std::false_type{}, t0, t_free);
  run(std::true_type{}, t_free, t1);

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l); empty rows give O = 0, LSE = -inf ----
  const float l = partner_sum(l_run + l_run2);
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : __builtin_amdgcn_rcpf(l);
  if (p.kv_splits > 1) {
    // partial result of this split: O over its keys in fp32 and its log2-sum-exp
    if (my_q < p.seq_q) {
      const size_t rows = (size_t)p.batch * p.heads_q * p.seq_q;
      const size_t row = (size_t)(b * p.heads_q + h) * p.seq_q + my_q;
      float* og = p.o_part + ((size_t)split * rows + row) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = acc[db][g4 * 4 + e] * inv;
          *(f32x4*)(og + db * 32 + g4 * 8 + hh * 4) = v4;
        }
      }
      if (hh == 0) p.lse_part[(size_t)split * rows + row] = empty ? -INFINITY : m_run + __builtin_amdgcn_logf(l);
    }
    return;
  }
  // Under the listed and padding masks O goes out as whole rows through LDS (2-4% faster there);
  // the no-mask and causal kernels store each lane's 8-byte pieces directly (as fast or faster)
  if constexpr (MASK == MASK_NONE || MASK == MASK_CAUSAL) {
    if (my_q < p.seq_q) {
      bf16* og = (bf16*)p.o + q_off + (size_t)my_q * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)(acc[db][g4 * 4 + e] * inv);
          *(bf16x4*)(og + db * 32 + g4 * 8 + hh * 4) = v4;
        }
      }
    }
  } else {
    // O as whole rows, staged in one of the four K/V stage arrays per wave (free once every wave
    // has passed the last tile)
    static_assert(NW <= 4 && 32 * (RB + 8) <= L::TILE_BYTES, "one stage array per wave");
    __syncthreads();
    char* rows_lds = wave == 0 ? k_st0 : wave == 1 ? v_st0 : wave == 2 ? k_st1 : v_st1;
    write_rows_bf16<D>(rows_lds, acc, inv, lane, (bf16*)p.o + q_off + (size_t)qw0 * D, p.seq_q - qw0);
  }
  if (my_q < p.seq_q && hh == 0) {
    const float lse = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
    p.lse[(size_t)(b * p.heads_q + h) * p.seq_q + my_q] = lse;
  }
}

// ------------------------------------------------------------------------------------------------
// Split-KV merge: the splits of one query row hold O_s (normalised over their keys) and
// lse_s = log2 of their partial denominators (in the reference of the row maximum); the row's
// result is LSE = log sum_s 2^lse_s and O = sum_s 2^(lse_s - LSE) O_s. D/4 lanes per row, 4 columns
// each. A row no split saw gives O = 0, LSE = -inf.
template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdParams p, int64_t rows) {
  constexpr int LPR = D / 4;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int col = (threadIdx.x % LPR) * 4;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < p.kv_splits; ++s) mx = vmax(mx, p.lse_part[(size_t)s * rows + row]);
  f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  float wsum = 0.0f;
  if (mx != -INFINITY) {
    for (int s = 0; s < p.kv_splits; ++s) {
      const float w = fast_exp2(p.lse_part[(size_t)s * rows + row] - mx);
      const f32x4 os = *(const f32x4*)(p.o_part + ((size_t)s * rows + row) * D + col);
      o += w * os;
      wsum += w;
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  bf16x4 v4;
#pragma unroll
  for (int e = 0; e < 4; ++e) v4[e] = (bf16)(o[e] * inv);
  *(bf16x4*)((bf16*)p.o + row * D + col) = v4;
  if (col == 0) p.lse[row] = wsum > 0.0f ? (mx + __builtin_amdgcn_logf(wsum)) * 0.69314718055994530942f : -INFINITY;
}

#ifndef ATTN_FWD_NW
#define ATTN_FWD_NW 4
#endif
#ifndef ATTN_FWD_MINW
#define ATTN_FWD_MINW 2
#endif

template <int D, int NW, int MASK, int MINW>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, MASK, MINW>), dim3((uint32_t)p.n_items * (uint32_t)p.kv_splits),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mask(const FwdParams& p, int mask, hipStream_t stream) {
  constexpr int NW = ATTN_FWD_NW, MW = ATTN_FWD_MINW;
  switch (mask) {
    case MASK_NONE: return launch_one<D, NW, MASK_NONE, MW>(p, stream);
    case MASK_CAUSAL: return launch_one<D, NW, MASK_CAUSAL, MW>(p, stream);
    case MASK_PADDING: return launch_one<D, NW, MASK_PADDING, MW>(p, stream);
    case MASK_DENSE: return launch_one<D, 4, MASK_DENSE, 2>(p, stream);
    default: return launch_one<D, 4, MASK_BLOCK, 2>(p, stream);
  }
}

}  // namespace

int fwd_bf16_block_m(int head_dim, int mask) {
  (void)head_dim;
  return (mask == MASK_BLOCK || mask == MASK_DENSE) ? 128 : 32 * ATTN_FWD_NW;
}

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, int mask, hipStream_t stream) {
  return head_dim == 128 ? launch_mask<128>(p, mask, stream) : launch_mask<64>(p, mask, stream);
}

hipError_t launch_fwd_merge(const FwdParams& p, int head_dim, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.heads_q * p.seq_q;
  const int rpb = 256 / (head_dim / 4);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (head_dim == 128)
    hipLaunchKernelGGL(fwd_merge_kernel<128>, dim3(grid), dim3(256), 0, stream, p, rows);
  else
    hipLaunchKernelGGL(fwd_merge_kernel<64>, dim3(grid), dim3(256), 0, stream, p, rows);
  return hipGetLastError();
}

}  // namespace attn
