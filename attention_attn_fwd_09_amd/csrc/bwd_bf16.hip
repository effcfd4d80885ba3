// Backward of fused attention (bf16 in, fp32 accumulate) for gfx950.
//
// The Xingchen-Cup report on the sparse FlashAttention backward operator (smzdm.com), section 03:
// the backward produces three gradients, dQ, dK and dV; the forward threw the attention matrix
// away, so the backward recomputes it block by block from the saved per-row statistics; and the
// gradients accumulate in conflicting directions: one traversal can complete two of them while
// the third runs the other way, so either two loops are made or many cores add into the same place
// and must resolve write conflicts. This file takes the two-loop option (no output atomics, a
// deterministic result):
//
//   dQ pass     (runs first) one workgroup per query tile: Q_i, dO_i stay in registers; the
//               workgroup first computes its rows' Delta_i = sum_d dO_id O_id (equal to
//               sum_j P_ij dP_ij; fp32, stored negated so that it can seed the dP accumulators)
//               and LSE_i log2(e), and writes both for the next pass; then the visible key tiles
//               stream through LDS, S, P, dP, dS are recomputed and dQ_i += scale dS K_j.
//   dK/dV pass  one workgroup per key tile: K_j, V_j stay in registers, every (query head of the
//               group, query tile) that sees the tile streams Q_i, dO_i, LSE_i, Delta_i through
//               LDS; S = Q_i K_j^T and dP = dO_i V_j^T are recomputed, P = exp(scale S - LSE),
//               dS = P (dP - Delta), and dV_j += P^T dO_i, dK_j += scale dS^T Q_i accumulate in
//               registers.
//   preprocess  the same row statistics as a kernel of their own, for the single-pass variant
//               (which has no dQ pass).
//
// Skipped blocks of a block-sparse layout (and fully masked causal/padding tiles) are never
// visited. Every product runs on v_mfma_f32_32x32x16_bf16; operands that must be read along the
// contraction dimension of a row-major tile come from LDS through ds_read_b64_tr_b16.
#include <type_traits>

#include "attn.h"
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int BQ = 64;   // queries per streamed tile in the dK/dV pass
constexpr int BN = 64;   // keys per streamed tile in the dQ pass
constexpr float LOG2E = 1.4426950408889634f;

// LSE (natural log) to the log2 domain used by the kernels; an empty row (-inf) maps to +inf so
// that exp2(x - lse2) = 0 for every key of that row.
__device__ __forceinline__ float lse_to_log2(float l) { return l == -INFINITY ? INFINITY : l * LOG2E; }

// ------------------------------------------------------------------------------------------------
// Preprocess of the single-pass variant: -Delta = -rowsum(dO * O) and the row's LSE in the log2
// domain (so the passes subtract it without converting per element). Two lanes per row, summing
// in the order the dQ pass uses for the same statistics (lane half h: columns 16 ks + 8 h + e in
// order, then the two halves added), so both variants see bit-identical -Delta.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int64_t rows) {
  constexpr int KS = D / 16;
  const int64_t row = (int64_t)blockIdx.x * 128 + threadIdx.x / 2;
  const int half = threadIdx.x & 1;
  float acc = 0.0f;
  if (row < rows) {
    const bf16* o = (const bf16*)p.o + row * D + half * 8;
    const bf16* g = (const bf16*)p.dout + row * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 o8 = *(const bf16x8*)(o + ks * 16);
      const bf16x8 g8 = *(const bf16x8*)(g + ks * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)o8[e], (float)g8[e], acc);
    }
  }
  acc += __shfl_xor(acc, 1, 2);
  if (p.dq_acc != nullptr && row < rows) {
    // single-pass mode: this row's half of the dQ accumulator starts at zero
    float* z = p.dq_acc + row * D + half * (D / 2);
#pragma unroll
    for (int i = 0; i < D / 2; i += 4) *(f32x4*)(z + i) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  if (row < rows && half == 0) {
    p.delta[row] = -acc;
    p.lse2[row] = lse_to_log2(p.lse[row]);
  }
}

// ------------------------------------------------------------------------------------------------
// dK/dV pass. Steps are (query head of the group, 64-row query tile) pairs; those that need no
// element mask for any wave of the workgroup come first and run a body without mask code.
template <int D>
struct KvLds {
  static constexpr int TILE = BQ * D * 2;
  static constexpr int STATS = 1024;        // 64 row values (256 B) plus the zero fill of the copy
  static constexpr int MAX_STEPS = 4096;    // listed (query head, layout row) pairs for block masks
};

// ATOMIC_DQ: the single-pass variant (the write-conflict option of the Xingchen-Cup report,
// section 03): the same pass also adds every step's dQ_i contribution, dS K_j, to an fp32
// accumulator with hardware float atomics; a convert kernel scales and rounds it afterwards.
template <int D, int NW, int MASK, bool ATOMIC_DQ = false>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int BK = NW * 32;   // keys per workgroup
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RB = D * 2;
  using L = KvLds<D>;
  // the single-pass variant copies only the 256 bytes of row statistics (lanes 0-15), which
  // leaves room for its per-wave dS tiles at two workgroups per CU
  constexpr int STATS = ATOMIC_DQ ? 256 : L::STATS;
  __shared__ __attribute__((aligned(16))) char q_st0[L::TILE];
  __shared__ __attribute__((aligned(16))) char o_st0[L::TILE];   // dO
  __shared__ __attribute__((aligned(16))) char q_st1[L::TILE];
  __shared__ __attribute__((aligned(16))) char o_st1[L::TILE];
  __shared__ __attribute__((aligned(16))) char l_st0[STATS];  // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) char d_st0[STATS];  // -Delta
  __shared__ __attribute__((aligned(16))) char l_st1[STATS];
  __shared__ __attribute__((aligned(16))) char d_st1[STATS];
  // block and dense masks list the kept (query head, layout row) pairs of the key tile's column
  // (a dense mask through its derived layout)
  constexpr bool LISTED = MASK == MASK_BLOCK || MASK == MASK_DENSE;
  __shared__ uint16_t list[LISTED ? L::MAX_STEPS : 1];
  __shared__ int list_count;
  // single-pass variant: each wave's dS of one 32-query block, [key][query] bf16, 64-byte rows
  __shared__ __attribute__((aligned(16))) char ds_t[ATOMIC_DQ ? NW * 2048 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hh = lane >> 5;
  const int dsub = ((lane >> 4) & 1) * 16, i16 = lane & 15;

  const uint32_t item = p.items_kv[blockIdx.x];
  // an item outside the problem (a list the caller kept from another call) does nothing
  if ((uint64_t)item >= (uint64_t)p.batch * p.heads_kv * p.n_ktiles) return;
  const int kt = (int)(item % (uint32_t)p.n_ktiles);
  const int bkv = (int)(item / (uint32_t)p.n_ktiles);
  const int kvh = bkv % p.heads_kv, b = bkv / p.heads_kv;
  const int k0 = kt * BK;
  const int kw0 = k0 + wave * 32;
  const int my_k = kw0 + c;

  const size_t kv_off = ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const bf16*)p.k + kv_off, (uint32_t)p.seq_k * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16*)p.v + kv_off, (uint32_t)p.seq_k * RB);

  // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)my_k * RB + (uint32_t)(ks * 32 + hh * 16);
    kf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    vf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
  }

  // ---- the (query head, query tile) steps that see this key tile ----
  int kv_len = p.seq_k, q_len = p.seq_q;
  const int n_qt = (p.seq_q + BQ - 1) / BQ;
  int qt_lo = 0, qt_hi = n_qt;
  if constexpr (MASK == MASK_PADDING) {
    kv_len = clamp_len(p.lengths[b], p.seq_k);
    q_len = clamp_len(p.lengths[b], p.seq_q);
    qt_hi = (k0 < kv_len) ? (q_len + BQ - 1) / BQ : 0;
  } else if constexpr (MASK == MASK_CAUSAL) {
    qt_lo = k0 / BQ;
  }
  const bool key_tail = k0 + BK > kv_len;    // some key of the tile is past the end
  // query tiles [qt_m, qt_f) need no mask; [qt_lo, qt_m) (causal diagonal) and the ragged last
  // tile [qt_f, qt_hi) do
  int qt_m = qt_lo, qt_f = qt_hi;
  if constexpr (MASK == MASK_CAUSAL) qt_m = min(qt_hi, max(qt_lo, (k0 + BK - 2) / BQ + 1));
  if (qt_hi > qt_m && (qt_hi * BQ > q_len)) qt_f = qt_hi - 1;
  if (key_tail) qt_f = qt_m;                 // every step masked
  qt_f = max(qt_f, qt_m);
  int n_free, n_steps;
  if constexpr (LISTED) {
    const int col = k0 / 64;
    if (wave == 0) {
      int count = 0;
      for (int g = 0; g < p.group; ++g) {
        const uint8_t* lay = p.layout + b * p.layout_stride_b + (kvh * p.group + g) * p.layout_stride_h;
        for (int r0 = 0; r0 < p.nb_q; r0 += 64) {
          const int r = r0 + lane;
          const bool keep = r < p.nb_q && lay[(size_t)r * p.nb_k + col] != 0;
          const uint64_t ball = __ballot(keep);
          const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(ball >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ball, 0));
          if (keep && count + before < L::MAX_STEPS) list[count + before] = (uint16_t)((g << 10) | r);
          count += __popcll(ball);
        }
      }
      if (lane == 0) list_count = min(count, L::MAX_STEPS);
    }
    lds_barrier();   // the K and V loads issued above stay in flight
    n_steps = list_count;
    // ragged shapes run every step through the masked body, and so does a dense mask
    n_free = (MASK == MASK_DENSE || key_tail || (p.seq_q % BQ) != 0) ? 0 : n_steps;
  } else {
    n_free = p.group * (qt_f - qt_m);
    n_steps = p.group * (qt_hi - qt_lo);
  }
  auto step_at = [&](int s, int& g, int& qt) __attribute__((always_inline)) {
    if constexpr (LISTED) {
      const uint32_t e = list[s];
      g = (int)(e >> 10);
      qt = (int)(e & 1023u);
    } else {
      if (s < n_free) {
        const int per = qt_f - qt_m;
        g = s / per;
        qt = qt_m + s % per;
      } else {
        // masked tiles: the causal diagonal [qt_lo, qt_m) then the tail [qt_f, qt_hi)
        const int r = s - n_free;
        const int per = (qt_m - qt_lo) + (qt_hi - qt_f);
        g = r / per;
        const int m = r % per;
        qt = m < qt_m - qt_lo ? qt_lo + m : qt_f + (m - (qt_m - qt_lo));
      }
    }
  };

  auto issue_step = [&](auto stage_tag, int s) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    int g, qt;
    step_at(s, g, qt);
    const int hq = kvh * p.group + g;
    const size_t q_off = ((size_t)(b * p.heads_q + hq) * p.seq_q) * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const bf16*)p.q + q_off, (uint32_t)p.seq_q * RB);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const bf16*)p.dout + q_off, (uint32_t)p.seq_q * RB);
    issue_rows<D, NW>(ST == 0 ? q_st0 : q_st1, rq, qt * BQ, wave, lane);
    issue_rows<D, NW>(ST == 0 ? o_st0 : o_st1, rdo, qt * BQ, wave, lane);
    if (wave == 0) {
      const size_t r_off = (size_t)(b * p.heads_q + hq) * p.seq_q;
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse2 + r_off, (uint32_t)p.seq_q * 4);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.delta + r_off, (uint32_t)p.seq_q * 4);
      // lanes 0-15 fetch the 64 row values; the others point past the buffer and write zeros
      // (the single-pass variant leaves them inactive, so only 256 bytes are written)
      const uint32_t off = lane < 16 ? (uint32_t)(qt * BQ + lane * 4) * 4 : 0x80000000u;
      if (!ATOMIC_DQ || lane < 16) {
        buffer_to_lds16(rl, ST == 0 ? l_st0 : l_st1, off);
        buffer_to_lds16(rd, ST == 0 ? d_st0 : d_st1, off);
      }
    }
  };

  // per-lane LDS offsets inside a 64-row Q/dO tile: row fragments of query block qb (rows
  // qb*32 + sigma32(c)) and transposed fragments (rows qb*32 + hh*16 + hc*8 + 0..7)
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = sigma32(c) * RB + (((2 * ks + hh) ^ swz<D>(sigma32(c))) * 16);
  int toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = hh * 16 + half * 4 + (i16 >> 2);
      const int d = db * 32 + dsub + 4 * (i16 & 3);
      toff[db][half] = row * RB + (((d >> 3) ^ swz<D>(row)) * 16) + (d & 7) * 2;
    }
  }

  // dense mask: bits of the step's queries q0 .. q0+63 for this lane's key and the step's query
  // head (0 past the key range), two words; loaded one step ahead of the step that tests them
  auto dcol_words = [&](int s, uint32_t (&w)[2]) __attribute__((always_inline)) {
    int g, qt;
    step_at(s, g, qt);
    const uint32_t* dcol = p.dense.cols + b * p.dense.cols_stride_b + (kvh * p.group + g) * p.dense.cols_stride_h +
                           (int64_t)min(my_k, p.seq_k - 1) * p.dense.col_words;
    dense_words(dcol, my_k < p.seq_k, p.dense.col_words, qt * BQ, w);
  };
  uint32_t dcur[2] = {0u, 0u}, dnext[2] = {0u, 0u};

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  const float cs = p.scale_log2;

  // One step: 64 queries in two 32-row blocks. For block qb, S = Q K^T and dP - Delta (the dP
  // accumulator starts at -Delta) are computed with this wave's 32 keys in the lane's column, then
  // P = exp2(scale log2(e) S - LSE log2(e)) and dS = P (dP - Delta), then dV += P^T dO and
  // dK += dS^T Q. The two blocks are software-pipelined so that the vector work of one block runs
  // under the MFMAs of the other: [S,dP 0] [S,dP 1 | P,dS 0] [dV,dK 0 | P,dS 1] [dV,dK 1].
  auto body = [&](auto stage_tag, auto masked_tag, int q0) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* ql = ST == 0 ? q_st0 : q_st1;
    const char* dol = ST == 0 ? o_st0 : o_st1;
    const float* lse_l = (const float*)(ST == 0 ? l_st0 : l_st1);
    const float* del_l = (const float*)(ST == 0 ? d_st0 : d_st1);

    // row statistics of the lane's 16 queries qb*32 + hh*16 + 0..15, in MFMA accumulator order
    auto stats = [&](int qb, f32x16& lse16, f32x16& nd16) __attribute__((always_inline)) {
      const int qbase = qb * 32 + hh * 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 l4 = *(const f32x4*)(lse_l + qbase + 4 * r);
        const f32x4 d4 = *(const f32x4*)(del_l + qbase + 4 * r);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lse16[4 * r + e] = l4[e];
          nd16[4 * r + e] = d4[e];
        }
      }
    };
    // S and dP - Delta of block qb; lane (c, hh) holds key my_k and queries qb*32 + hh*16 + i
    auto scores = [&](int qb, const f32x16& nd16, f32x16& sc, f32x16& dp) __attribute__((always_inline)) {
      bf16x8 qa[KS], oa[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qa[ks] = *(const bf16x8*)(ql + roff[ks] + qb * 32 * RB);
        oa[ks] = *(const bf16x8*)(dol + roff[ks] + qb * 32 * RB);
      }
      sc = f32x16{};
      dp = nd16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc = mfma32(qa[ks], kf[ks], sc);
        dp = mfma32(oa[ks], vf[ks], dp);
      }
    };
    // transposed dO and Q fragments of block qb (B operands of the dV and dK products)
    auto tr_frags = [&](int qb, bf16x8 (&ot)[2][DB], bf16x8 (&qt)[2][DB]) __attribute__((always_inline)) {
#pragma unroll
      for (int hc = 0; hc < 2; ++hc) {
        const int rows = (qb * 32 + hc * 8) * RB;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4 olo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, dol + toff[db][0] + rows));
          const i16x4 ohi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, dol + toff[db][1] + rows));
          const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, ql + toff[db][0] + rows));
          const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, ql + toff[db][1] + rows));
          ot[hc][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7));
          qt[hc][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
    };
    // P and dS of block qb in bf16 (A operands of the dV and dK products)
    auto probs = [&](int qb, const f32x16& sc, const f32x16& dp, const f32x16& lse16, bf16x8 (&pb)[2],
                     bf16x8 (&dsb)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = fast_exp2(fmaf(sc[i], cs, -lse16[i]));
        if constexpr (MASKED) {
          const int q = q0 + qb * 32 + hh * 16 + i;
          bool vis = q < q_len && my_k < kv_len;
          if constexpr (MASK == MASK_CAUSAL) vis = vis && my_k <= q;
          if constexpr (MASK == MASK_DENSE) vis = vis && ((dcur[qb] >> (hh * 16 + i)) & 1u);
          pv = vis ? pv : 0.0f;
        }
        pb[i >> 3][i & 7] = (bf16)pv;
        dsb[i >> 3][i & 7] = (bf16)(pv * dp[i]);
      }
    };
    // dV += P^T dO and dK += dS^T Q: rows = this wave's keys, contraction over the 32 queries
    auto grads = [&](const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2], const bf16x8 (&ot)[2][DB],
                     const bf16x8 (&qt)[2][DB]) __attribute__((always_inline)) {
#pragma unroll
      for (int hc = 0; hc < 2; ++hc) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = mfma32(pb[hc], ot[hc][db], dv[db]);
          dk[db] = mfma32(dsb[hc], qt[hc][db], dk[db]);
        }
      }
    };

    constexpr int NM = 2 * KS;   // MFMAs of scores(); grads() has 4 * DB
    f32x16 lse0, nd0, lse1, nd1, sc0, dp0, sc1, dp1;
    bf16x8 ot0[2][DB], qt0[2][DB], ot1[2][DB], qt1[2][DB];
    bf16x8 pb0[2], ds0[2], pb1[2], ds1[2];

    // [S,dP 0]: statistics first (the dP chain starts from -Delta), fragment reads two k-steps ahead
    stats(0, lse0, nd0);
    scores(0, nd0, sc0, dp0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8 + 4, 0);
#pragma unroll
    for (int m = 0; m < KS - 2; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

    // [S,dP 1 | P,dS 0]: block 1's statistics and fragments, block 0's transposed fragments
    stats(1, lse1, nd1);
    scores(1, nd1, sc1, dp1);
    tr_frags(0, ot0, qt0);
    probs(0, sc0, dp0, lse0, pb0, ds0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8 + 4, 0);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }

    // [dV,dK 0 | P,dS 1]: block 1's transposed fragments replace block 0's as they are consumed
    tr_frags(1, ot1, qt1);
    grads(pb0, ds0, ot0, qt0);
    probs(1, sc1, dp1, lse1, pb1, ds1);
#pragma unroll
    for (int m = 0; m < 4 * DB; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }

    // [dV,dK 1]
    grads(pb1, ds1, ot1, qt1);
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * DB, 0);
  };

  // ---- single-pass variant: K fragments along the key direction (B operand of dQ = dS K) ----
  // lane (c, hh) holds K[kw0 + kk*16 + hh*8 + e][db*32 + c], e = 0..7, read once per workgroup
  bf16x8 kcol[ATOMIC_DQ ? DB : 1][2];
  if constexpr (ATOMIC_DQ) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t off = ((uint32_t)(kw0 + kk * 16 + hh * 8 + e) * D + (uint32_t)(db * 32 + c)) * 2;
          kcol[db][kk][e] = __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(rk, off, 0, 0));
        }
      }
    }
  }

  // One step of the single-pass variant, one 32-query block at a time: the two-pass body's
  // products, then dQ_i += dS K_j for this wave's 32 keys, added to the fp32 accumulator.
  auto body_atomic = [&](auto stage_tag, auto masked_tag, int q0, int hq)
                         __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* ql = ST == 0 ? q_st0 : q_st1;
    const char* dol = ST == 0 ? o_st0 : o_st1;
    const float* lse_l = (const float*)(ST == 0 ? l_st0 : l_st1);
    const float* del_l = (const float*)(ST == 0 ? d_st0 : d_st1);
    char* dsl = ds_t + wave * 2048;
    float* dqa = p.dq_acc + ((size_t)(b * p.heads_q + hq) * p.seq_q) * D;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qbase = qb * 32 + hh * 16;
      f32x16 sc = f32x16{}, dp;
      f32x4 lse4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lse4[r] = *(const f32x4*)(lse_l + qbase + 4 * r);
        const f32x4 d4 = *(const f32x4*)(del_l + qbase + 4 * r);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * r + e] = d4[e];
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 qa = *(const bf16x8*)(ql + roff[ks] + qb * 32 * RB);
        const bf16x8 oa = *(const bf16x8*)(dol + roff[ks] + qb * 32 * RB);
        sc = mfma32(qa, kf[ks], sc);
        dp = mfma32(oa, vf[ks], dp);
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = fast_exp2(fmaf(sc[i], cs, -lse4[i >> 2][i & 3]));
        if constexpr (MASKED) {
          const int q = q0 + qbase + i;
          bool vis = q < q_len && my_k < kv_len;
          if constexpr (MASK == MASK_CAUSAL) vis = vis && my_k <= q;
          if constexpr (MASK == MASK_DENSE) vis = vis && ((dcur[qb] >> (hh * 16 + i)) & 1u);
          pv = vis ? pv : 0.0f;
        }
        pb[i >> 3][i & 7] = (bf16)pv;
        dsb[i >> 3][i & 7] = (bf16)(pv * dp[i]);
      }
      // dV += P^T dO, dK += dS^T Q
#pragma unroll
      for (int hc = 0; hc < 2; ++hc) {
        const int rows = (qb * 32 + hc * 8) * RB;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4 olo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, dol + toff[db][0] + rows));
          const i16x4 ohi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, dol + toff[db][1] + rows));
          const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, ql + toff[db][0] + rows));
          const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, ql + toff[db][1] + rows));
          dv[db] = mfma32(pb[hc], __builtin_bit_cast(bf16x8, __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7)), dv[db]);
          dk[db] = mfma32(dsb[hc], __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7)), dk[db]);
        }
      }
      // dS to this wave's LDS tile as [key][query] (lane (c, hh) holds key c, queries hh*16 + 0..15)
      *(bf16x8*)(dsl + c * 64 + (hh * 16) * 2) = dsb[0];
      *(bf16x8*)(dsl + c * 64 + (hh * 16 + 8) * 2) = dsb[1];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // A operand of dQ = dS K (rows = queries): lane l gets query l % 32 and keys kk*16 + (l/32)*8 + 0..7,
      // transposed reads of the [key][query] tile (16-lane group: query half (l/16)&1, key half l/32)
      bf16x8 dsa[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int row = kk * 16 + hh * 8 + (i16 >> 2);
        const int col = dsub + 4 * (i16 & 3);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, dsl + row * 64 + col * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, dsl + (row + 4) * 64 + col * 2));
        dsa[kk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      // the tile is rewritten by the next block: its reads complete before those writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // dQ rows q0 + qb*32 + (i/4)*8 + hh*4 + i%4, column db*32 + c: 32 consecutive floats per row
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x16 part = f32x16{};
        part = mfma32(dsa[0], kcol[db][0], part);
        part = mfma32(dsa[1], kcol[db][1], part);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = q0 + qb * 32 + (i >> 2) * 8 + hh * 4 + (i & 3);
          if (q < p.seq_q) unsafeAtomicAdd(dqa + (size_t)q * D + db * 32 + c, part[i]);
        }
      }
    }
  };

  auto step = [&](auto stage_tag, auto masked_tag, int s) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    wait_vmem();
    __syncthreads();
    if (s + 1 < n_steps) issue_step(std::integral_constant<int, 1 - ST>{}, s + 1);
    int g, qt;
    step_at(s, g, qt);
    const int q0 = qt * BQ;
    if constexpr (MASK == MASK_DENSE) {
      dcur[0] = dnext[0];
      dcur[1] = dnext[1];
      if (s + 1 < n_steps) dcol_words(s + 1, dnext);
    }
    auto run_body = [&]() __attribute__((always_inline)) {
      if constexpr (ATOMIC_DQ) body_atomic(stage_tag, masked_tag, q0, kvh * p.group + g);
      else body(stage_tag, masked_tag, q0);
    };
    if constexpr (!MASKED) {
      run_body();
    } else {
      bool active = kw0 < kv_len;
      if constexpr (MASK == MASK_CAUSAL) active = active && kw0 <= q0 + BQ - 1;
      if constexpr (MASK == MASK_PADDING) active = active && q0 < q_len;
      if (active) run_body();
    }
  };
  auto run = [&](auto masked_tag, int s0, int s1) __attribute__((always_inline)) {
    int s = s0;
    if (s < s1 && (s & 1)) step(std::integral_constant<int, 1>{}, masked_tag, s++);
    for (; s + 1 < s1; s += 2) {
      step(std::integral_constant<int, 0>{}, masked_tag, s);
      step(std::integral_constant<int, 1>{}, masked_tag, s + 1);
    }
    if (s < s1) step(std::integral_constant<int, 0>{}, masked_tag, s);
  };

  if constexpr (MASK == MASK_DENSE)
    if (n_steps > 0) dcol_words(0, dnext);
  if (n_steps > 0) issue_step(std::integral_constant<int, 0>{}, 0);
  run(std::false_type{}, 0, n_free);
  run(std::true_type{}, n_free, n_steps);

  // ---- write dK (times scale) and dV; lane (c, hh) holds column db*32 + c of keys kw0 + row ----
  bf16* dkg = (bf16*)p.dk + kv_off;
  bf16* dvg = (bf16*)p.dv + kv_off;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw0 + (i >> 2) * 8 + hh * 4 + (i & 3);
      if (key < p.seq_k) {
        dkg[(size_t)key * D + db * 32 + c] = (bf16)(dk[db][i] * p.scale);
        dvg[(size_t)key * D + db * 32 + c] = (bf16)dv[db][i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// dK/dV pass with wave pairs (two-pass mode). One workgroup per 64-key tile, four waves: two pairs
// of 32 keys. A step is one 64-row query tile of one query head of the group, two blocks of 32
// queries. Wave r of a pair owns query block r of every step: it computes S = Q K^T (accumulator
// seeded with -LSE / scale, so P = exp2(scale log2(e) acc)) and dP - Delta = dO V^T (seeded with
// -Delta) for its block, then P and dS = P (dP - Delta). Wave 0 accumulates dV += P^T dO, wave 1
// dK += dS^T Q: each adds its own block at once and, after one exchange barrier, the partner's,
// which the partner hands over in bf16 through LDS (dS of block 0 to wave 1, P of block 1 to
// wave 0; 4 KiB per pair). Each wave holds K and V fragments and one accumulator, so two waves
// share each SIMD and cover each other's latencies; no product is computed twice, and each wave
// runs half of the step's exponentials. A step: copy barrier, scores, exponentials, own-block
// product, exchange barrier, partner-block product.
constexpr int PAIR_LEAD = 4;   // k-steps of row-fragment reads in flight ahead of the score MFMAs
constexpr int PAIR_PRIO_MIN_STEPS = 32;   // steps per item from which the hand-over runs at raised priority

template <int D>
struct PairLds {
  static constexpr int TILE = BQ * D * 2;
  static constexpr int STATS = 256;          // 64 row values
  static constexpr int XCH = 4096;           // one pair's hand-over: [dS0 | P1][half][lane] x 16 bytes
  static constexpr int MAX_STEPS = 2048;     // listed (query head, layout row) pairs for block masks
};

template <int D, int MASK, int MINW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MINW))) void bwd_dkdv_pair_kernel(BwdParams p) {
  constexpr int NW = 4;
  constexpr int BK = 64;        // keys per workgroup
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RB = D * 2;
  using L = PairLds<D>;
  __shared__ __attribute__((aligned(16))) char q_st0[L::TILE];
  __shared__ __attribute__((aligned(16))) char o_st0[L::TILE];   // dO
  __shared__ __attribute__((aligned(16))) char q_st1[L::TILE];
  __shared__ __attribute__((aligned(16))) char o_st1[L::TILE];
  __shared__ __attribute__((aligned(16))) char s_st0[L::STATS];  // -LSE / scale
  __shared__ __attribute__((aligned(16))) char d_st0[L::STATS];  // -Delta
  __shared__ __attribute__((aligned(16))) char s_st1[L::STATS];
  __shared__ __attribute__((aligned(16))) char d_st1[L::STATS];
  __shared__ __attribute__((aligned(16))) char xch[2 * L::XCH];
  constexpr bool LISTED = MASK == MASK_BLOCK || MASK == MASK_DENSE;
  __shared__ uint16_t list[LISTED ? L::MAX_STEPS : 1];
  __shared__ int list_count;

  __shared__ int simd_of[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hh = lane >> 5;
  const int dsub = ((lane >> 4) & 1) * 16, i16 = lane & 15;

  // Pair and role of this wave. A CU holds two of these workgroups (workgroup slots 0 and 1), and
  // the four waves of each spread over the four SIMDs. Ranking the waves by SIMD and flipping the
  // role with the slot's parity puts one wave of each role on every SIMD. Any placement gives a
  // valid assignment: the ranks are a permutation, and each pair gets one wave of each role.
  const uint32_t hw_id = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_REG_HW_ID
  const int my_simd = (int)((hw_id >> 4) & 3), slot = (int)((hw_id >> 16) & 1);
  if (lane == 0) simd_of[wave] = my_simd;
  lds_barrier();
  int rank = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int sw = simd_of[w];
    rank += (sw < my_simd || (sw == my_simd && w < wave)) ? 1 : 0;
  }
  rank = __builtin_amdgcn_readfirstlane(rank);
  const int pair = rank >> 1, role = (rank & 1) ^ slot;   // role r: query block r, then dV (0) or dK (1)

  const uint32_t item = p.items_kv[blockIdx.x];
  // an item outside the problem (a list the caller kept from another call) does nothing
  if ((uint64_t)item >= (uint64_t)p.batch * p.heads_kv * p.n_ktiles) return;
  const int kt = (int)(item % (uint32_t)p.n_ktiles);
  const int bkv = (int)(item / (uint32_t)p.n_ktiles);
  const int kvh = bkv % p.heads_kv, b = bkv / p.heads_kv;
  const int k0 = kt * BK;
  const int kp0 = k0 + pair * 32;   // this pair's keys
  const int my_k = kp0 + c;

  const size_t kv_off = ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const bf16*)p.k + kv_off, (uint32_t)p.seq_k * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16*)p.v + kv_off, (uint32_t)p.seq_k * RB);
  bf16x8 kfrag[KS], vfrag[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)my_k * RB + (uint32_t)(ks * 32 + hh * 16);
    kfrag[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    vfrag[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
  }

  // ---- the (query head, query tile) steps that see this key tile ----
  int kv_len = p.seq_k, q_len = p.seq_q;
  const int n_qt = (p.seq_q + BQ - 1) / BQ;
  int qt_lo = 0, qt_hi = n_qt;
  if constexpr (MASK == MASK_PADDING) {
    kv_len = clamp_len(p.lengths[b], p.seq_k);
    q_len = clamp_len(p.lengths[b], p.seq_q);
    qt_hi = (k0 < kv_len) ? (q_len + BQ - 1) / BQ : 0;
  } else if constexpr (MASK == MASK_CAUSAL) {
    qt_lo = k0 / BQ;
  }
  const bool key_tail = k0 + BK > kv_len;    // some key of the tile is past the end
  // query tiles [qt_m, qt_f) need no mask; [qt_lo, qt_m) (causal diagonal) and the ragged last
  // tile [qt_f, qt_hi) do
  int qt_m = qt_lo, qt_f = qt_hi;
  if constexpr (MASK == MASK_CAUSAL) qt_m = min(qt_hi, max(qt_lo, (k0 + BK - 2) / BQ + 1));
  if (qt_hi > qt_m && (qt_hi * BQ > q_len)) qt_f = qt_hi - 1;
  if (key_tail) qt_f = qt_m;                 // every step masked
  qt_f = max(qt_f, qt_m);
  int n_free, n_steps;
  if constexpr (LISTED) {
    const int col = k0 / 64;
    if (wave == 0) {
      int count = 0;
      for (int g = 0; g < p.group; ++g) {
        const uint8_t* lay = p.layout + b * p.layout_stride_b + (kvh * p.group + g) * p.layout_stride_h;
        for (int r0 = 0; r0 < p.nb_q; r0 += 64) {
          const int r = r0 + lane;
          const bool keep = r < p.nb_q && lay[(size_t)r * p.nb_k + col] != 0;
          const uint64_t ball = __ballot(keep);
          const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(ball >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ball, 0));
          if (keep && count + before < L::MAX_STEPS) list[count + before] = (uint16_t)((g << 10) | r);
          count += __popcll(ball);
        }
      }
      if (lane == 0) list_count = min(count, L::MAX_STEPS);
    }
    lds_barrier();   // the fragment loads issued above stay in flight
    n_steps = list_count;
    // ragged shapes run every step through the masked body, and so does a dense mask
    n_free = (MASK == MASK_DENSE || key_tail || (p.seq_q % BQ) != 0) ? 0 : n_steps;
  } else {
    n_free = p.group * (qt_f - qt_m);
    n_steps = p.group * (qt_hi - qt_lo);
  }
  auto step_at = [&](int s, int& g, int& qt) __attribute__((always_inline)) {
    if constexpr (LISTED) {
      const uint32_t e = list[s];
      g = (int)(e >> 10);
      qt = (int)(e & 1023u);
    } else {
      if (s < n_free) {
        const int per = qt_f - qt_m;
        g = s / per;
        qt = qt_m + s % per;
      } else {
        const int r = s - n_free;
        const int per = (qt_m - qt_lo) + (qt_hi - qt_f);
        g = r / per;
        const int m = r % per;
        qt = m < qt_m - qt_lo ? qt_lo + m : qt_f + (m - (qt_m - qt_lo));
      }
    }
  };

  auto issue_step = [&](auto stage_tag, int s) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    int g, qt;
    step_at(s, g, qt);
    const int hq = kvh * p.group + g;
    const size_t q_off = ((size_t)(b * p.heads_q + hq) * p.seq_q) * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const bf16*)p.q + q_off, (uint32_t)p.seq_q * RB);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const bf16*)p.dout + q_off, (uint32_t)p.seq_q * RB);
    issue_rows<D, NW>(ST == 0 ? q_st0 : q_st1, rq, qt * BQ, wave, lane);
    issue_rows<D, NW>(ST == 0 ? o_st0 : o_st1, rdo, qt * BQ, wave, lane);
    if (wave == 0 && lane < 16) {
      // 64 row values; rows past the sequence read as 0 (their steps run the masked body)
      const size_t r_off = (size_t)(b * p.heads_q + hq) * p.seq_q;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.sseed + r_off, (uint32_t)p.seq_q * 4);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.delta + r_off, (uint32_t)p.seq_q * 4);
      const uint32_t off = (uint32_t)(qt * BQ + lane * 4) * 4;
      buffer_to_lds16(rs, ST == 0 ? s_st0 : s_st1, off);
      buffer_to_lds16(rd, ST == 0 ? d_st0 : d_st1, off);
    }
  };

  // per-lane LDS offsets inside a 64-row Q/dO tile: row fragments of query block qb (rows
  // qb*32 + sigma32(c)) and transposed fragments (rows qb*32 + hh*16 + hc*8 + 0..7)
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = sigma32(c) * RB + (((2 * ks + hh) ^ swz<D>(sigma32(c))) * 16);
  int toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = hh * 16 + half * 4 + (i16 >> 2);
      const int d = db * 32 + dsub + 4 * (i16 & 3);
      toff[db][half] = row * RB + (((d >> 3) ^ swz<D>(row)) * 16) + (d & 7) * 2;
    }
  }
  // this pair's hand-over tile (dS of block 0 at +0, P of block 1 at +2048); lane-linear 16-byte
  // chunks, so writes and reads are conflict free
  char* xp = xch + pair * L::XCH + lane * 16;

  // dense mask: bits of the queries q0 + qoff .. q0 + qoff + 31 of step s (this wave's query block)
  // for this lane's key and the step's query head (0 past the key range), in w[0]; loaded one step
  // ahead of the step that tests them
  auto dcol_words = [&](int s, int qoff, uint32_t (&w)[2]) __attribute__((always_inline)) {
    int g, qt;
    step_at(s, g, qt);
    const uint32_t* dcol = p.dense.cols + b * p.dense.cols_stride_b + (kvh * p.group + g) * p.dense.cols_stride_h +
                           (int64_t)min(my_k, p.seq_k - 1) * p.dense.col_words;
    dense_words(dcol, my_k < p.seq_k, p.dense.col_words, qt * BQ + qoff, w);
  };

  f32x16 acc[DB];   // dV (role 0) or dK / scale (role 1) of this pair's 32 keys
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  const float cs = p.scale_log2;

  // 16 row values of query block qb in MFMA accumulator order (queries qb*32 + hh*16 + 0..15)
  auto stats16 = [&](const char* st, int qb) __attribute__((always_inline)) -> f32x16 {
    f32x16 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 v = *(const f32x4*)(st + (qb * 32 + hh * 16 + 4 * k) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) r[4 * k + e] = v[e];
    }
    return r;
  };
  // S (seeded with -LSE / scale) and dP - Delta (seeded with -Delta) of query block QB, as two
  // interleaved MFMA chains over the Q and dO rows of the block. The row-fragment reads run
  // PAIR_LEAD k-steps ahead of the MFMAs that consume them (order pinned with
  // sched_group_barrier; masks 0x100 LDS read, 0x008 MFMA).
  auto scores = [&](auto qb_tag, const char* qtile, const char* otile, const char* sst, const char* dst, f32x16& sa,
                    f32x16& da) __attribute__((always_inline)) {
    constexpr int QB = decltype(qb_tag)::value;
    sa = stats16(sst, QB);
    da = stats16(dst, QB);
    bf16x8 xq[KS], xo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      xq[ks] = *(const bf16x8*)(qtile + roff[ks] + QB * 32 * RB);
      xo[ks] = *(const bf16x8*)(otile + roff[ks] + QB * 32 * RB);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sa = mfma32(xq[ks], kfrag[ks], sa);
      da = mfma32(xo[ks], vfrag[ks], da);
    }
    constexpr int KL = PAIR_LEAD < KS ? PAIR_LEAD : KS;
    __builtin_amdgcn_sched_group_barrier(0x100, 8 + 2 * KL, 0);   // the 8 seed reads, KL k-steps
#pragma unroll
    for (int ks = 0; ks < KS - KL; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * KL, 0);
  };
  // transposed fragments of `tile` for query block qb (rows qb*32 + hh*16 + hc*8 + 0..7): the B
  // operands of acc += A^T B. The tile does not change during a step, so a wave issues these reads
  // before it waits at an exchange barrier and the barrier's wait covers their latency.
  auto load_t = [&](const char* tile, int qb, bf16x8 (&t)[2][DB]) __attribute__((always_inline)) {
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      const int rows = (qb * 32 + hc * 8) * RB;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, tile + toff[db][0] + rows));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, tile + toff[db][1] + rows));
        t[hc][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };
  // acc += A^T B over the 32 queries of one block: A = this lane's bf16 operand of chunk hc
  auto grads = [&](const bf16x8 (&a)[2], const bf16x8 (&t)[2][DB]) __attribute__((always_inline)) {
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = mfma32(a[hc], t[hc][db], acc[db]);
    }
  };

  uint32_t dcur[2] = {0u, 0u}, dnext[2] = {0u, 0u};

  // One step of wave ROLE of a pair. Every wave passes both barriers of
  // every step; a pair whose keys see none of the step's queries skips its products.
  auto step = [&](auto role_tag, auto stage_tag, auto masked_tag, int s) __attribute__((always_inline)) {
    constexpr int ROLE = decltype(role_tag)::value;
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* ql = ST == 0 ? q_st0 : q_st1;
    const char* dol = ST == 0 ? o_st0 : o_st1;
    wait_vmem();
    __syncthreads();   // step s is in LDS; every wave is done with the stage step s+1 overwrites
    if (s + 1 < n_steps) issue_step(std::integral_constant<int, 1 - ST>{}, s + 1);
    int g, qt;
    step_at(s, g, qt);
    const int q0 = qt * BQ;
    if constexpr (MASK == MASK_DENSE) {
      dcur[0] = dnext[0];
      if (s + 1 < n_steps) dcol_words(s + 1, ROLE * 32, dnext);
    }
    bool active = true;
    if constexpr (MASKED) {
      active = kp0 < kv_len;
      if constexpr (MASK == MASK_CAUSAL) active = active && kp0 <= q0 + BQ - 1;
      if constexpr (MASK == MASK_PADDING) active = active && q0 < q_len;
    }
    // Wave ROLE owns query block QB = ROLE of the step: its S, P, dP - Delta and dS. It adds its
    // own block's product to its accumulator (dV += P0^T dO0 for ROLE 0, dK += dS1^T Q1 for
    // ROLE 1), hands its partner the operand the partner accumulates (dS0 to ROLE 1, P1 to
    // ROLE 0) through LDS, and after one barrier adds the partner's block.
    constexpr int QB = ROLE;
    const char* tt = ROLE == 0 ? dol : ql;   // transposed operand: dO (dV) or Q (dK)
    bf16x8 t_own[2][DB], t_other[2][DB];
    if (active) {
      // what the partner waits for goes first at the instruction arbiter on long items (on items
      // of a few steps this measured slower, so they do not)
      if (n_steps >= PAIR_PRIO_MIN_STEPS) __builtin_amdgcn_s_setprio(2);
      f32x16 sc, dp;
      scores(std::integral_constant<int, QB>{}, ql, dol, ST == 0 ? s_st0 : s_st1, ST == 0 ? d_st0 : d_st1, sc, dp);
      load_t(tt, QB, t_own);
      float pv[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = fast_exp2(sc[i] * cs);
        if constexpr (MASKED) {
          const int q = q0 + QB * 32 + hh * 16 + i;
          bool vis = q < q_len && my_k < kv_len;
          if constexpr (MASK == MASK_CAUSAL) vis = vis && my_k <= q;
          if constexpr (MASK == MASK_DENSE) vis = vis && ((dcur[0] >> (hh * 16 + i)) & 1u);
          pv[i] = vis ? pv[i] : 0.0f;
        }
        ds[i] = pv[i] * dp[i];
      }
      const bf16x8 pb[2] = {pack_bf16x8(pv), pack_bf16x8(pv + 8)};
      const bf16x8 db[2] = {pack_bf16x8(ds), pack_bf16x8(ds + 8)};
      if constexpr (ROLE == 0) {
        *(bf16x8*)(xp) = db[0];
        *(bf16x8*)(xp + 1024) = db[1];
        __builtin_amdgcn_s_setprio(0);
        grads(pb, t_own);   // dV += P0^T dO0
      } else {
        *(bf16x8*)(xp + 2048) = pb[0];
        *(bf16x8*)(xp + 3072) = pb[1];
        __builtin_amdgcn_s_setprio(0);
        grads(db, t_own);   // dK += dS1^T Q1
      }
      load_t(tt, 1 - QB, t_other);
    }
    lds_barrier();   // the partner's operand is in LDS
    if (active) {
      const char* src = xp + (1 - ROLE) * 2048;
      const bf16x8 got[2] = {*(const bf16x8*)src, *(const bf16x8*)(src + 1024)};
      grads(got, t_other);   // dV += P1^T dO1 (ROLE 0) or dK += dS0^T Q0 (ROLE 1)
    }
  };
  auto run_role = [&](auto role_tag) __attribute__((always_inline)) {
    auto run = [&](auto masked_tag, int s0, int s1) __attribute__((always_inline)) {
      int s = s0;
      if (s < s1 && (s & 1)) step(role_tag, std::integral_constant<int, 1>{}, masked_tag, s++);
      for (; s + 1 < s1; s += 2) {
        step(role_tag, std::integral_constant<int, 0>{}, masked_tag, s);
        step(role_tag, std::integral_constant<int, 1>{}, masked_tag, s + 1);
      }
      if (s < s1) step(role_tag, std::integral_constant<int, 0>{}, masked_tag, s);
    };
    run(std::false_type{}, 0, n_free);
    run(std::true_type{}, n_free, n_steps);
  };

  if constexpr (MASK == MASK_DENSE)
    if (n_steps > 0) dcol_words(0, role * 32, dnext);
  if (n_steps > 0) issue_step(std::integral_constant<int, 0>{}, 0);
  if (role == 0) run_role(std::integral_constant<int, 0>{});
  else run_role(std::integral_constant<int, 1>{});

  // ---- write dV (role 0) or dK = scale * acc (role 1); lane (c, hh) holds column db*32 + c of
  // keys kp0 + (i / 4) * 8 + hh * 4 + i % 4. Each wave stages its 32 rows in bf16 through LDS (the
  // Q/dO stage buffers, free once every wave has passed the last step) and writes whole rows with
  // 16-byte stores. ----
  bf16* out = (bf16*)(role == 0 ? p.dv : p.dk) + kv_off;
  const float f = role == 0 ? 1.0f : p.scale;
  __syncthreads();   // every wave is done with the last step's tiles
  char* rows_lds = (wave < 2 ? q_st0 : q_st1) + (wave & 1) * (32 * RB);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = (i >> 2) * 8 + hh * 4 + (i & 3);
      *(bf16*)(rows_lds + r * RB + (db * 32 + c) * 2) = (bf16)(acc[db][i] * f);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's own rows are in LDS
  constexpr int CPR = RB / 16;                          // 16-byte chunks per row
#pragma unroll
  for (int j = 0; j < 32 * CPR / 64; ++j) {
    const int chunk = j * 64 + lane;
    const int r = chunk / CPR, cc = chunk % CPR;
    const uint4 v = *(const uint4*)(rows_lds + r * RB + cc * 16);
    if (kp0 + r < p.seq_k) *(uint4*)(out + (size_t)(kp0 + r) * D + cc * 8) = v;
  }
}

// ------------------------------------------------------------------------------------------------
// dQ pass: same tile loop as the forward kernel (K and V tiles double-buffered in four separately
// named LDS arrays, per-lane precomputed swizzled offsets, mask-free tiles in their own loop).
template <int D>
struct QLds {
  static constexpr int TILE = BN * D * 2;
  static constexpr int MAX_LIST = 1024;
};

template <int D, int NW, int MASK, int MINW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(MINW))) void bwd_dq_kernel(BwdParams p) {
  constexpr int BM = NW * 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int RB = D * 2;
  using L = QLds<D>;
  __shared__ __attribute__((aligned(16))) char k_st0[L::TILE];
  __shared__ __attribute__((aligned(16))) char v_st0[L::TILE];
  __shared__ __attribute__((aligned(16))) char k_st1[L::TILE];
  __shared__ __attribute__((aligned(16))) char v_st1[L::TILE];
  constexpr bool LISTED = MASK == MASK_BLOCK || MASK == MASK_DENSE;
  __shared__ uint32_t list[LISTED ? L::MAX_LIST + 1 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hh = lane >> 5;
  const int dsub = ((lane >> 4) & 1) * 16, i16 = lane & 15;

  const uint32_t item = p.items_q[blockIdx.x];
  // an item outside the problem (a list the caller kept from another call) does nothing
  if ((uint64_t)item >= (uint64_t)p.batch * p.heads_q * p.n_qtiles) return;
  const Item it = decode_item(item, p.heads_q, p.n_qtiles);
  const int b = it.b, h = it.h, kvh = h / p.group;
  const int q0 = it.t * BM;
  // the 32 query rows of this wave: waves 0-1 cover the tile's first layout row, 2-3 its second
  // (under a block layout, the two rows the planner paired for the tile)
  const int qw0 = (MASK == MASK_BLOCK && BM == 128) ? tile_row(p.row_pairs, it.t, wave >> 1) * 64 + (wave & 1) * 32
                                                    : q0 + wave * 32;
  const int my_q = qw0 + c;

  const size_t q_off = ((size_t)(b * p.heads_q + h) * p.seq_q) * D;
  const size_t kv_off = ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const bf16*)p.q + q_off, (uint32_t)p.seq_q * RB);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const bf16*)p.dout + q_off, (uint32_t)p.seq_q * RB);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const bf16*)p.k + kv_off, (uint32_t)p.seq_k * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16*)p.v + kv_off, (uint32_t)p.seq_k * RB);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc((const bf16*)p.o + q_off, (uint32_t)p.seq_q * RB);

  // Q and dO rows of this lane's query (B operands of S^T = K Q^T and dP^T = V dO^T), and its O
  // row for the row statistics below; issued before the key-tile list so that they overlap it
  bf16x8 qf[KS], dof[KS], of8[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)my_q * RB + (uint32_t)(ks * 32 + hh * 16);
    qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    dof[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0));
    of8[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
  }

  int kv_len = p.seq_k, q_len = p.seq_q;
  int n_tiles;
  if constexpr (MASK == MASK_PADDING) {
    kv_len = clamp_len(p.lengths[b], p.seq_k);
    q_len = clamp_len(p.lengths[b], p.seq_q);
    n_tiles = (q0 < q_len) ? (kv_len + BN - 1) / BN : 0;
  } else if constexpr (MASK == MASK_CAUSAL) {
    n_tiles = min((p.seq_k + BN - 1) / BN, (min(q0 + BM, p.seq_q) - 1) / BN + 1);
  } else if constexpr (LISTED) {
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
      if (lane == 0) list[L::MAX_LIST] = (uint32_t)count;
    }
    lds_barrier();   // the row loads issued above stay in flight
    n_tiles = (int)list[L::MAX_LIST];
  } else {
    n_tiles = (p.seq_k + BN - 1) / BN;
  }

  const size_t row_off = (size_t)(b * p.heads_q + h) * p.seq_q;
  const uint32_t* dense_row = MASK == MASK_DENSE
      ? p.dense.rows + b * p.dense.rows_stride_b + h * p.dense.rows_stride_h + (int64_t)my_q * p.dense.row_words
      : nullptr;
  // The backward's row statistics of this workgroup's queries, computed here rather than by a
  // preprocess kernel: -Delta = -rowsum(dO * O) in fp32 (the lane and its partner lane c + 32 hold
  // the two halves of the row) and LSE in the log2 domain. The dK/dV pass, launched after this
  // one, reads them from the workspace.
  float dsum = 0.0f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = fmaf((float)of8[ks][e], (float)dof[ks][e], dsum);
  }
  dsum = partner_sum(dsum);
  const bool row_ok = my_q < p.seq_q;
  const float lse2 = row_ok ? lse_to_log2(p.lse[row_off + my_q]) : INFINITY;
  const float ndelta = row_ok ? -dsum : 0.0f;   // -Delta
  const float sseed = -lse2 * p.inv_scale_log2;  // -LSE / scale; -inf for empty rows and rows past the end
  if (row_ok && hh == 0) {
    p.delta[row_off + my_q] = ndelta;
    p.lse2[row_off + my_q] = lse2;
    // the wave-pair dK/dV pass starts its score accumulator at -LSE / scale (-inf for empty rows)
    if (p.sseed != nullptr) p.sseed[row_off + my_q] = sseed;
  }

  // per-lane LDS offsets: row fragments (K and V tiles share the layout) and transposed K reads
  int roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) roff[ks] = sigma32(c) * RB + (((2 * ks + hh) ^ swz<D>(sigma32(c))) * 16);
  int toff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int row = hh * 16 + half * 4 + (i16 >> 2);
      const int d = db * 32 + dsub + 4 * (i16 & 3);
      toff[db][half] = row * RB + (((d >> 3) ^ swz<D>(row)) * 16) + (d & 7) * 2;
    }
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
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

  // One 64-key tile, processed as two 32-key halves: S^T and dP^T of the half, then dS, then the
  // dQ^T += K^T dS^T contributions of its two 16-key chunks.
  auto tile = [&](auto stage_tag, auto masked_tag, int k0) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* kl = ST == 0 ? k_st0 : k_st1;
    const char* vl = ST == 0 ? v_st0 : v_st1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // the score accumulator starts at -LSE / scale and the dP one at -Delta, so that
      // P = exp2(scale log2(e) acc) and dS = P acc need no per-element offset
      f32x16 sc, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[i] = sseed;
        dp[i] = ndelta;
      }
      bf16x8 ka[KS], va[KS];
      uint32_t dw = 0;
      if constexpr (MASK == MASK_DENSE) {
        const int w = (k0 >> 5) + kb;
        if (my_q < p.seq_q && w < p.dense.row_words) dw = dense_row[w];
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        ka[ks] = *(const bf16x8*)(kl + roff[ks] + kb * 32 * RB);
        va[ks] = *(const bf16x8*)(vl + roff[ks] + kb * 32 * RB);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc = mfma32(ka[ks], qf[ks], sc);
        dp = mfma32(va[ks], dof[ks], dp);
      }
      // K and V reads run DL k-steps ahead of the MFMAs: two under the structured masks (1% faster
      // there), one for the listed masks (as fast on a block layout, and a dense mask's extra
      // registers would spill)
      constexpr int DL = LISTED ? 1 : 2;
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * DL, 0);
#pragma unroll
      for (int ks = 0; ks < KS - 2 * DL; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * DL, 0);

      // transposed K fragments for this half's two chunks go out before the element-wise work
      bf16x8 kt[2][DB];
#pragma unroll
      for (int hc = 0; hc < 2; ++hc) {
        const int rows = (kb * 32 + hc * 8) * RB;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, kl + toff[db][0] + rows));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, kl + toff[db][1] + rows));
          kt[hc][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      }
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = fast_exp2(sc[i] * cs);
        if constexpr (MASKED) {
          const int key = k0 + kb * 32 + hh * 16 + i;
          bool vis = key < kv_len && my_q < q_len;
          if constexpr (MASK == MASK_CAUSAL) vis = vis && key <= my_q;
          if constexpr (MASK == MASK_DENSE) vis = vis && ((dw >> (hh * 16 + i)) & 1u);
          pv = vis ? pv : 0.0f;
        }
        ds[i] = pv * dp[i];
      }
      const bf16x8 dsb[2] = {pack_bf16x8(ds), pack_bf16x8(ds + 8)};
#pragma unroll
      for (int hc = 0; hc < 2; ++hc) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma32(kt[hc][db], dsb[hc], acc[db]);
      }
    }
  };

  int n_free;
  if constexpr (MASK == MASK_CAUSAL) {
    n_free = min(q0 / BN, p.seq_k / BN);
  } else if constexpr (MASK == MASK_PADDING) {
    n_free = (q0 + BM <= q_len) ? kv_len / BN : 0;
  } else if constexpr (MASK == MASK_BLOCK) {
    n_free = (n_tiles > 0 && tile_index(n_tiles - 1) * BN + BN > p.seq_k) ? n_tiles - 1 : n_tiles;
  } else if constexpr (MASK == MASK_DENSE) {
    n_free = 0;   // every kept tile is tested pair by pair
  } else {
    n_free = p.seq_k / BN;
  }
  n_free = min(n_free, n_tiles);

  auto step = [&](auto stage_tag, auto masked_tag, int j) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    wait_vmem();
    __syncthreads();
    if (j + 1 < n_tiles) issue_tile(std::integral_constant<int, 1 - ST>{}, tile_index(j + 1));
    const int k0 = tile_index(j) * BN;
    if constexpr (!MASKED) {
      bool active = true;
      if constexpr (LISTED && BM > 64) active = ((list[j] >> 16) >> ((wave * 32) / 64)) & 1u;
      if (active) tile(stage_tag, masked_tag, k0);
    } else {
      bool active = k0 < kv_len;
      if constexpr (MASK == MASK_CAUSAL) active = active && k0 <= qw0 + 31;
      if constexpr (MASK == MASK_PADDING) active = active && qw0 < q_len;
      if constexpr (LISTED) active = ((list[j] >> 16) >> ((wave * 32) / 64)) & 1u;
      if (active) tile(stage_tag, masked_tag, k0);
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

  if (n_tiles > 0) issue_tile(std::integral_constant<int, 0>{}, tile_index(0));
  run(std::false_type{}, 0, n_free);
  run(std::true_type{}, n_free, n_tiles);

  // dQ as whole rows, staged in one of the four K/V stage arrays per wave (free once every wave has
  // passed the last tile)
  static_assert(NW <= 4 && 32 * (RB + 8) <= L::TILE, "one stage array per wave");
  __syncthreads();
  char* rows_lds = wave == 0 ? k_st0 : wave == 1 ? v_st0 : wave == 2 ? k_st1 : v_st1;
  write_rows_bf16<D>(rows_lds, acc, p.scale, lane, (bf16*)p.dq + q_off + (size_t)qw0 * D, p.seq_q - qw0);
}

// ------------------------------------------------------------------------------------------------
template <int D, int NW, int MASK, bool ATOMIC_DQ = false>
hipError_t launch_dkdv_one(const BwdParams& p, int n_items, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, MASK, ATOMIC_DQ>), dim3(n_items), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

template <int D, int NW, int MASK, int MINW>
hipError_t launch_dq_one(const BwdParams& p, int n_items, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dq_kernel<D, NW, MASK, MINW>), dim3(n_items), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

template <int D, int MASK>
hipError_t launch_pair_one(const BwdParams& p, int n_items, hipStream_t s) {
  hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, MASK, 2>), dim3(n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t dkdv_pair_mask(const BwdParams& p, int mask, int n_items, hipStream_t s) {
  switch (mask) {
    case MASK_NONE: return launch_pair_one<D, MASK_NONE>(p, n_items, s);
    case MASK_CAUSAL: return launch_pair_one<D, MASK_CAUSAL>(p, n_items, s);
    case MASK_PADDING: return launch_pair_one<D, MASK_PADDING>(p, n_items, s);
    case MASK_DENSE: return launch_pair_one<D, MASK_DENSE>(p, n_items, s);
    default: return launch_pair_one<D, MASK_BLOCK>(p, n_items, s);
  }
}

template <int D>
hipError_t dkdv_mask(const BwdParams& p, int mask, int n_items, hipStream_t s) {
  if (p.dq_acc != nullptr) {
    switch (mask) {
      case MASK_NONE: return launch_dkdv_one<D, 4, MASK_NONE, true>(p, n_items, s);
      case MASK_CAUSAL: return launch_dkdv_one<D, 4, MASK_CAUSAL, true>(p, n_items, s);
      case MASK_PADDING: return launch_dkdv_one<D, 4, MASK_PADDING, true>(p, n_items, s);
      case MASK_DENSE: return launch_dkdv_one<D, 2, MASK_DENSE, true>(p, n_items, s);
      default: return launch_dkdv_one<D, 2, MASK_BLOCK, true>(p, n_items, s);
    }
  }
  switch (mask) {
    case MASK_NONE: return launch_dkdv_one<D, 4, MASK_NONE>(p, n_items, s);
    case MASK_CAUSAL: return launch_dkdv_one<D, 4, MASK_CAUSAL>(p, n_items, s);
    case MASK_PADDING: return launch_dkdv_one<D, 4, MASK_PADDING>(p, n_items, s);
    case MASK_DENSE: return launch_dkdv_one<D, 2, MASK_DENSE>(p, n_items, s);
    default: return launch_dkdv_one<D, 2, MASK_BLOCK>(p, n_items, s);
  }
}

// Single-pass mode: dQ = scale * (accumulated dS K), rounded to bf16; D/4 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(BwdParams p, int64_t rows) {
  constexpr int LPR = D / 4;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int col = (threadIdx.x % LPR) * 4;
  if (row >= rows) return;
  const f32x4 a = *(const f32x4*)(p.dq_acc + row * D + col);
  bf16x4 v4;
#pragma unroll
  for (int e = 0; e < 4; ++e) v4[e] = (bf16)(a[e] * p.scale);
  *(bf16x4*)((bf16*)p.dq + row * D + col) = v4;
}

template <int D>
hipError_t dq_mask(const BwdParams& p, int mask, int n_items, hipStream_t s) {
  switch (mask) {
    case MASK_NONE: return launch_dq_one<D, 4, MASK_NONE, 2>(p, n_items, s);
    case MASK_CAUSAL: return launch_dq_one<D, 4, MASK_CAUSAL, 2>(p, n_items, s);
    case MASK_PADDING: return launch_dq_one<D, 4, MASK_PADDING, 2>(p, n_items, s);
    case MASK_DENSE: return launch_dq_one<D, 4, MASK_DENSE, 2>(p, n_items, s);
    default: return launch_dq_one<D, 4, MASK_BLOCK, 2>(p, n_items, s);
  }
}

}  // namespace

// Tile sizes: dQ items are 128 query rows (4 waves; a block layout's two rows are listed as the
// union of their kept tiles and each wave pair computes only its own row's). dK/dV items are 128
// keys, or one 64-key layout column for block masks (2 waves).
int bwd_block_q(int head_dim, int mask) { (void)head_dim; (void)mask; return 128; }
int bwd_dkdv_variant(int mask, int flags, int group, int nb_q) {
  if ((flags & ATTN_BWD_ATOMIC_DQ) != 0) return DKDV_ONE_WAVE;
  if ((mask == MASK_BLOCK || mask == MASK_DENSE) && (int64_t)group * nb_q > PairLds<128>::MAX_STEPS)
    return DKDV_ONE_WAVE;
  return DKDV_PAIR;
}
int bwd_block_k(int head_dim, int mask, int variant) {
  (void)head_dim;
  const bool listed = mask == MASK_BLOCK || mask == MASK_DENSE;
  if (variant == DKDV_PAIR || listed) return 64;
  return 128;
}
int bwd_max_steps() { return KvLds<128>::MAX_STEPS; }

hipError_t launch_bwd_preprocess(const BwdParams& p, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)p.batch * p.heads_q * p.seq_q;
  const unsigned grid = (unsigned)((rows + 127) / 128);   // two lanes per row
  if (head_dim == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(grid), dim3(256), 0, s, p, rows);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(grid), dim3(256), 0, s, p, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdParams& p, int head_dim, int mask, int n_items, hipStream_t s) {
  return head_dim == 128 ? dkdv_mask<128>(p, mask, n_items, s) : dkdv_mask<64>(p, mask, n_items, s);
}

hipError_t launch_bwd_dkdv_pair(const BwdParams& p, int head_dim, int mask, int n_items, hipStream_t s) {
  return head_dim == 128 ? dkdv_pair_mask<128>(p, mask, n_items, s) : dkdv_pair_mask<64>(p, mask, n_items, s);
}


hipError_t launch_bwd_dq(const BwdParams& p, int head_dim, int mask, int n_items, hipStream_t s) {
  return head_dim == 128 ? dq_mask<128>(p, mask, n_items, s) : dq_mask<64>(p, mask, n_items, s);
}

hipError_t launch_bwd_dq_convert(const BwdParams& p, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)p.batch * p.heads_q * p.seq_q;
  const int rpb = 256 / (head_dim / 4);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (head_dim == 128)
    hipLaunchKernelGGL(bwd_dq_convert_kernel<128>, dim3(grid), dim3(256), 0, s, p, rows);
  else
    hipLaunchKernelGGL(bwd_dq_convert_kernel<64>, dim3(grid), dim3(256), 0, s, p, rows);
  return hipGetLastError();
}

}  // namespace attn
