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
//   preprocess  Delta_i = sum_d dO_id O_id (equal to sum_j P_ij dP_ij; fp32, one value per row)
//   dK/dV pass  one workgroup per key tile: K_j, V_j stay in registers, every (query head of the
//               group, query tile) that sees the tile streams Q_i, dO_i, LSE_i, Delta_i through
//               LDS; S = Q_i K_j^T and dP = dO_i V_j^T are recomputed, P = exp(scale S - LSE),
//               dS = P (dP - Delta), and dV_j += P^T dO_i, dK_j += scale dS^T Q_i accumulate in
//               registers.
//   dQ pass     one workgroup per query tile: Q_i, dO_i stay in registers, the visible key tiles
//               stream through LDS, S, P, dP, dS are recomputed and dQ_i += scale dS K_j.
//
// Skipped blocks of a block-sparse layout (and fully masked causal/padding tiles) are never
// visited. Every product runs on v_mfma_f32_32x32x16_bf16; operands that must be read along the
// contraction dimension of a row-major tile come from LDS through ds_read_b64_tr_b16.
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
// Preprocess: Delta = rowsum(dO * O), one group of D/8 lanes per row (16 bytes per lane).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int64_t rows) {
  constexpr int LPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const bf16x8 o = *((const bf16x8*)((const bf16*)p.o + row * D) + sub);
    const bf16x8 g = *((const bf16x8*)((const bf16*)p.dout + row * D) + sub);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && sub == 0) p.delta[row] = acc;
}

// ------------------------------------------------------------------------------------------------
// dK/dV pass.
template <int D>
struct KvLds {
  static constexpr int TILE = BQ * D * 2;
  static constexpr int STATS = 1024;                        // LSE (bytes 0..255) then zero fill
  static constexpr int STAGE = 2 * TILE + 2 * STATS;        // Q, dO, LSE block, Delta block
  static constexpr int LIST_OFF = 2 * STAGE;
  static constexpr int MAX_STEPS = 4096;                    // (query head, query tile) pairs
  static constexpr int BYTES = LIST_OFF + MAX_STEPS * 2 + 16;
};

template <int D, int NW, int MASK>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int BK = NW * 32;   // keys per workgroup
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  using L = KvLds<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, hh = lane >> 5;
  const int dsub = ((lane >> 4) & 1) * 16, i16 = lane & 15;

  const uint32_t item = p.items_kv[blockIdx.x];
  const int kt = (int)(item % (uint32_t)p.n_ktiles);
  const int bkv = (int)(item / (uint32_t)p.n_ktiles);
  const int kvh = bkv % p.heads_kv, b = bkv / p.heads_kv;
  const int k0 = kt * BK;
  const int kw0 = k0 + wave * 32;
  const int my_k = kw0 + c;

  const size_t kv_off = ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const bf16*)p.k + kv_off, (uint32_t)p.seq_k * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16*)p.v + kv_off, (uint32_t)p.seq_k * D * 2);

  // K and V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)my_k * (D * 2) + (uint32_t)(ks * 32 + hh * 16);
    kf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    vf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
  }

  // ---- the (query head, query tile) steps that see this key tile ----
  int kv_len = p.seq_k, q_len = p.seq_q;
  const int n_qt = (p.seq_q + BQ - 1) / BQ;
  int qt_lo = 0, qt_hi = n_qt;
  int n_steps;
  uint16_t* list = (uint16_t*)(smem + L::LIST_OFF);
  if constexpr (MASK == MASK_BLOCK) {
    // kept layout rows of column k0/64 (BK == 64 for block masks), for each query head of the group
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
      if (lane == 0) *(int*)(smem + L::LIST_OFF + L::MAX_STEPS * 2) = min(count, L::MAX_STEPS);
    }
    __syncthreads();
    n_steps = *(const int*)(smem + L::LIST_OFF + L::MAX_STEPS * 2);
  } else {
    if constexpr (MASK == MASK_PADDING) {
      kv_len = clamp_len(p.lengths[b], p.seq_k);
      q_len = clamp_len(p.lengths[b], p.seq_q);
      qt_hi = (k0 < kv_len) ? (q_len + BQ - 1) / BQ : 0;
    } else if constexpr (MASK == MASK_CAUSAL) {
      qt_lo = k0 / BQ;
    }
    n_steps = p.group * max(qt_hi - qt_lo, 0);
  }
  auto step_at = [&](int s, int& g, int& qt) {
    if constexpr (MASK == MASK_BLOCK) {
      const uint32_t e = list[s];
      g = (int)(e >> 10);
      qt = (int)(e & 1023u);
    } else {
      const int per = qt_hi - qt_lo;
      g = s / per;
      qt = qt_lo + s % per;
    }
  };

  auto issue_step = [&](char* stage, int s) {
    int g, qt;
    step_at(s, g, qt);
    const int hq = kvh * p.group + g;
    const size_t q_off = ((size_t)(b * p.heads_q + hq) * p.seq_q) * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const bf16*)p.q + q_off, (uint32_t)p.seq_q * D * 2);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const bf16*)p.dout + q_off, (uint32_t)p.seq_q * D * 2);
    issue_rows<D, NW>(stage, rq, qt * BQ, wave, lane);
    issue_rows<D, NW>(stage + L::TILE, rdo, qt * BQ, wave, lane);
    if (wave == 0) {
      const size_t r_off = (size_t)(b * p.heads_q + hq) * p.seq_q;
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + r_off, (uint32_t)p.seq_q * 4);
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.delta + r_off, (uint32_t)p.seq_q * 4);
      // lanes 0-15 fetch the 64 row values; the others point past the buffer and write zeros
      const uint32_t off = lane < 16 ? (uint32_t)(qt * BQ + lane * 4) * 4 : 0x80000000u;
      buffer_to_lds16(rl, stage + 2 * L::TILE, off);
      buffer_to_lds16(rd, stage + 2 * L::TILE + L::STATS, off);
    }
  };

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  const float cs = p.scale_log2;

  if (n_steps > 0) issue_step(smem, 0);
  for (int s = 0; s < n_steps; ++s) {
    wait_vmem();
    __syncthreads();
    if (s + 1 < n_steps) issue_step(smem + ((s + 1) & 1) * L::STAGE, s + 1);

    int g, qt;
    step_at(s, g, qt);
    const int q0 = qt * BQ;
    bool active = kw0 < kv_len;
    bool need_mask = (q0 + BQ > q_len) || (kw0 + 32 > kv_len);
    if constexpr (MASK == MASK_CAUSAL) {
      active = active && kw0 <= q0 + BQ - 1;
      need_mask = need_mask || (kw0 + 31 > q0);
    } else if constexpr (MASK == MASK_PADDING) {
      active = active && q0 < q_len;
    }
    if (!active) continue;

    const char* ql = smem + (s & 1) * L::STAGE;
    const char* dol = ql + L::TILE;
    const float* lse_l = (const float*)(ql + 2 * L::TILE);
    const float* del_l = (const float*)(ql + 2 * L::TILE + L::STATS);

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S and dP for 32 queries x this wave's 32 keys; lane (c, hh) holds key my_k and queries
      // q0 + qb*32 + hh*16 + i
      f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int row = qb * 32 + sigma32(c);
        sc = mfma32(lds_row_frag<D>(ql, row, 2 * ks + hh), kf[ks], sc);
        dp = mfma32(lds_row_frag<D>(dol, row, 2 * ks + hh), vf[ks], dp);
      }
      const int qbase = qb * 32 + hh * 16;
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float lse2 = lse_to_log2(lse_l[qbase + i]);
        float pv = fast_exp2(fmaf(sc[i], cs, -lse2));
        if (need_mask) {
          const int q = q0 + qbase + i;
          bool vis = q < q_len && my_k < kv_len;
          if constexpr (MASK == MASK_CAUSAL) vis = vis && my_k <= q;
          pv = vis ? pv : 0.0f;
        }
        const float dsv = pv * (dp[i] - del_l[qbase + i]);
        pb[i >> 3][i & 7] = (bf16)pv;
        dsb[i >> 3][i & 7] = (bf16)dsv;
      }
      // dV += P^T dO and dK += dS^T Q: rows = this wave's keys, contraction over the 32 queries
#pragma unroll
      for (int hc = 0; hc < 2; ++hc) {
        const int row0 = qb * 32 + hh * 16 + hc * 8;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dv[db] = mfma32(pb[hc], lds_tr_frag<D>(dol, row0, db * 32 + dsub, i16), dv[db]);
          dk[db] = mfma32(dsb[hc], lds_tr_frag<D>(ql, row0, db * 32 + dsub, i16), dk[db]);
        }
      }
    }
  }

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
// dQ pass.
template <int D>
struct QLds {
  static constexpr int TILE = BN * D * 2;
  static constexpr int STAGE = 2 * TILE;   // K, V
  static constexpr int LIST_OFF = 2 * STAGE;
  static constexpr int MAX_LIST = 1024;
  static constexpr int BYTES = LIST_OFF + MAX_LIST * 4 + 16;
};

template <int D, int NW, int MASK>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(BwdParams p) {
  constexpr int BM = NW * 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  using L = QLds<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, hh = lane >> 5;
  const int dsub = ((lane >> 4) & 1) * 16, i16 = lane & 15;

  const Item it = decode_item(p.items_q[blockIdx.x], p.heads_q, p.n_qtiles);
  const int b = it.b, h = it.h, kvh = h / p.group;
  const int q0 = it.t * BM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + c;

  const size_t q_off = ((size_t)(b * p.heads_q + h) * p.seq_q) * D;
  const size_t kv_off = ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const bf16*)p.q + q_off, (uint32_t)p.seq_q * D * 2);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const bf16*)p.dout + q_off, (uint32_t)p.seq_q * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const bf16*)p.k + kv_off, (uint32_t)p.seq_k * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16*)p.v + kv_off, (uint32_t)p.seq_k * D * 2);

  int kv_len = p.seq_k, q_len = p.seq_q;
  int n_tiles;
  uint32_t* list = (uint32_t*)(smem + L::LIST_OFF);
  if constexpr (MASK == MASK_PADDING) {
    kv_len = clamp_len(p.lengths[b], p.seq_k);
    q_len = clamp_len(p.lengths[b], p.seq_q);
    n_tiles = (q0 < q_len) ? (kv_len + BN - 1) / BN : 0;
  } else if constexpr (MASK == MASK_CAUSAL) {
    n_tiles = min((p.seq_k + BN - 1) / BN, (min(q0 + BM, p.seq_q) - 1) / BN + 1);
  } else if constexpr (MASK == MASK_BLOCK) {
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
            const int row = r0 + r;
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
    __syncthreads();
    n_tiles = (int)list[L::MAX_LIST];
  } else {
    n_tiles = (p.seq_k + BN - 1) / BN;
  }

  // Q and dO rows of this lane's query (B operands of S^T = K Q^T and dP^T = V dO^T)
  bf16x8 qf[KS], dof[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)my_q * (D * 2) + (uint32_t)(ks * 32 + hh * 16);
    qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    dof[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0));
  }
  const size_t row_off = (size_t)(b * p.heads_q + h) * p.seq_q;
  const float lse2 = my_q < p.seq_q ? lse_to_log2(p.lse[row_off + my_q]) : INFINITY;
  const float delta = my_q < p.seq_q ? p.delta[row_off + my_q] : 0.0f;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  const float cs = p.scale_log2;

  auto tile_index = [&](int j) -> int {
    if constexpr (MASK == MASK_BLOCK) return (int)(list[j] & 0xffffu);
    return j;
  };
  auto issue_tile = [&](char* stage, int kt) {
    issue_rows<D, NW>(stage, rk, kt * BN, wave, lane);
    issue_rows<D, NW>(stage + L::TILE, rv, kt * BN, wave, lane);
  };
  if (n_tiles > 0) issue_tile(smem, tile_index(0));

  for (int j = 0; j < n_tiles; ++j) {
    wait_vmem();
    __syncthreads();
    if (j + 1 < n_tiles) issue_tile(smem + ((j + 1) & 1) * L::STAGE, tile_index(j + 1));

    const int k0 = tile_index(j) * BN;
    bool active = true, need_mask = (k0 + BN > kv_len);
    if constexpr (MASK == MASK_CAUSAL) {
      active = k0 <= qw0 + 31;
      need_mask = need_mask || (k0 + BN - 1 > qw0);
    } else if constexpr (MASK == MASK_PADDING) {
      active = qw0 < q_len;
      need_mask = need_mask || (qw0 + 31 >= q_len);
    } else if constexpr (MASK == MASK_BLOCK) {
      active = ((list[j] >> 16) >> ((wave * 32) / 64)) & 1u;
    }
    if (!active) continue;

    const char* kl = smem + (j & 1) * L::STAGE;
    const char* vl = kl + L::TILE;
    f32x16 sc[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = kb * 32 + sigma32(c);
        sc[kb] = mfma32(lds_row_frag<D>(kl, row, 2 * ks + hh), qf[ks], sc[kb]);
        dp[kb] = mfma32(lds_row_frag<D>(vl, row, 2 * ks + hh), dof[ks], dp[kb]);
      }
    }
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = fast_exp2(fmaf(sc[kb][i], cs, -lse2));
        if (need_mask) {
          const int key = k0 + kb * 32 + hh * 16 + i;
          bool vis = key < kv_len && my_q < q_len;
          if constexpr (MASK == MASK_CAUSAL) vis = vis && key <= my_q;
          pv = vis ? pv : 0.0f;
        }
        dsb[kb * 2 + (i >> 3)][i & 7] = (bf16)(pv * (dp[kb][i] - delta));
      }
    }
    // dQ^T += K^T dS^T: A = K^T from the transposed read of the K tile
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int row0 = (kc >> 1) * 32 + hh * 16 + (kc & 1) * 8;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] = mfma32(lds_tr_frag<D>(kl, row0, db * 32 + dsub, i16), dsb[kc], acc[db]);
    }
  }

  if (my_q < p.seq_q) {
    bf16* dqg = (bf16*)p.dq + q_off + (size_t)my_q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)(acc[db][g4 * 4 + e] * p.scale);
        *(bf16x4*)(dqg + db * 32 + g4 * 8 + hh * 4) = v4;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
template <typename K>
hipError_t set_lds(K kernel, int bytes, bool& done) {
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done = true;
  return e;
}

template <int D, int NW, int MASK>
hipError_t launch_dkdv_one(const BwdParams& p, int n_items, hipStream_t s) {
  static bool done = false;
  hipError_t e = set_lds(bwd_dkdv_kernel<D, NW, MASK>, KvLds<D>::BYTES, done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, MASK>), dim3(n_items), dim3(NW * 64), KvLds<D>::BYTES, s, p);
  return hipGetLastError();
}

template <int D, int NW, int MASK>
hipError_t launch_dq_one(const BwdParams& p, int n_items, hipStream_t s) {
  static bool done = false;
  hipError_t e = set_lds(bwd_dq_kernel<D, NW, MASK>, QLds<D>::BYTES, done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, NW, MASK>), dim3(n_items), dim3(NW * 64), QLds<D>::BYTES, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t dkdv_mask(const BwdParams& p, int mask, int n_items, hipStream_t s) {
  switch (mask) {
    case MASK_NONE: return launch_dkdv_one<D, 4, MASK_NONE>(p, n_items, s);
    case MASK_CAUSAL: return launch_dkdv_one<D, 4, MASK_CAUSAL>(p, n_items, s);
    case MASK_PADDING: return launch_dkdv_one<D, 4, MASK_PADDING>(p, n_items, s);
    default: return launch_dkdv_one<D, 2, MASK_BLOCK>(p, n_items, s);
  }
}

template <int D>
hipError_t dq_mask(const BwdParams& p, int mask, int n_items, hipStream_t s) {
  switch (mask) {
    case MASK_NONE: return launch_dq_one<D, 4, MASK_NONE>(p, n_items, s);
    case MASK_CAUSAL: return launch_dq_one<D, 4, MASK_CAUSAL>(p, n_items, s);
    case MASK_PADDING: return launch_dq_one<D, 4, MASK_PADDING>(p, n_items, s);
    default: return launch_dq_one<D, 2, MASK_BLOCK>(p, n_items, s);
  }
}

}  // namespace

// Tile sizes: the block-sparse layout works on 64 x 64 tiles, so its passes use 64-row tiles
// (2 waves); other masks use 128-row tiles (4 waves).
int bwd_block_q(int head_dim, int mask) { (void)head_dim; return mask == MASK_BLOCK ? 64 : 128; }
int bwd_block_k(int head_dim, int mask) { (void)head_dim; return mask == MASK_BLOCK ? 64 : 128; }
int bwd_max_steps() { return KvLds<128>::MAX_STEPS; }

hipError_t launch_bwd_preprocess(const BwdParams& p, int head_dim, hipStream_t s) {
  const int64_t rows = (int64_t)p.batch * p.heads_q * p.seq_q;
  const int rpb = 256 / (head_dim / 8);
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (head_dim == 128)
    hipLaunchKernelGGL(bwd_pre_kernel<128>, dim3(grid), dim3(256), 0, s, p, rows);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<64>, dim3(grid), dim3(256), 0, s, p, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const BwdParams& p, int head_dim, int mask, int n_items, hipStream_t s) {
  return head_dim == 128 ? dkdv_mask<128>(p, mask, n_items, s) : dkdv_mask<64>(p, mask, n_items, s);
}

hipError_t launch_bwd_dq(const BwdParams& p, int head_dim, int mask, int n_items, hipStream_t s) {
  return head_dim == 128 ? dq_mask<128>(p, mask, n_items, s) : dq_mask<64>(p, mask, n_items, s);
}

}  // namespace attn
