// Fused attention forward with fp8 (OCP e4m3) Q, K, V inputs for gfx950 (CDNA4).
//
// Same method as the bf16 forward (the "fused multi-head attention operator" write-up, zwxr.cn,
// sections 3.1-3.3: tiles of keys streamed through on-chip memory, online softmax, P V
// accumulated in registers) and the same work decomposition (fwd_shared.h); the pages mention fp8
// only in passing, so this is the plain reading: the products run on the fp8 matrix cores,
// everything else in fp32, the output is bf16.
//
//  * S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (scales 2^0): a lane of each operand holds
//    32 bytes along k, and the two operands pair their k positions by (lane half, byte), so the
//    lane's bytes are d = ks*64 + half*32 + 0..31 for both K (LDS row fragments) and Q (registers).
//    K rows are permuted with sigma32 as in the bf16 kernel: lane (c, h) of S^T holds query c and
//    keys h*16 + 0..15 of each 32-key block.
//  * P = 2^7 * exp2(scale*log2(e)*S - m) is rounded to e4m3 and packed as the B operand of
//    O^T += V^T P^T with byte J of lane (c, h) = key (J/16)*32 + h*16 + J%16; the V^T operand uses
//    the same key order, read from the V tile with ds_read_b64_tr_b8 (8 keys of one column per
//    read, four reads per fragment). The maximum is re-based when it grows by more than 2^1, so
//    2^7 P stays below 2^8 (e4m3's largest finite value is 448) and values down to 2^-16 of the
//    row maximum stay representable.
//  * The row sum is one more MFMA of P^T against an all-ones A operand (every row of the result
//    is the sum of the same rounded P that enters P V), so O is an exact convex combination of
//    the rounded weights.
//  * LDS tiles are 64 rows of D bytes with 16-byte chunks XOR-swizzled per row (swz8) so that
//    both the row fragment reads and the transposed reads are free of bank conflicts.
#include <type_traits>

#include "common.h"
#include "fwd_shared.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int BN = 64;                    // keys per tile
constexpr float RESCALE_SLACK_FP8 = 1.0f; // log2 headroom before the reference maximum is re-based
constexpr float P_EXP = 7.0f;             // P is stored as 2^7 * p

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// Chunk swizzle of an 8-bit tile row. Row fragment reads: 16 lanes read one logical chunk of rows
// {0-7, 16-23} (+8, +32); transposed reads: 16 lanes read one chunk of 8 consecutive rows.
template <int D> __device__ __forceinline__ int swz8(int row);
template <> __device__ __forceinline__ int swz8<128>(int row) { return ((row >> 1) & 3) | ((row >> 2) & 4); }
template <> __device__ __forceinline__ int swz8<64>(int row) { return ((row >> 2) & 1) | ((row >> 3) & 2); }

// Rows [row0, row0 + 64) of a [rows][D] byte tensor into an LDS tile, swizzled; rows past the end
// of the buffer read as 0. All NW*64 threads take part.
template <int D, int NW>
__device__ __forceinline__ void issue_rows8(char* lds_tile, __amdgpu_buffer_rsrc_t r, int row0, int wave, int lane) {
  constexpr int CPR = D / 16;
  constexpr int ROUNDS = (64 * CPR) / (NW * 64);
#pragma unroll
  for (int it = 0; it < ROUNDS; ++it) {
    const int blk = it * NW + wave;
    const int pos = blk * 64 + lane;
    const int row = pos / CPR;
    const int pc = pos % CPR;
    buffer_to_lds16(r, lds_tile + blk * 1024, (uint32_t)(row0 + row) * D + (uint32_t)((pc ^ swz8<D>(row)) * 16));
  }
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int D>
struct Fp8Lds {
  static constexpr int TILE_BYTES = BN * D;
  static constexpr int MAX_LIST = 1024;
};

template <int D, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fwd_fp8_kernel(FwdParams p) {
  constexpr int NW = 4;
  constexpr int BM = NW * 32;
  constexpr int KS = D / 64;   // k-steps of the score product
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  constexpr int RB = D;        // bytes per tile row
  constexpr bool LISTED = MASK == MASK_BLOCK || MASK == MASK_DENSE;
  using L = Fp8Lds<D>;
  __shared__ __attribute__((aligned(16))) char k_st0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_st0[L::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char k_st1[L::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_st1[L::TILE_BYTES];
  __shared__ uint32_t list[LISTED ? L::MAX_LIST + 1 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, hh = lane >> 5;
  const int i16 = lane & 15, g16 = lane >> 4;

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
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + c;
  const uint32_t* dense_row = MASK == MASK_DENSE
      ? p.dense.rows + b * p.dense.rows_stride_b + h * p.dense.rows_stride_h + (int64_t)my_q * p.dense.row_words
      : nullptr;

  const size_t q_off = ((size_t)(b * p.heads_q + h) * p.seq_q) * D;
  const size_t kv_off = ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint8_t*)p.q + q_off, (uint32_t)p.seq_q * RB);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint8_t*)p.k + kv_off, (uint32_t)p.seq_k * RB);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint8_t*)p.v + kv_off, (uint32_t)p.seq_k * RB);

  // Q fragments (B operand of S^T = K Q^T): lane (c, hh) holds Q[my_q][ks*64 + hh*32 + 0..31]
  i32x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)my_q * RB + (uint32_t)(ks * 64 + hh * 32);
    const i32x4 lo = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    const i32x4 hi = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0));
    qf[ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  int kv_len, q_len;
  const int n_tiles = fwd_key_tiles<MASK, BM, BN>(p, b, h, q0, wave, lane, list, L::MAX_LIST, kv_len, q_len);

  // per-lane LDS offsets: K row fragment of k-step ks, chunk half j (key block kb adds 32 rows)
  int koff[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int row = sigma32(c);
#pragma unroll
    for (int j = 0; j < 2; ++j) koff[ks][j] = row * RB + (((ks * 4 + hh * 2 + j) ^ swz8<D>(row)) * 16);
  }
  // transposed V reads: 16-lane group g16 covers columns db*32 + (g16 & 1)*16 + i16 and key runs of
  // lane half g16 >> 1; lane i16 supplies the address of row (run base + i16/2), bytes (i16 & 1)*8
  int voff[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int chunk = db * 2 + (g16 & 1);
#pragma unroll
    for (int run = 0; run < 4; ++run) {
      const int row = (run >> 1) * 32 + (g16 >> 1) * 16 + (run & 1) * 8 + (i16 >> 1);
      voff[db][run] = row * RB + ((chunk ^ swz8<D>(row)) * 16) + (i16 & 1) * 8;
    }
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  f32x16 acc_l = f32x16{};     // every row: the query's running sum of the rounded 2^7 P
  float m_run = -INFINITY;     // reference maximum, log2 domain
  const float cs = p.scale_log2;
  const int ones_v = 0x38383838;   // four e4m3 1.0
  const i32x8 ones = {ones_v, ones_v, ones_v, ones_v, ones_v, ones_v, ones_v, ones_v};

  auto tile_index = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (LISTED) return (int)(list[j] & 0xffffu);
    return j;
  };
  auto issue_tile = [&](auto stage_tag, int kt) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    issue_rows8<D, NW>(ST == 0 ? k_st0 : k_st1, rk, kt * BN, wave, lane);
    issue_rows8<D, NW>(ST == 0 ? v_st0 : v_st1, rv, kt * BN, wave, lane);
  };

  auto tile = [&](auto stage_tag, auto masked_tag, int k0) __attribute__((always_inline)) {
    constexpr int ST = decltype(stage_tag)::value;
    constexpr bool MASKED = decltype(masked_tag)::value;
    const char* kl = ST == 0 ? k_st0 : k_st1;
    const char* vl = ST == 0 ? v_st0 : v_st1;

    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x8 ka, kb1;
      {
        const i32x4 a0 = *(const i32x4*)(kl + koff[ks][0]);
        const i32x4 a1 = *(const i32x4*)(kl + koff[ks][1]);
        const i32x4 b0 = *(const i32x4*)(kl + koff[ks][0] + 32 * RB);
        const i32x4 b1 = *(const i32x4*)(kl + koff[ks][1] + 32 * RB);
        ka = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        kb1 = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      s0 = mfma_fp8(ka, qf[ks], s0);
      s1 = mfma_fp8(kb1, qf[ks], s1);
    }

    // ---- mask (boundary tiles only) ----
    uint32_t dw0 = 0, dw1 = 0;
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

    // ---- online softmax ----
    float ma = vmax(s0[0], s0[1]), mb = vmax(s1[0], s1[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      ma = vmax3(ma, s0[i], s0[i + 1]);
      mb = vmax3(mb, s1[i], s1[i + 1]);
    }
    const float mx = partner_max(vmax(ma, mb)) * cs;
    if (__builtin_expect(__ballot(mx > m_run + RESCALE_SLACK_FP8) != 0, 0)) {
      const float m_new = vmax(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
      m_run = m_new;
      acc_l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float msub = (m_run == -INFINITY) ? 0.0f : m_run;

    // V^T fragments: four transposed reads of 8 keys each per column block
    i32x8 va[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      i32x2 r[4];
#pragma unroll
      for (int run = 0; run < 4; ++run)
        r[run] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(vl + voff[db][run]));
      va[db] = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
    }
    // 2^7 P in e4m3, byte J of the lane = key (J/16)*32 + hh*16 + J%16
    i32x8 pb;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const f32x16& sv = w < 4 ? s0 : s1;
      const int i0 = (w & 3) * 4;
      const float e0 = fast_exp2(fmaf(sv[i0], cs, P_EXP - msub));
      const float e1 = fast_exp2(fmaf(sv[i0 + 1], cs, P_EXP - msub));
      const float e2 = fast_exp2(fmaf(sv[i0 + 2], cs, P_EXP - msub));
      const float e3 = fast_exp2(fmaf(sv[i0 + 3], cs, P_EXP - msub));
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
      pb[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, word, true);
    }
    // O^T += V^T P^T; the all-ones operand gives the row sums of the same rounded P
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = mfma_fp8(va[db], pb, acc[db]);
    acc_l = mfma_fp8(ones, pb, acc_l);
  };

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
    if (j + 1 < t1) issue_tile(std::integral_constant<int, 1 - ST>{}, tile_index(j + 1));
    const int k0 = tile_index(j) * BN;
    bool active = true;
    if constexpr (LISTED) active = ((list[j] >> 16) >> ((wave * 32) / 64)) & 1u;
    if constexpr (MASKED) {
      active = active && k0 < kv_len;
      if constexpr (MASK == MASK_CAUSAL) active = active && k0 <= qw0 + 31;
      if constexpr (MASK == MASK_PADDING) active = active && qw0 < q_len;
    }
    if (active) tile(stage_tag, masked_tag, k0);
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

  if (t0 < t1) {
    if (t0 & 1) issue_tile(std::integral_constant<int, 1>{}, tile_index(t0));
    else issue_tile(std::integral_constant<int, 0>{}, tile_index(t0));
  }
  run(std::false_type{}, t0, t_free);
  run(std::true_type{}, t_free, t1);

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2(l) - 7); empty rows: O = 0, LSE = -inf ----
  const float l = acc_l[0];
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : __builtin_amdgcn_rcpf(l);
  if (p.kv_splits > 1) {
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
      if (hh == 0)
        p.lse_part[(size_t)split * rows + row] = empty ? -INFINITY : m_run + __builtin_amdgcn_logf(l) - P_EXP;
    }
    return;
  }
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
    if (hh == 0) {
      const float lse = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l) - P_EXP) * 0.69314718055994530942f;
      p.lse[(size_t)(b * p.heads_q + h) * p.seq_q + my_q] = lse;
    }
  }
}

template <int D, int MASK>
hipError_t launch_fp8_one(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_fp8_kernel<D, MASK>), dim3((uint32_t)p.n_items * (uint32_t)p.kv_splits), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fp8_mask(const FwdParams& p, int mask, hipStream_t stream) {
  switch (mask) {
    case MASK_NONE: return launch_fp8_one<D, MASK_NONE>(p, stream);
    case MASK_CAUSAL: return launch_fp8_one<D, MASK_CAUSAL>(p, stream);
    case MASK_PADDING: return launch_fp8_one<D, MASK_PADDING>(p, stream);
    case MASK_DENSE: return launch_fp8_one<D, MASK_DENSE>(p, stream);
    default: return launch_fp8_one<D, MASK_BLOCK>(p, stream);
  }
}

}  // namespace

int fwd_fp8_block_m() { return 128; }

hipError_t launch_fwd_fp8(const FwdParams& p, int head_dim, int mask, hipStream_t stream) {
  return head_dim == 128 ? launch_fp8_mask<128>(p, mask, stream) : launch_fp8_mask<64>(p, mask, stream);
}

}  // namespace attn
