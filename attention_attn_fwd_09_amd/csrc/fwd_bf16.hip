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
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int BN = 64;           // keys per tile
constexpr float RESCALE_SLACK = 8.0f;  // log2 headroom before the reference maximum is re-based

template <int D>
struct FwdLds {
  static constexpr int TILE_BYTES = BN * D * 2;              // one K or V tile
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;         // K + V
  static constexpr int LIST_OFF = 2 * STAGE_BYTES;           // block list after two stages
  static constexpr int MAX_LIST = 1024;                      // kept key tiles per query tile
  static constexpr int BYTES = LIST_OFF + MAX_LIST * 4 + 16;
};

template <int D, int NW, int MASK>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdParams p) {
  constexpr int BM = NW * 32;
  constexpr int KS = D / 16;   // k-steps of the score product
  constexpr int DB = D / 32;   // 32-row blocks of O^T
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 31, hh = lane >> 5;

  // ---- which tile of which (batch, head) ----
  Item it;
  if constexpr (MASK == MASK_NONE || MASK == MASK_CAUSAL) {
    it = closed_form_item(blockIdx.x, p.batch, p.heads_q, p.heads_kv, p.n_qtiles, MASK == MASK_CAUSAL);
  } else {
    it = decode_item(p.items[blockIdx.x], p.heads_q, p.n_qtiles);
  }
  const int b = it.b, h = it.h, kvh = h / p.group;
  const int q0 = it.t * BM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + c;

  const size_t q_off = ((size_t)(b * p.heads_q + h) * p.seq_q) * D;
  const size_t kv_off = ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  const bf16* qg = (const bf16*)p.q + q_off;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg, (uint32_t)p.seq_q * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const bf16*)p.k + kv_off, (uint32_t)p.seq_k * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const bf16*)p.v + kv_off, (uint32_t)p.seq_k * D * 2);

  // ---- key range of this item ----
  int kv_len = p.seq_k;   // keys at or beyond kv_len are masked
  int q_len = p.seq_q;    // queries at or beyond q_len see nothing
  int n_tiles;
  uint32_t* list = (uint32_t*)(smem + FwdLds<D>::LIST_OFF);
  if constexpr (MASK == MASK_PADDING) {
    const int L = clamp_len(p.lengths[b], p.seq_k);
    kv_len = L;
    q_len = clamp_len(p.lengths[b], p.seq_q);
    n_tiles = (q0 < q_len) ? (L + BN - 1) / BN : 0;
  } else if constexpr (MASK == MASK_CAUSAL) {
    const int last_q = min(q0 + BM, p.seq_q) - 1;
    n_tiles = min((p.seq_k + BN - 1) / BN, last_q / BN + 1);
  } else if constexpr (MASK == MASK_BLOCK) {
    // kept key tiles of the layout rows this workgroup covers, with one bit per 64-row layout row
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
      if (lane == 0) list[FwdLds<D>::MAX_LIST] = (uint32_t)count;
    }
    __syncthreads();
    n_tiles = (int)list[FwdLds<D>::MAX_LIST];
  } else {
    n_tiles = (p.seq_k + BN - 1) / BN;
  }

  // ---- Q fragments: B operand of S^T = K Q^T; lane (c, hh) holds Q[my_q][16 ks + 8 hh .. +7] ----
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const i32x4 raw = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
        rq, (uint32_t)my_q * (D * 2) + (uint32_t)(ks * 32 + hh * 16), 0, 0));
    qf[ks] = __builtin_bit_cast(bf16x8, raw);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;   // reference maximum, log2 domain (scores times scale*log2(e))
  float l_run = 0.0f;        // this lane's partial denominator (its 16 keys of each 32-key block)
  const float cs = p.scale_log2;

  auto tile_index = [&](int j) -> int {
    if constexpr (MASK == MASK_BLOCK) return (int)(list[j] & 0xffffu);
    return j;
  };

  auto issue_tile = [&](char* stage, int kt) {
    issue_rows<D, NW>(stage, rk, kt * BN, wave, lane);
    issue_rows<D, NW>(stage + FwdLds<D>::TILE_BYTES, rv, kt * BN, wave, lane);
  };
  if (n_tiles > 0) issue_tile(smem, tile_index(0));

  for (int j = 0; j < n_tiles; ++j) {
    wait_vmem();
    __syncthreads();  // tile j is in LDS; every wave is done with the stage tile j+1 will overwrite
    if (j + 1 < n_tiles)
      issue_tile(smem + ((j + 1) & 1) * FwdLds<D>::STAGE_BYTES, tile_index(j + 1));

    const int kt = tile_index(j);
    const int k0 = kt * BN;
    // wave-uniform: does this wave see any key of the tile, and does it need per-element masking?
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

    const char* kl = smem + (j & 1) * FwdLds<D>::STAGE_BYTES;
    const char* vl = kl + FwdLds<D>::TILE_BYTES;

    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = mfma32(lds_row_frag<D>(kl, kb * 32 + sigma32(c), 2 * ks + hh), qf[ks], s[kb]);
    }

    // ---- online softmax on this lane's 32 scores (keys k0 + kb*32 + hh*16 + i) ----
    float mx = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + hh * 16 + i;
          bool vis = key < kv_len;
          if constexpr (MASK == MASK_CAUSAL) vis = vis && key <= my_q;
          if constexpr (MASK == MASK_PADDING) vis = vis && my_q < q_len;
          const float t = vis ? s[kb][i] * cs : -INFINITY;
          s[kb][i] = t;
          mx = fmaxf(mx, t);
        }
      mx = partner_max(mx);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = partner_max(mx) * cs;
    }
    if (__ballot(mx > m_run + RESCALE_SLACK) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float msub = (m_run == -INFINITY) ? 0.0f : m_run;
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = need_mask ? fast_exp2(s[kb][i] - msub) : fast_exp2(fmaf(s[kb][i], cs, -msub));
        l_run += e;
        pb[kb * 2 + (i >> 3)][i & 7] = (bf16)e;
      }
    }

    // ---- O^T += V^T P^T; chunk kc holds keys kb*32 + hh*16 + hc*8 + 0..7 for lane half hh ----
    const int dsub = ((lane >> 4) & 1) * 16, i16 = lane & 15;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int row0 = (kc >> 1) * 32 + hh * 16 + (kc & 1) * 8;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc[db] = mfma32(lds_tr_frag<D>(vl, row0, db * 32 + dsub, i16), pb[kc], acc[db]);
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l); empty rows give O = 0, LSE = -inf ----
  const float l = partner_sum(l_run);
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : __builtin_amdgcn_rcpf(l);
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
      const float lse = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994530942f;
      p.lse[(size_t)(b * p.heads_q + h) * p.seq_q + my_q] = lse;
    }
  }
}

template <int D, int NW, int MASK>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  static bool attr_done = false;
  const int lds = FwdLds<D>::BYTES;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)fwd_bf16_kernel<D, NW, MASK>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, MASK>), dim3(p.n_items), dim3(NW * 64), lds, stream, p);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_mask(const FwdParams& p, int mask, hipStream_t stream) {
  switch (mask) {
    case MASK_NONE: return launch_one<D, NW, MASK_NONE>(p, stream);
    case MASK_CAUSAL: return launch_one<D, NW, MASK_CAUSAL>(p, stream);
    case MASK_PADDING: return launch_one<D, NW, MASK_PADDING>(p, stream);
    default: return launch_one<D, NW, MASK_BLOCK>(p, stream);
  }
}

}  // namespace

int fwd_bf16_block_m(int head_dim, int mask) {
  (void)head_dim;
  return mask == MASK_BLOCK ? 64 : 128;
}

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, int mask, hipStream_t stream) {
  const int bm = fwd_bf16_block_m(head_dim, mask);
  if (head_dim == 128) return bm == 64 ? launch_mask<128, 2>(p, mask, stream) : launch_mask<128, 4>(p, mask, stream);
  return bm == 64 ? launch_mask<64, 2>(p, mask, stream) : launch_mask<64, 4>(p, mask, stream);
}

}  // namespace attn
