// Fused attention forward in fp32 (inputs, arithmetic and outputs all float32).
//
// Same method as the bf16 kernel (fused-attention write-up, zwxr.cn, sections 3.2-3.3: key/value
// tiles streamed through on-chip memory, online softmax with a correction factor, O and LSE written
// once), but on the vector ALU. Two kernels:
//  * tile kernel: one wave per 64-query tile, one query row per lane, key/value tiles shared
//    through LDS; used when there are enough tiles to occupy the chip;
//  * row kernel: one wave per query row, one key per lane in every 64-key step, K and V rows read
//    straight from the caches; used for small problems, where the tile kernel would run a handful
//    of waves whose lanes each walk every key serially.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int BM32 = 64;  // queries per workgroup (one per lane)
constexpr int BN32 = 64;  // keys per tile

template <int D>
struct F32Lds {
  static constexpr int QP = D + 1;  // padded Q row pitch (floats): lanes read different rows
  static constexpr int Q_OFF = 0;
  static constexpr int K_OFF = Q_OFF + BM32 * QP * 4;
  static constexpr int V_OFF = K_OFF + BN32 * D * 4;
  static constexpr int BYTES = V_OFF + BN32 * D * 4;
};

template <int D, int MASK>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* ql = (float*)(smem + F32Lds<D>::Q_OFF);
  float* kl = (float*)(smem + F32Lds<D>::K_OFF);
  float* vl = (float*)(smem + F32Lds<D>::V_OFF);
  constexpr int QP = F32Lds<D>::QP;

  const int lane = threadIdx.x;
  const Item it = decode_item(blockIdx.x, p.heads_q, p.n_qtiles);
  const int b = it.b, h = it.h, kvh = h / p.group;
  const int q0 = it.t * BM32;
  const int my_q = q0 + lane;
  const size_t q_off = ((size_t)(b * p.heads_q + h) * p.seq_q) * D;
  const size_t kv_off = ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  const float* qg = (const float*)p.q + q_off;
  const float* kg = (const float*)p.k + kv_off;
  const float* vg = (const float*)p.v + kv_off;

  int kv_len = p.seq_k, q_len = p.seq_q;
  if constexpr (MASK == MASK_PADDING) {
    kv_len = clamp_len(p.lengths[b], p.seq_k);
    q_len = clamp_len(p.lengths[b], p.seq_q);
  }
  const uint8_t* lay_row = nullptr;
  if constexpr (MASK == MASK_BLOCK) {
    lay_row = p.layout + b * p.layout_stride_b + h * p.layout_stride_h + (size_t)(q0 / 64) * p.nb_k;
  }
  // dense mask: this query's row of bytes (queries past the end see nothing)
  const uint8_t* dense_row = nullptr;
  if constexpr (MASK == MASK_DENSE) {
    dense_row = p.dense_bytes + b * p.dense_stride_b + h * p.dense_stride_h + (int64_t)min(my_q, p.seq_q - 1) * p.seq_k;
  }

  // stage this tile's queries (rows past the end read as 0)
  for (int e = lane; e < BM32 * D; e += 64) {
    const int r = e / D, d = e % D;
    ql[r * QP + d] = (q0 + r < p.seq_q) ? qg[(size_t)(q0 + r) * D + d] : 0.0f;
  }

  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const float cs = p.scale_log2;

  int n_kt = (kv_len + BN32 - 1) / BN32;
  if constexpr (MASK == MASK_CAUSAL) n_kt = min(n_kt, (min(q0 + BM32, p.seq_q) - 1) / BN32 + 1);
  if constexpr (MASK == MASK_PADDING) n_kt = (q0 < q_len) ? n_kt : 0;

  for (int kt = 0; kt < n_kt; ++kt) {
    if constexpr (MASK == MASK_BLOCK) {
      if (lay_row[kt] == 0) continue;  // wave-uniform: whole 64x64 tile skipped
    }
    const int k0 = kt * BN32;
    __syncthreads();
    for (int e = lane; e < BN32 * D; e += 64) {
      const int r = e / D;
      const bool in = k0 + r < p.seq_k;
      kl[e] = in ? kg[(size_t)k0 * D + e] : 0.0f;
      vl[e] = in ? vg[(size_t)k0 * D + e] : 0.0f;
    }
    __syncthreads();

    float s[BN32];
    float mx = -INFINITY;
#pragma unroll 4
    for (int j = 0; j < BN32; ++j) {
      float dot = 0.0f;
#pragma unroll 16
      for (int d = 0; d < D; ++d) dot = fmaf(ql[lane * QP + d], kl[j * D + d], dot);
      const int key = k0 + j;
      bool vis = key < kv_len;
      if constexpr (MASK == MASK_CAUSAL) vis = vis && key <= my_q;
      if constexpr (MASK == MASK_PADDING) vis = vis && my_q < q_len;
      if constexpr (MASK == MASK_DENSE) vis = vis && my_q < p.seq_q && dense_row[min(key, p.seq_k - 1)] != 0;
      s[j] = vis ? dot * cs : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    // rows that have seen no visible key yet keep m = -inf, alpha = 1 and add exp2(-inf) = 0
    const float m_new = fmaxf(m_run, mx);
    const bool any = m_new != -INFINITY;
    const float msub = any ? m_new : 0.0f;
    const float alpha = any ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // m_run = -inf gives 0
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
    for (int j = 0; j < BN32; ++j) {
      const float e = __builtin_amdgcn_exp2f(s[j] - msub);
      l_run += e;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(e, vl[j * D + d], acc[d]);
    }
  }

  if (my_q < p.seq_q) {
    const bool empty = !(l_run > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / l_run;
    float* og = (float*)p.o + q_off + (size_t)my_q * D;
#pragma unroll
    for (int d = 0; d < D; ++d) og[d] = acc[d] * inv;
    p.lse[(size_t)(b * p.heads_q + h) * p.seq_q + my_q] =
        empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f;
  }
}

// ---- row kernel ----
constexpr int ROW_WAVES = 4;   // query rows (waves) per workgroup

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Query row r = (b * heads_q + h) * seq_q + i. Each 64-key step: lane j scores key k0 + j against
// the row (its K row read with 16-byte loads), the wave reduces the step's maximum and sum, and
// every lane accumulates its D/64 output columns over the step's 64 keys (P_j broadcast from lane
// j, V rows read column-contiguous across the wave).
template <int D, int MASK>
__global__ __launch_bounds__(64 * ROW_WAVES) void fwd_f32_row_kernel(FwdParams p, int64_t rows) {
  constexpr int DPL = D / 64;   // output columns per lane
  constexpr int VC = 64 / DPL;  // keys of V in registers at a time (64 values per lane)
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * ROW_WAVES + (threadIdx.x >> 6);
  if (r >= rows) return;   // wave-uniform; the kernel has no barriers
  const int i = (int)(r % p.seq_q);
  const int64_t bh = r / p.seq_q;
  const int h = (int)(bh % p.heads_q), b = (int)(bh / p.heads_q);
  const int kvh = h / p.group;
  const float* qrow = (const float*)p.q + r * D;
  const float* kg = (const float*)p.k + ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;
  const float* vg = (const float*)p.v + ((size_t)(b * p.heads_kv + kvh) * p.seq_k) * D;

  // keys [0, n_keys) can be visible to this row
  int n_keys = p.seq_k;
  if constexpr (MASK == MASK_CAUSAL) n_keys = min(p.seq_k, i + 1);
  if constexpr (MASK == MASK_PADDING) {
    const int len_k = clamp_len(p.lengths[b], p.seq_k);
    n_keys = i < clamp_len(p.lengths[b], p.seq_q) ? len_k : 0;
  }
  const uint8_t* lay_row = nullptr;
  if constexpr (MASK == MASK_BLOCK) lay_row = p.layout + b * p.layout_stride_b + h * p.layout_stride_h + (size_t)(i / 64) * p.nb_k;
  const uint8_t* dense_row = nullptr;
  if constexpr (MASK == MASK_DENSE) dense_row = p.dense_bytes + b * p.dense_stride_b + h * p.dense_stride_h + (int64_t)i * p.seq_k;

  float q[D];   // the row, in every lane (all lanes load the same addresses)
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const f32x4 v4 = *(const f32x4*)(qrow + d);
    q[d] = v4[0]; q[d + 1] = v4[1]; q[d + 2] = v4[2]; q[d + 3] = v4[3];
  }
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const float cs = p.scale_log2;

  for (int k0 = 0; k0 < n_keys; k0 += 64) {
    if constexpr (MASK == MASK_BLOCK) {
      if (lay_row[k0 / 64] == 0) continue;   // wave-uniform: the whole 64-key block is hidden
    }
    const int key = k0 + lane;
    bool vis = key < n_keys;
    if constexpr (MASK == MASK_DENSE) vis = vis && dense_row[key] != 0;
    float dot = 0.0f;
    if (key < p.seq_k) {
      const float* krow = kg + (size_t)key * D;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const f32x4 k4 = *(const f32x4*)(krow + d);
        dot = fmaf(q[d], k4[0], dot);
        dot = fmaf(q[d + 1], k4[1], dot);
        dot = fmaf(q[d + 2], k4[2], dot);
        dot = fmaf(q[d + 3], k4[3], dot);
      }
    }
    const float sc = vis ? dot * cs : -INFINITY;
    // online softmax; a row that has seen no visible key keeps m = -inf and adds exp2(-inf) = 0
    const float m_new = fmaxf(m_run, wave_max(sc));
    const bool any = m_new != -INFINITY;
    const float alpha = any ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    const float pj = __builtin_amdgcn_exp2f(sc - (any ? m_new : 0.0f));
    l_run = l_run * alpha + wave_sum(pj);
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] *= alpha;
    // P V over the step's keys, VC keys at a time: the chunk's V values are all loaded before the
    // first is used, so the loads of a chunk overlap instead of running one key after another
    // (keys past the sequence read as 0; their P is 0)
    const int nj = min(64, p.seq_k - k0);   // keys of the step that exist
    for (int j0 = 0; j0 < nj; j0 += VC) {
      float vv[VC][DPL];
#pragma unroll
      for (int j = 0; j < VC; ++j) {
        const float* vrow = vg + (size_t)(k0 + j0 + j) * D;
#pragma unroll
        for (int e = 0; e < DPL; ++e) vv[j][e] = (j0 + j < nj) ? vrow[lane + 64 * e] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < VC; ++j) {
        const float pb = __shfl(pj, j0 + j, 64);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(pb, vv[j][e], acc[e]);
      }
    }
  }

  const bool empty = !(l_run > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l_run;
  float* og = (float*)p.o + r * D;
#pragma unroll
  for (int e = 0; e < DPL; ++e) og[lane + 64 * e] = acc[e] * inv;
  if (lane == 0) p.lse[r] = empty ? -INFINITY : (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994530942f;
}

template <int D, int MASK>
hipError_t launch_f32_row(const FwdParams& p, int64_t rows, hipStream_t stream) {
  const unsigned grid = (unsigned)((rows + ROW_WAVES - 1) / ROW_WAVES);
  hipLaunchKernelGGL((fwd_f32_row_kernel<D, MASK>), dim3(grid), dim3(64 * ROW_WAVES), 0, stream, p, rows);
  return hipGetLastError();
}

template <int D, int MASK>
hipError_t launch_f32_one(const FwdParams& p, hipStream_t stream) {
  // Small problems go to the row kernel: fewer 64-query tiles than compute units, and few enough
  // (query, key) pairs that every row reading its head's K and V rows from the caches stays cheap.
  const int64_t rows = (int64_t)p.batch * p.heads_q * p.seq_q;
  if (p.n_items < 256 && rows * p.seq_k <= ((int64_t)1 << 22)) return launch_f32_row<D, MASK>(p, rows, stream);
  static bool attr_done = false;
  const int lds = F32Lds<D>::BYTES;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)fwd_f32_kernel<D, MASK>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL((fwd_f32_kernel<D, MASK>), dim3(p.n_items), dim3(64), lds, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32_mask(const FwdParams& p, int mask, hipStream_t stream) {
  switch (mask) {
    case MASK_NONE: return launch_f32_one<D, MASK_NONE>(p, stream);
    case MASK_CAUSAL: return launch_f32_one<D, MASK_CAUSAL>(p, stream);
    case MASK_PADDING: return launch_f32_one<D, MASK_PADDING>(p, stream);
    case MASK_DENSE: return launch_f32_one<D, MASK_DENSE>(p, stream);
    default: return launch_f32_one<D, MASK_BLOCK>(p, stream);
  }
}

}  // namespace

int fwd_f32_block_m() { return BM32; }

hipError_t launch_fwd_f32(const FwdParams& p, int head_dim, int mask, hipStream_t stream) {
  return head_dim == 128 ? launch_f32_mask<128>(p, mask, stream) : launch_f32_mask<64>(p, mask, stream);
}

}  // namespace attn
