// C ABI of libattn: argument checks, workspace sizing, planning and kernel dispatch.
//
// Every check runs on the host before the first HIP call, so a rejected call launches nothing and
// writes nothing (the fused-attention write-up, zwxr.cn, section 2.3, on declaring format, dtype
// and tiling metadata up front so that a mismatch fails at once instead of late).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "api_internal.h"
#include "attn.h"
#include "kernels.h"
#include "params.h"

using namespace attn;

namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_BLOCK_COLS = 1024;  // key tiles per layout row the forward kernel can list

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// bytes of one input element, and of one output (O) element: fp8 inputs give a bf16 output
size_t elem_size(int32_t dtype) { return dtype == ATTN_F32 ? 4 : dtype == ATTN_FP8_E4M3 ? 1 : 2; }
size_t out_elem_size(int32_t dtype) { return dtype == ATTN_F32 ? 4 : 2; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range range_of(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

const attn_mask kNoMask = {ATTN_MASK_NONE, nullptr, nullptr, 0, 0, 64, 64, nullptr, 0, 0};

// Checks shared by forward and backward. `mask` is never null here.
attn_status check_problem(const attn_problem* p, const attn_mask* m, float scale) {
  if (p->batch < 1 || p->heads_q < 1 || p->heads_kv < 1 || p->seq_q < 1 || p->seq_k < 1 || p->head_dim < 1)
    return ATTN_ERR_SHAPE;
  if (p->heads_q % p->heads_kv != 0) return ATTN_ERR_SHAPE;
  if (p->dtype != ATTN_F32 && p->dtype != ATTN_BF16 && p->dtype != ATTN_FP8_E4M3) return ATTN_ERR_DTYPE;
  if (!(std::isfinite(scale) && scale >= 0.0f)) return ATTN_ERR_SHAPE;
  switch (m->kind) {
    case ATTN_MASK_NONE: break;
    case ATTN_MASK_CAUSAL:
      if (p->seq_q != p->seq_k) return ATTN_ERR_SHAPE;
      break;
    case ATTN_MASK_PADDING:
      if (m->lengths == nullptr) return ATTN_ERR_MASK;
      break;
    case ATTN_MASK_BLOCK:
      if (m->block_layout == nullptr) return ATTN_ERR_MASK;
      if (m->block_q != 64 || m->block_k != 64) return ATTN_ERR_MASK;
      if (m->layout_stride_b < 0 || m->layout_stride_h < 0) return ATTN_ERR_MASK;
      if (ceil_div(p->seq_k, 64) > MAX_BLOCK_COLS) return ATTN_ERR_UNSUPPORTED;
      break;
    case ATTN_MASK_DENSE:
      if (m->dense == nullptr) return ATTN_ERR_MASK;
      if (m->dense_stride_b < 0 || m->dense_stride_h < 0) return ATTN_ERR_MASK;
      if (ceil_div(p->seq_k, 64) > MAX_BLOCK_COLS) return ATTN_ERR_UNSUPPORTED;
      break;
    default: return ATTN_ERR_MASK;
  }
  if (p->head_dim != 64 && p->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  // per-(batch, head) slices are addressed with 32-bit byte offsets
  const int64_t es = (int64_t)elem_size(p->dtype);
  if ((int64_t)p->seq_q * p->head_dim * es >= (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)p->seq_k * p->head_dim * es >= (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->heads_q * ceil_div(p->seq_q, 64) >= (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int64_t layout_bytes(const attn_problem* p, const attn_mask* m) {
  const int64_t nbq = ceil_div(p->seq_q, 64), nbk = ceil_div(p->seq_k, 64);
  return (int64_t)(p->batch - 1) * m->layout_stride_b + (int64_t)(p->heads_q - 1) * m->layout_stride_h + nbq * nbk;
}

int64_t dense_bytes(const attn_problem* p, const attn_mask* m) {
  return (int64_t)(p->batch - 1) * m->dense_stride_b + (int64_t)(p->heads_q - 1) * m->dense_stride_h +
         (int64_t)p->seq_q * p->seq_k;
}

// Workspace of a packed dense mask (bf16 kernels): row bits, column bits (backward only) and the
// derived 64x64 block layout, per distinct (batch element, query head) of the mask.
struct DenseSizes {
  int32_t batch_m, heads_m, row_words, col_words, nb_q, nb_k;
  size_t rows_off, cols_off, layout_off, total;   // offsets from the region's start
};

DenseSizes dense_sizes(const attn_problem* p, const attn_mask* m, bool with_cols) {
  DenseSizes z{};
  if (m->kind != ATTN_MASK_DENSE || p->dtype == ATTN_F32) return z;
  z.batch_m = m->dense_stride_b != 0 ? p->batch : 1;
  z.heads_m = m->dense_stride_h != 0 ? p->heads_q : 1;
  z.row_words = ceil_div(p->seq_k, 32);
  z.col_words = ceil_div(p->seq_q, 32);
  z.nb_q = ceil_div(p->seq_q, 64);
  z.nb_k = ceil_div(p->seq_k, 64);
  const size_t n = (size_t)z.batch_m * z.heads_m;
  z.rows_off = 0;
  z.cols_off = align_up(n * p->seq_q * z.row_words * 4);
  z.layout_off = z.cols_off + (with_cols ? align_up(n * p->seq_k * z.col_words * 4) : 0);
  z.total = z.layout_off + align_up(n * z.nb_q * z.nb_k);
  return z;
}

// Packs the caller's byte mask into the workspace region at `base` and returns the bit views.
hipError_t pack_dense(const attn_problem* p, const attn_mask* m, const DenseSizes& z, char* base, bool with_cols,
                      DenseBits* bits, const uint8_t** layout, int64_t* layout_sb, int64_t* layout_sh,
                      hipStream_t s) {
  DensePackParams dp;
  std::memset(&dp, 0, sizeof(dp));
  dp.mask = m->dense;
  dp.stride_b = m->dense_stride_b;
  dp.stride_h = m->dense_stride_h;
  dp.batch_m = z.batch_m; dp.heads_m = z.heads_m;
  dp.seq_q = p->seq_q; dp.seq_k = p->seq_k; dp.nb_q = z.nb_q; dp.nb_k = z.nb_k;
  dp.row_bits = (uint32_t*)(base + z.rows_off);
  dp.col_bits = with_cols ? (uint32_t*)(base + z.cols_off) : nullptr;
  dp.row_words = z.row_words; dp.col_words = z.col_words;
  dp.layout = (uint8_t*)(base + z.layout_off);
  std::memset(bits, 0, sizeof(*bits));
  bits->rows = dp.row_bits;
  bits->cols = dp.col_bits;
  bits->row_words = z.row_words;
  bits->col_words = z.col_words;
  bits->rows_stride_h = m->dense_stride_h != 0 ? (int64_t)p->seq_q * z.row_words : 0;
  bits->rows_stride_b = m->dense_stride_b != 0 ? (int64_t)z.heads_m * p->seq_q * z.row_words : 0;
  bits->cols_stride_h = m->dense_stride_h != 0 ? (int64_t)p->seq_k * z.col_words : 0;
  bits->cols_stride_b = m->dense_stride_b != 0 ? (int64_t)z.heads_m * p->seq_k * z.col_words : 0;
  *layout = dp.layout;
  *layout_sh = m->dense_stride_h != 0 ? (int64_t)z.nb_q * z.nb_k : 0;
  *layout_sb = m->dense_stride_b != 0 ? (int64_t)z.heads_m * z.nb_q * z.nb_k : 0;
  return launch_dense_pack(dp, s);
}

int fwd_tile_m(const attn_problem* p, const attn_mask* m) {
  if (p->dtype == ATTN_F32) return fwd_f32_block_m();
  if (p->dtype == ATTN_FP8_E4M3) return fwd_fp8_block_m();
  return fwd_bf16_block_m(p->head_dim, m->kind);
}

bool fwd_needs_plan(const attn_problem* p, const attn_mask* m) {
  return p->dtype != ATTN_F32 &&
         (m->kind == ATTN_MASK_PADDING || m->kind == ATTN_MASK_BLOCK || m->kind == ATTN_MASK_DENSE);
}

int64_t fwd_items(const attn_problem* p, const attn_mask* m) {
  return (int64_t)p->batch * p->heads_q * ceil_div(p->seq_q, fwd_tile_m(p, m));
}

// Compute units and XCDs of the current device, queried once per device (plain attribute queries:
// nothing is allocated). MI355X in its single-partition mode has 256 CUs in 8 XCDs, and the
// dispatcher deals workgroup w to XCD w % 8; a partition mode exposes fewer of both. Without a
// device (host-only size queries) the single-partition MI355X figures are used; if a query fails on
// a device, the kernels get one XCD (no per-XCD grouping) and 256 CUs.
struct DeviceInfo {
  int32_t cus, xcds;
};
constexpr int kMaxDevices = 64;
std::atomic<int32_t> g_device_info[kMaxDevices];   // cus << 8 | xcds; 0 = not yet queried

DeviceInfo device_info() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return DeviceInfo{256, 8};
  }
  if (dev >= kMaxDevices) return DeviceInfo{256, 1};
  int32_t v = g_device_info[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1 ||
        xcds > kMaxXcd || cus % xcds != 0)
      xcds = 1;
    (void)hipGetLastError();
    v = (std::min(cus, 1 << 22) << 8) | xcds;
    g_device_info[dev].store(v, std::memory_order_relaxed);
  }
  return DeviceInfo{v >> 8, v & 0xff};
}

// Workgroups that share one item's key range (split-KV). requested: 0 = choose, 1 = never split,
// n = n splits (at most one per 64-key tile). The automatic choice splits only when there are
// fewer items than CUs, aiming at about two workgroups per CU and keeping at least 8 key tiles per
// split so that the merge stays small next to the split's work. Measured on MI355X (256 CUs):
// 128 items of 128 queries x 32768 keys run 1.55x faster with 4 splits; 256 items of 128 x 16384
// run 6% slower with 2 splits than without.
constexpr int kMaxSplits = 32;
int32_t fwd_splits(const attn_problem* p, const attn_mask* m, int32_t requested) {
  if (p->dtype == ATTN_F32 || requested == 1) return 1;
  const int32_t kv_tiles = ceil_div(p->seq_k, 64);
  if (requested > 1) return std::max(1, std::min(requested, kv_tiles));
  const int64_t items = fwd_items(p, m);
  const int64_t cus = device_info().cus;
  if (items >= cus) return 1;
  int64_t n = (2 * cus + items - 1) / items;
  n = std::min<int64_t>(n, kv_tiles / 8);
  n = std::min<int64_t>(n, kMaxSplits);
  return n >= 2 ? (int32_t)n : 1;
}

struct FwdSizes {
  size_t plan_bytes, pairs_off, pairs_bytes, dense_off, o_part_off, lse_part_off, total;
  DenseSizes dense;
};

// Whether the forward's planner pairs layout rows into its 128-row query tiles (bf16 inputs, a
// block layout shared by every (batch, head); see plan_pairs_rows).
bool fwd_pairs_rows(const attn_problem* p, const attn_mask* m) {
  if (p->dtype != ATTN_BF16 || m->kind != ATTN_MASK_BLOCK) return false;
  const int bm = fwd_tile_m(p, m);
  return plan_pairs_rows(MASK_BLOCK, m->layout_stride_b, m->layout_stride_h, bm, ceil_div(p->seq_q, bm),
                         ceil_div(p->seq_q, 64), ceil_div(p->seq_k, 64));
}

// Forward workspace: planner items, the planner's row pairs, packed dense mask, split-KV partials.
FwdSizes fwd_sizes(const attn_problem* p, const attn_mask* m, int32_t splits) {
  FwdSizes z{};
  z.plan_bytes = fwd_needs_plan(p, m) ? align_up((size_t)fwd_items(p, m) * 4) : 0;
  z.pairs_off = z.plan_bytes;
  z.pairs_bytes = fwd_pairs_rows(p, m) ? align_up((size_t)ceil_div(p->seq_q, fwd_tile_m(p, m)) * 4) : 0;
  z.dense = dense_sizes(p, m, false);
  z.dense_off = z.pairs_off + z.pairs_bytes;
  z.o_part_off = z.lse_part_off = z.total = z.dense_off + z.dense.total;
  if (splits > 1) {
    const size_t rows = (size_t)p->batch * p->heads_q * p->seq_q;
    z.lse_part_off = z.o_part_off + align_up((size_t)splits * rows * p->head_dim * 4);
    z.total = z.lse_part_off + align_up((size_t)splits * rows * 4);
  }
  return z;
}

attn_status check_splits(const attn_problem* p, const attn_mask* m, int32_t requested) {
  if (requested < 0 || requested > kMaxSplits) return ATTN_ERR_SHAPE;
  if (requested > 1 && p->dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (fwd_items(p, m) * fwd_splits(p, m, requested) >= (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

struct BwdSizes {
  int dkdv;    // dK/dV kernel variant (DKDV_*)
  int bq, bk, n_qt, n_kt;
  int64_t q_items, kv_items;
  size_t delta_off, lse2_off, sseed_off, kv_off, q_off, pairs_off, dq_acc_off, dense_off, total;
  bool pairs;  // the dQ list pairs layout rows (see plan_pairs_rows)
  DenseSizes dense;
};

// Two-pass layout: -Delta, LSE*log2(e), -LSE/scale (wave-pair dK/dV kernel only), dK/dV items, dQ
// items, the dQ list's row pairs (when paired). Single pass (ATTN_BWD_ATOMIC_DQ): -Delta, LSE*log2(e),
// dK/dV items, then the fp32 dQ accumulator [B, Hq, Sq, D]. A dense mask's packed bits follow either.
BwdSizes bwd_sizes(const attn_problem* p, const attn_mask* m, int32_t flags = 0) {
  BwdSizes s;
  s.dkdv = bwd_dkdv_variant(m->kind, flags, p->heads_q / p->heads_kv, ceil_div(p->seq_q, 64));
  s.bq = bwd_block_q(p->head_dim, m->kind);
  s.bk = bwd_block_k(p->head_dim, m->kind, s.dkdv);
  s.n_qt = ceil_div(p->seq_q, s.bq);
  s.n_kt = ceil_div(p->seq_k, s.bk);
  s.q_items = (int64_t)p->batch * p->heads_q * s.n_qt;
  s.kv_items = (int64_t)p->batch * p->heads_kv * s.n_kt;
  s.delta_off = 0;
  s.lse2_off = align_up((size_t)p->batch * p->heads_q * p->seq_q * 4);
  s.sseed_off = s.lse2_off + align_up((size_t)p->batch * p->heads_q * p->seq_q * 4);
  s.kv_off = s.sseed_off + (s.dkdv != DKDV_ONE_WAVE ? align_up((size_t)p->batch * p->heads_q * p->seq_q * 4) : 0);
  s.q_off = s.kv_off + align_up((size_t)s.kv_items * 4);
  s.pairs = false;
  s.pairs_off = 0;
  if (flags & ATTN_BWD_ATOMIC_DQ) {
    s.dq_acc_off = s.q_off;
    s.total = s.dq_acc_off + align_up((size_t)p->batch * p->heads_q * p->seq_q * p->head_dim * 4);
  } else {
    s.dq_acc_off = 0;
    s.total = s.q_off + align_up((size_t)s.q_items * 4);
    s.pairs = m->kind == ATTN_MASK_BLOCK &&
              plan_pairs_rows(MASK_BLOCK, m->layout_stride_b, m->layout_stride_h, s.bq, s.n_qt, ceil_div(p->seq_q, 64),
                              ceil_div(p->seq_k, 64));
    if (s.pairs) {
      s.pairs_off = s.total;
      s.total += align_up((size_t)s.n_qt * 4);
    }
  }
  // a dense mask's bits (rows and columns) and block layout follow
  s.dense = dense_sizes(p, m, true);
  s.dense_off = s.total;
  s.total += s.dense.total;
  return s;
}

// Problems the backward supports beyond check_problem: bf16, and for block and dense masks at most
// bwd_max_steps() listed (query head, layout row) pairs per key column (6 + 10 bits each).
attn_status check_bwd_support(const attn_problem* p, const attn_mask* m) {
  if (p->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (m->kind == ATTN_MASK_BLOCK || m->kind == ATTN_MASK_DENSE) {
    const int64_t nbq = ceil_div(p->seq_q, 64), group = p->heads_q / p->heads_kv;
    if (nbq > 1024 || group > 63 || group * nbq > bwd_max_steps()) return ATTN_ERR_UNSUPPORTED;
  }
  return ATTN_OK;
}

// The bytes of the caller's mask data (lengths, layout or dense mask; empty for none and causal).
Range mask_data_range(const attn_problem* p, const attn_mask* m) {
  if (m->kind == ATTN_MASK_PADDING) return range_of(m->lengths, (size_t)p->batch * 4);
  if (m->kind == ATTN_MASK_BLOCK) return range_of(m->block_layout, (size_t)layout_bytes(p, m));
  if (m->kind == ATTN_MASK_DENSE) return range_of(m->dense, (size_t)dense_bytes(p, m));
  return Range{0, 0};
}

// Planner parameters of the backward's two lists (into workspace `ws` laid out by bs), on a block
// layout (the caller's, or one derived from a dense mask) with these strides.
void bwd_plan_params(const attn_problem* p, const attn_mask* m, const BwdSizes& bs, const uint8_t* layout,
                     int64_t layout_stride_b, int64_t layout_stride_h, char* ws, PlanParams* pk, PlanParams* pq) {
  PlanParams pp;
  std::memset(&pp, 0, sizeof(pp));
  pp.mask = m->kind == ATTN_MASK_DENSE ? ATTN_MASK_BLOCK : m->kind;
  pp.group = p->heads_q / p->heads_kv; pp.seq_q = p->seq_q; pp.seq_k = p->seq_k;
  pp.nb_q = ceil_div(p->seq_q, 64); pp.nb_k = ceil_div(p->seq_k, 64);
  pp.lengths = m->lengths; pp.layout = layout;
  pp.layout_stride_b = layout_stride_b; pp.layout_stride_h = layout_stride_h;
  pp.n_xcd = device_info().xcds;
  *pk = pp;
  *pq = pp;
  pk->mode = PLAN_BWD_KV; pk->heads = p->heads_kv; pk->n_tiles = bs.n_kt; pk->tile = bs.bk;
  pk->n_items = (int32_t)bs.kv_items; pk->items = (uint32_t*)(ws + bs.kv_off);
  pq->mode = PLAN_FWD_Q; pq->heads = p->heads_q; pq->n_tiles = bs.n_qt; pq->tile = bs.bq;
  pq->n_items = (int32_t)bs.q_items; pq->items = (uint32_t*)(ws + bs.q_off);
  pq->row_pairs = bs.pairs ? (uint16_t*)(ws + bs.pairs_off) : nullptr;
}

attn_status hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Optional per-class event brackets (attn_set_timing_events).
struct TimingSlot {
  void* const* start = nullptr;
  void* const* stop = nullptr;
  int32_t capacity = 0;
  int32_t* count = nullptr;
};
TimingSlot g_timing[ATTN_KERNEL_CLASSES];

// Runs `launch` bracketed by the class's events when a hook is set.
template <typename F>
hipError_t timed(int cls, hipStream_t s, F&& launch) {
  TimingSlot& t = g_timing[cls];
  const bool on = t.capacity > 0 && t.count != nullptr && *t.count < t.capacity;
  if (on) {
    hipError_t e = hipEventRecord((hipEvent_t)t.start[*t.count], s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch();
  if (on && e == hipSuccess) {
    e = hipEventRecord((hipEvent_t)t.stop[*t.count], s);
    ++*t.count;
  }
  return e;
}

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid sizes (dimension < 1, heads_q not a multiple of heads_kv, seq_q != seq_k for a causal mask, or scale not finite and >= 0)";
    case ATTN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case ATTN_ERR_DTYPE: return "unknown dtype";
    case ATTN_ERR_MASK: return "invalid mask descriptor (unknown kind, missing lengths, layout or dense mask, block size other than 64, negative stride)";
    case ATTN_ERR_WORKSPACE: return "workspace too small or missing";
    case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case ATTN_ERR_UNSUPPORTED: return "valid but unsupported problem (head_dim must be 64 or 128; sizes beyond the 32-bit slice limit; backward needs bf16)";
    case ATTN_ERR_HIP: return "the HIP runtime reported an error";
    case ATTN_ERR_TOO_LARGE:
      return "the problem's backward workspace exceeds the fixed scratch array of attn_bwd_noalloc "
             "(attn_bwd_noalloc_scratch_bytes); call attn_bwd with a workspace instead";
  }
  return "unknown status";
}

int32_t attn_version(void) { return 103; }

attn_status attn_set_timing_events(int32_t kernel_class, void* const* start_events, void* const* stop_events,
                                   int32_t capacity, int32_t* count) {
  if (kernel_class < 0 || kernel_class >= ATTN_KERNEL_CLASSES) return ATTN_ERR_SHAPE;
  TimingSlot& t = g_timing[kernel_class];
  if (capacity <= 0 || start_events == nullptr || stop_events == nullptr) {
    t = TimingSlot{};
    return ATTN_OK;
  }
  if (count == nullptr) return ATTN_ERR_NULL;
  t.start = start_events;
  t.stop = stop_events;
  t.capacity = capacity;
  t.count = count;
  return ATTN_OK;
}

size_t attn_fwd_ex_workspace_bytes(const attn_problem* problem, const attn_mask* mask, int32_t kv_splits) {
  if (problem == nullptr) return 0;
  const attn_mask* m = mask ? mask : &kNoMask;
  if (check_problem(problem, m, 1.0f) != ATTN_OK || check_splits(problem, m, kv_splits) != ATTN_OK) return 0;
  return fwd_sizes(problem, m, fwd_splits(problem, m, kv_splits)).total;
}

size_t attn_fwd_workspace_bytes(const attn_problem* problem, const attn_mask* mask) {
  return attn_fwd_ex_workspace_bytes(problem, mask, 0);
}

int32_t attn_fwd_kv_splits(const attn_problem* problem, const attn_mask* mask, int32_t kv_splits) {
  if (problem == nullptr) return 0;
  const attn_mask* m = mask ? mask : &kNoMask;
  if (check_problem(problem, m, 1.0f) != ATTN_OK || check_splits(problem, m, kv_splits) != ATTN_OK) return 0;
  return fwd_splits(problem, m, kv_splits);
}

attn_status attn_fwd(const attn_problem* problem, const void* Q, const void* K, const void* V,
                     const attn_mask* mask, float scale, void* O, float* LSE, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return attn_fwd_ex(problem, Q, K, V, mask, scale, O, LSE, workspace, workspace_bytes, 0, stream);
}

attn_status attn_fwd_ex(const attn_problem* problem, const void* Q, const void* K, const void* V,
                        const attn_mask* mask, float scale, void* O, float* LSE, void* workspace,
                        size_t workspace_bytes, int32_t kv_splits, void* stream) {
  return attn::fwd_call(problem, Q, K, V, mask, scale, O, LSE, workspace, workspace_bytes, kv_splits, nullptr, 0,
                        false, stream);
}

attn_status attn_fwd_with_bwd_plan(const attn_problem* problem, const void* Q, const void* K, const void* V,
                                   const attn_mask* mask, float scale, void* O, float* LSE, void* workspace,
                                   size_t workspace_bytes, void* bwd_workspace, size_t bwd_workspace_bytes,
                                   void* stream) {
  return attn::fwd_call(problem, Q, K, V, mask, scale, O, LSE, workspace, workspace_bytes, 0, bwd_workspace,
                        bwd_workspace_bytes, true, stream);
}

}  // extern "C"

namespace attn {

attn_status fwd_call(const attn_problem* problem, const void* Q, const void* K, const void* V,
                     const attn_mask* mask, float scale, void* O, float* LSE, void* workspace,
                     size_t workspace_bytes, int32_t kv_splits, void* bwd_workspace, size_t bwd_workspace_bytes,
                     bool plan_bwd, void* stream) {
  if (problem == nullptr || Q == nullptr || K == nullptr || V == nullptr || O == nullptr || LSE == nullptr)
    return ATTN_ERR_NULL;
  if (plan_bwd && bwd_workspace == nullptr) return ATTN_ERR_NULL;
  const attn_mask* m = mask ? mask : &kNoMask;
  const attn_problem* p = problem;
  attn_status st = check_problem(p, m, scale);
  if (st != ATTN_OK) return st;
  st = check_splits(p, m, kv_splits);
  if (st != ATTN_OK) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return ATTN_ERR_ALIGN;
  const int32_t splits = fwd_splits(p, m, kv_splits);
  const FwdSizes fz = fwd_sizes(p, m, splits);
  const size_t need = fz.total;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return ATTN_ERR_ALIGN;

  const size_t es = elem_size(p->dtype);
  const size_t qbytes = (size_t)p->batch * p->heads_q * p->seq_q * p->head_dim * es;
  const size_t kvbytes = (size_t)p->batch * p->heads_kv * p->seq_k * p->head_dim * es;
  const Range rq = range_of(Q, qbytes), rk = range_of(K, kvbytes), rv = range_of(V, kvbytes);
  const size_t obytes = (size_t)p->batch * p->heads_q * p->seq_q * p->head_dim * out_elem_size(p->dtype);
  const Range ro = range_of(O, obytes), rl = range_of(LSE, (size_t)p->batch * p->heads_q * p->seq_q * 4);
  const Range rw = range_of(workspace, need);
  for (Range out : {ro, rl}) {
    if (overlap(out, rq) || overlap(out, rk) || overlap(out, rv)) return ATTN_ERR_ALIAS;
  }
  if (overlap(ro, rl)) return ATTN_ERR_ALIAS;
  if (need > 0) {
    for (Range r : {rq, rk, rv, ro, rl})
      if (overlap(rw, r)) return ATTN_ERR_ALIAS;
  }
  if (m->kind == ATTN_MASK_PADDING) {
    const Range rlen = range_of(m->lengths, (size_t)p->batch * 4);
    if (overlap(rlen, ro) || overlap(rlen, rl) || (need > 0 && overlap(rlen, rw))) return ATTN_ERR_ALIAS;
  }
  if (m->kind == ATTN_MASK_BLOCK) {
    const Range rlay = range_of(m->block_layout, (size_t)layout_bytes(p, m));
    if (overlap(rlay, ro) || overlap(rlay, rl) || (need > 0 && overlap(rlay, rw))) return ATTN_ERR_ALIAS;
  }
  if (m->kind == ATTN_MASK_DENSE) {
    const Range rden = range_of(m->dense, (size_t)dense_bytes(p, m));
    if (overlap(rden, ro) || overlap(rden, rl) || (need > 0 && overlap(rden, rw))) return ATTN_ERR_ALIAS;
  }
  // the backward's lists: a problem the backward supports, and a workspace of its size that
  // overlaps nothing else of the call
  BwdSizes bs{};
  if (plan_bwd) {
    st = check_bwd_support(p, m);
    if (st != ATTN_OK) return st;
    bs = bwd_sizes(p, m, 0);
    if (bwd_workspace_bytes < bs.total) return ATTN_ERR_WORKSPACE;
    if (!aligned16(bwd_workspace)) return ATTN_ERR_ALIGN;
    const Range rb = range_of(bwd_workspace, bs.total);
    for (Range r : {rq, rk, rv, ro, rl})
      if (overlap(rb, r)) return ATTN_ERR_ALIAS;
    if (need > 0 && overlap(rb, rw)) return ATTN_ERR_ALIAS;
    if (overlap(rb, mask_data_range(p, m))) return ATTN_ERR_ALIAS;
  }

  // ---- launch ----
  hipStream_t s = (hipStream_t)stream;
  const int bm = fwd_tile_m(p, m);
  FwdParams fp;
  std::memset(&fp, 0, sizeof(fp));
  fp.q = Q; fp.k = K; fp.v = V; fp.o = O; fp.lse = LSE;
  fp.lengths = m->lengths;
  fp.layout = m->block_layout;
  fp.layout_stride_b = m->layout_stride_b;
  fp.layout_stride_h = m->layout_stride_h;
  fp.batch = p->batch; fp.heads_q = p->heads_q; fp.heads_kv = p->heads_kv;
  fp.seq_q = p->seq_q; fp.seq_k = p->seq_k;
  fp.group = p->heads_q / p->heads_kv;
  fp.n_qtiles = ceil_div(p->seq_q, bm);
  fp.n_items = p->batch * p->heads_q * fp.n_qtiles;
  fp.nb_q = ceil_div(p->seq_q, 64);
  fp.nb_k = ceil_div(p->seq_k, 64);
  fp.scale = scale;
  // kernels rely on scale*log2(e) > 0 (masked scores are -inf); scale 0 runs as 1e-30, which
  // changes no score by more than 1e-29 relative
  fp.scale_log2 = (scale > 0.0f ? scale : 1e-30f) * 1.4426950408889634f;
  fp.dense_bytes = m->dense;
  fp.dense_stride_b = m->dense_stride_b;
  fp.dense_stride_h = m->dense_stride_h;
  fp.kv_splits = splits;
  fp.n_xcd = device_info().xcds;
  if (splits > 1) {
    fp.o_part = (float*)((char*)workspace + fz.o_part_off);
    fp.lse_part = (float*)((char*)workspace + fz.lse_part_off);
  }

  if (p->dtype == ATTN_F32)
    return hip_status(timed(ATTN_KERNEL_FWD, s, [&] { return launch_fwd_f32(fp, p->head_dim, m->kind, s); }));

  if (m->kind == ATTN_MASK_DENSE) {
    // the dense mask becomes bits plus a block layout, which the planner and kernels then use
    st = hip_status(timed(ATTN_KERNEL_MASK_PACK, s, [&] {
      return pack_dense(p, m, fz.dense, (char*)workspace + fz.dense_off, false, &fp.dense, &fp.layout,
                        &fp.layout_stride_b, &fp.layout_stride_h, s);
    }));
    if (st != ATTN_OK) return st;
  }
  // the backward's two lists, planned on the same layout the forward plans on
  PlanParams pk, pq;
  if (plan_bwd)
    bwd_plan_params(p, m, bs, fp.layout, fp.layout_stride_b, fp.layout_stride_h, (char*)bwd_workspace, &pk, &pq);
  if (fz.plan_bytes > 0) {
    PlanParams pp;
    std::memset(&pp, 0, sizeof(pp));
    pp.mode = PLAN_FWD_Q; pp.mask = m->kind == ATTN_MASK_DENSE ? ATTN_MASK_BLOCK : m->kind;
    pp.heads = p->heads_q; pp.group = fp.group;
    pp.seq_q = p->seq_q; pp.seq_k = p->seq_k; pp.n_tiles = fp.n_qtiles; pp.tile = bm;
    pp.n_items = fp.n_items; pp.nb_q = fp.nb_q; pp.nb_k = fp.nb_k;
    pp.lengths = m->lengths; pp.layout = fp.layout;
    pp.layout_stride_b = fp.layout_stride_b; pp.layout_stride_h = fp.layout_stride_h;
    pp.items = (uint32_t*)workspace;
    pp.n_xcd = fp.n_xcd;
    pp.row_pairs = fz.pairs_bytes > 0 ? (uint16_t*)((char*)workspace + fz.pairs_off) : nullptr;
    st = hip_status(timed(ATTN_KERNEL_PLAN, s, [&] {
      return plan_bwd ? launch_plan_triple(pp, pk, pq, s) : launch_plan(pp, s);
    }));
    if (st != ATTN_OK) return st;
    fp.items = (const uint32_t*)workspace;
    fp.row_pairs = pp.row_pairs;
  } else if (plan_bwd) {
    // the forward orders its items in closed form; the backward's lists still need a launch
    st = hip_status(timed(ATTN_KERNEL_PLAN, s, [&] { return launch_plan_pair(pk, pq, s); }));
    if (st != ATTN_OK) return st;
  }
  if (p->dtype == ATTN_FP8_E4M3)
    st = hip_status(timed(ATTN_KERNEL_FWD, s, [&] { return launch_fwd_fp8(fp, p->head_dim, m->kind, s); }));
  else
    st = hip_status(timed(ATTN_KERNEL_FWD, s, [&] { return launch_fwd_bf16(fp, p->head_dim, m->kind, s); }));
  if (st != ATTN_OK || splits == 1) return st;
  return hip_status(timed(ATTN_KERNEL_FWD_MERGE, s, [&] { return launch_fwd_merge(fp, p->head_dim, s); }));
}

}  // namespace attn

extern "C" {

size_t attn_bwd_ex_workspace_bytes(const attn_problem* problem, const attn_mask* mask, int32_t flags) {
  if (problem == nullptr) return 0;
  const attn_mask* m = mask ? mask : &kNoMask;
  if (check_problem(problem, m, 1.0f) != ATTN_OK) return 0;
  if (problem->dtype != ATTN_BF16 || (flags & ~(ATTN_BWD_ATOMIC_DQ | ATTN_BWD_PLANNED)) != 0) return 0;
  if ((flags & ATTN_BWD_ATOMIC_DQ) && (flags & ATTN_BWD_PLANNED)) return 0;
  return bwd_sizes(problem, m, flags & ATTN_BWD_ATOMIC_DQ).total;
}

size_t attn_bwd_workspace_bytes(const attn_problem* problem, const attn_mask* mask) {
  return attn_bwd_ex_workspace_bytes(problem, mask, 0);
}

attn_status attn_bwd(const attn_problem* problem, const void* Q, const void* K, const void* V, const void* O,
                     const void* dO, const float* LSE, const attn_mask* mask, float scale, void* dQ, void* dK,
                     void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_ex(problem, Q, K, V, O, dO, LSE, mask, scale, dQ, dK, dV, workspace, workspace_bytes, 0, stream);
}

attn_status attn_bwd_ex(const attn_problem* problem, const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* LSE, const attn_mask* mask, float scale, void* dQ, void* dK,
                        void* dV, void* workspace, size_t workspace_bytes, int32_t flags, void* stream) {
  return attn::bwd_call(problem, Q, K, V, O, dO, LSE, mask, scale, dQ, dK, dV, workspace, workspace_bytes, flags,
                        stream, nullptr);
}

}  // extern "C"

namespace attn {

attn_status bwd_call(const attn_problem* problem, const void* Q, const void* K, const void* V, const void* O,
                     const void* dO, const float* LSE, const attn_mask* mask, float scale, void* dQ, void* dK,
                     void* dV, void* workspace, size_t workspace_bytes, int32_t flags, void* stream,
                     WorkspaceProvider provide) {
  if (problem == nullptr || Q == nullptr || K == nullptr || V == nullptr || O == nullptr || dO == nullptr ||
      LSE == nullptr || dQ == nullptr || dK == nullptr || dV == nullptr)
    return ATTN_ERR_NULL;
  const attn_mask* m = mask ? mask : &kNoMask;
  const attn_problem* p = problem;
  attn_status st = check_problem(p, m, scale);
  if (st != ATTN_OK) return st;
  if ((flags & ~(ATTN_BWD_ATOMIC_DQ | ATTN_BWD_PLANNED)) != 0) return ATTN_ERR_SHAPE;
  const bool atomic_dq = (flags & ATTN_BWD_ATOMIC_DQ) != 0;
  const bool planned = (flags & ATTN_BWD_PLANNED) != 0;
  if (atomic_dq && planned) return ATTN_ERR_UNSUPPORTED;
  st = check_bwd_support(p, m);
  if (st != ATTN_OK) return st;
  for (const void* ptr : {Q, K, V, O, dO, (const void*)LSE, (const void*)dQ, (const void*)dK, (const void*)dV})
    if (!aligned16(ptr)) return ATTN_ERR_ALIGN;
  const BwdSizes bs = bwd_sizes(p, m, flags & ATTN_BWD_ATOMIC_DQ);

  const size_t es = 2;
  const size_t qbytes = (size_t)p->batch * p->heads_q * p->seq_q * p->head_dim * es;
  const size_t kvbytes = (size_t)p->batch * p->heads_kv * p->seq_k * p->head_dim * es;
  const Range ins[] = {range_of(Q, qbytes), range_of(K, kvbytes), range_of(V, kvbytes), range_of(O, qbytes),
                       range_of(dO, qbytes), range_of(LSE, (size_t)p->batch * p->heads_q * p->seq_q * 4)};
  Range outs[] = {range_of(dQ, qbytes), range_of(dK, kvbytes), range_of(dV, kvbytes), Range{0, 0}};
  Range mask_range{0, 0};
  if (m->kind == ATTN_MASK_PADDING) mask_range = range_of(m->lengths, (size_t)p->batch * 4);
  if (m->kind == ATTN_MASK_BLOCK) mask_range = range_of(m->block_layout, (size_t)layout_bytes(p, m));
  if (m->kind == ATTN_MASK_DENSE) mask_range = range_of(m->dense, (size_t)dense_bytes(p, m));
  // outputs against inputs, each other and the mask data
  for (int i = 0; i < 3; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return ATTN_ERR_ALIAS;
    if (overlap(mask_range, outs[i])) return ATTN_ERR_ALIAS;
  }
  // the workspace: the caller's, or (for the no-allocation entry point) one the provider names
  if (provide != nullptr) {
    st = provide(bs.total, &workspace, &workspace_bytes);
    if (st != ATTN_OK) return st;
  }
  if (workspace == nullptr || workspace_bytes < bs.total) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  outs[3] = range_of(workspace, bs.total);
  for (int i = 0; i < 3; ++i)
    if (overlap(outs[3], outs[i])) return ATTN_ERR_ALIAS;
  for (const Range& r : ins)
    if (overlap(outs[3], r)) return ATTN_ERR_ALIAS;
  if (overlap(mask_range, outs[3])) return ATTN_ERR_ALIAS;

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  BwdParams bp;
  std::memset(&bp, 0, sizeof(bp));
  bp.q = Q; bp.k = K; bp.v = V; bp.o = O; bp.dout = dO; bp.lse = LSE;
  bp.dq = dQ; bp.dk = dK; bp.dv = dV;
  bp.delta = (float*)(ws + bs.delta_off);
  bp.lse2 = (float*)(ws + bs.lse2_off);
  bp.sseed = bs.dkdv != DKDV_ONE_WAVE ? (float*)(ws + bs.sseed_off) : nullptr;
  bp.lengths = m->lengths; bp.layout = m->block_layout;
  bp.layout_stride_b = m->layout_stride_b; bp.layout_stride_h = m->layout_stride_h;
  bp.items_kv = (const uint32_t*)(ws + bs.kv_off);
  bp.items_q = (const uint32_t*)(ws + bs.q_off);
  bp.row_pairs = bs.pairs ? (const uint16_t*)(ws + bs.pairs_off) : nullptr;
  bp.batch = p->batch; bp.heads_q = p->heads_q; bp.heads_kv = p->heads_kv;
  bp.seq_q = p->seq_q; bp.seq_k = p->seq_k;
  bp.group = p->heads_q / p->heads_kv;
  bp.n_qtiles = bs.n_qt; bp.n_ktiles = bs.n_kt;
  bp.nb_q = ceil_div(p->seq_q, 64); bp.nb_k = ceil_div(p->seq_k, 64);
  bp.scale = scale;
  bp.scale_log2 = (scale > 0.0f ? scale : 1e-30f) * 1.4426950408889634f;
  bp.inv_scale_log2 = 1.0f / bp.scale_log2;
  if (atomic_dq) bp.dq_acc = (float*)(ws + bs.dq_acc_off);

  if (m->kind == ATTN_MASK_DENSE) {
    // the dense mask becomes bits plus a block layout, which the planner and kernels then use
    st = hip_status(timed(ATTN_KERNEL_MASK_PACK, s, [&] {
      return pack_dense(p, m, bs.dense, ws + bs.dense_off, true, &bp.dense, &bp.layout, &bp.layout_stride_b,
                        &bp.layout_stride_h, s);
    }));
    if (st != ATTN_OK) return st;
  }

  // dK/dV items (b, kv head, key tile) and dQ items (b, query head, query tile), one launch (none
  // when the forward of the pair already wrote them into this workspace)
  PlanParams pk, pq;
  bwd_plan_params(p, m, bs, bp.layout, bp.layout_stride_b, bp.layout_stride_h, ws, &pk, &pq);
  if (atomic_dq)
    st = hip_status(timed(ATTN_KERNEL_PLAN, s, [&] { return launch_plan(pk, s); }));
  else if (!planned)
    st = hip_status(timed(ATTN_KERNEL_PLAN, s, [&] { return launch_plan_pair(pk, pq, s); }));
  if (st != ATTN_OK) return st;

  if (atomic_dq) {
    // single pass: the preprocess writes the row statistics and zeroes the dQ accumulator
    st = hip_status(timed(ATTN_KERNEL_BWD_PRE, s, [&] { return launch_bwd_preprocess(bp, p->head_dim, s); }));
    if (st != ATTN_OK) return st;
    st = hip_status(timed(ATTN_KERNEL_BWD_DKDV, s,
                          [&] { return launch_bwd_dkdv(bp, p->head_dim, m->kind, (int)bs.kv_items, s); }));
    if (st != ATTN_OK) return st;
    return hip_status(timed(ATTN_KERNEL_BWD_DQ_CONVERT, s, [&] { return launch_bwd_dq_convert(bp, p->head_dim, s); }));
  }
  // two passes: the dQ pass computes the row statistics (-Delta, LSE*log2(e)) of its queries as it
  // starts and writes them for the dK/dV pass, so it runs first and no preprocess is launched
  st = hip_status(
      timed(ATTN_KERNEL_BWD_DQ, s, [&] { return launch_bwd_dq(bp, p->head_dim, m->kind, (int)bs.q_items, s); }));
  if (st != ATTN_OK) return st;
  return hip_status(timed(ATTN_KERNEL_BWD_DKDV, s, [&] {
    if (bs.dkdv == DKDV_PAIR) return launch_bwd_dkdv_pair(bp, p->head_dim, m->kind, (int)bs.kv_items, s);
    return launch_bwd_dkdv(bp, p->head_dim, m->kind, (int)bs.kv_items, s);
  }));
}

}  // namespace attn
