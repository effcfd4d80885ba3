// Shared device helpers for the gfx950 attention kernels: vector types, LDS swizzles, buffer
// descriptors, mask geometry and the item encoding used by the planner and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "params.h"

namespace attn {

typedef __bf16 bf16;
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// --- buffer descriptors: raw buffers with hardware range checking (out-of-range lanes read 0) ---
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from global memory straight into LDS; lane i's bytes land at lds_base + 16*i.
// lds_base must be wave-uniform.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds_base), 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// --- LDS swizzles of 16-byte chunks within a key row ---
// LDS serves 256 bytes per clock from 64 four-byte banks, so a 16-byte chunk's bank group is its
// byte offset / 16 modulo 16. K tiles are read with ds_read_b128 by 16 lanes at a time from 16
// different rows (keys {0-3,16-19,4-7,20-23} or {8-15,24-31} of a 32-key block, same logical
// chunk): swz_k gives those rows 16 distinct bank groups. V tiles are read with the transposing
// ds_read_b64_tr_b16, 32 lanes at a time from 4 consecutive rows x 4 consecutive chunks: swz_v
// gives those 16 (row, chunk) pairs distinct bank groups. Writes fill one row's chunks per 16
// lanes, which any per-row XOR permutes without conflict.
template <int D> __device__ __forceinline__ int swz_k(int row);
template <> __device__ __forceinline__ int swz_k<128>(int row) { return (row & 7) | ((row >> 1) & 8); }
template <> __device__ __forceinline__ int swz_k<64>(int row) { return ((row >> 1) & 3) | ((row >> 2) & 4); }
template <int D> __device__ __forceinline__ int swz_v(int row);
template <> __device__ __forceinline__ int swz_v<128>(int row) { return (row & 3) << 2; }
template <> __device__ __forceinline__ int swz_v<64>(int row) { return ((row >> 1) & 1) << 2; }

// Row permutation of a 32-key block inside the score MFMA: MFMA row r reads key sigma(r), so that
// in the 32x32 output each half-wave holds 16 consecutive keys of its query column.
__device__ __forceinline__ int sigma32(int r) { return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3); }

// --- wavefront helpers ---
__device__ __forceinline__ float partner_max(float x) {
  // value of lane l^32 combined with our own: permlane32_swap(x, x) returns {x[l], x[l^32]} in some order.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// --- item encoding: item = (b * heads_q + h) * n_qtiles + qtile ---
struct Item {
  int b, h, t;
};
__device__ __forceinline__ Item decode_item(uint32_t it, int heads_q, int n_qtiles) {
  Item r;
  r.t = (int)(it % (uint32_t)n_qtiles);
  uint32_t bh = it / (uint32_t)n_qtiles;
  r.h = (int)(bh % (uint32_t)heads_q);
  r.b = (int)(bh / (uint32_t)heads_q);
  return r;
}

// Closed-form longest-first order for masks whose per-tile cost is known without data (NONE, CAUSAL).
// Workgroup i runs on XCD i % 8; when the (batch, kv-head) units divide evenly over the 8 XCDs, all
// items of one unit go to one XCD so that its K/V stay in that XCD's L2.
__device__ __forceinline__ Item closed_form_item(int i, int batch, int heads_q, int heads_kv, int n_qtiles,
                                                 bool descending) {
  const int group = heads_q / heads_kv;
  const int units = batch * heads_kv;
  Item r;
  int rank;
  if ((units & 7) == 0) {
    const int xcd = i & 7, slot = i >> 3;
    const int per_rank = (units >> 3) * group;
    rank = slot / per_rank;
    const int rem = slot - rank * per_rank;
    const int unit = xcd + 8 * (rem / group);
    r.b = unit / heads_kv;
    r.h = (unit - r.b * heads_kv) * group + rem % group;
  } else {
    const int bh_n = batch * heads_q;
    rank = i / bh_n;
    const int bh = i - rank * bh_n;
    r.b = bh / heads_q;
    r.h = bh - r.b * heads_q;
  }
  r.t = descending ? (n_qtiles - 1 - rank) : rank;
  return r;
}

__device__ __forceinline__ int clamp_len(int32_t len, int seq) { return len < 0 ? 0 : (len > seq ? seq : len); }

}  // namespace attn
