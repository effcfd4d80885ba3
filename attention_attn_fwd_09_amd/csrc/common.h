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

// Workgroup barrier that publishes LDS writes only: this wave's LDS operations complete, then
// s_barrier. Unlike __syncthreads it does not wait for outstanding global loads, so loads issued
// before it (a workgroup's row fragments) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt fields at their maximum
  asm volatile("s_barrier" ::: "memory");
}

// --- LDS tiles: 64 rows x D bf16, rows of D*2 bytes, 16-byte chunks XOR-swizzled per row ---
// LDS serves 256 bytes per clock from 64 four-byte banks; a 16-byte chunk's bank group is
// (byte offset / 16) mod 16. Tiles are read in two patterns:
//  * row fragments (ds_read_b128): 16 lanes read the same logical chunk of 16 different rows,
//    rows {0-3,16-19,4-7,20-23} or {8-11,24-27,12-15,28-31} (+32) of the sigma32 permutation;
//  * transposed fragments (ds_read_b64_tr_b16): 32 lanes read 4 consecutive rows (aligned to 4)
//    times 4 consecutive chunks.
// swz<D>(row) gives both patterns 16 distinct bank groups: its bits 2-3 (D=128) or bit 2 (D=64,
// where two rows share one 256-byte bank span) follow the row's position inside its group of 4,
// and its low bits separate the four 4-row groups of a row-fragment read. Writes fill one row's
// chunks per 16 lanes, which any per-row XOR permutes without conflict.
// ds_read_b64_tr_b16 works on 16-lane groups: the 4 rows of one read are each assembled from 4
// lanes' 8-byte pieces (lanes 4r..4r+3 supply row r) and lane i receives element i of every row,
// so two reads give a lane 8 consecutive rows of one column (an MFMA operand along the rows).
template <int D> __device__ __forceinline__ int swz(int row);
template <> __device__ __forceinline__ int swz<128>(int row) {
  return ((row & 3) << 2) | ((row >> 2) & 1) | ((row >> 3) & 2);
}
template <> __device__ __forceinline__ int swz<64>(int row) {
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 1) | ((row >> 3) & 2);
}

// Copy rows [row0, row0 + 64) of a [rows][D] bf16 tensor (buffer descriptor r) into an LDS tile.
// All NW*64 threads of the workgroup take part; rows past the end of the buffer read as 0.
template <int D, int NW>
__device__ __forceinline__ void issue_rows(char* lds_tile, __amdgpu_buffer_rsrc_t r, int row0, int wave, int lane) {
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int ROUNDS = (64 * CPR) / (NW * 64);
#pragma unroll
  for (int it = 0; it < ROUNDS; ++it) {
    const int blk = it * NW + wave;                // 64-chunk (1 KiB) block written by this wave
    const int pos = blk * 64 + lane;               // physical chunk index in the tile
    const int row = pos / CPR;
    const int pc = pos % CPR;
    buffer_to_lds16(r, lds_tile + blk * 1024, (uint32_t)(row0 + row) * (D * 2) + (uint32_t)((pc ^ swz<D>(row)) * 16));
  }
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row permutation of a 32-key block inside the score MFMA: MFMA row r reads key sigma(r), so that
// in the 32x32 output each half-wave holds 16 consecutive keys of its query column.
__device__ __forceinline__ int sigma32(int r) { return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3); }

// NaN-propagating maximum (v_maximum3_f32 on gfx950). fmaxf would first quiet every operand the
// compiler cannot prove canonical (one extra VALU op per MFMA result).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Eight fp32 values to bf16 (round to nearest even), converted in pairs: four v_cvt_pk_bf16_f32.
// Storing element by element into a vector makes the compiler convert one value per instruction
// and merge the halves with extra permutes.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const bf16x2 h = __builtin_convertvector((f32x2){v[i], v[i + 1]}, bf16x2);
    r[i] = h[0];
    r[i + 1] = h[1];
  }
  return r;
}

// acc + sum of the 8 bf16 values of x, in fp32, four v_dot2 ops against (1, 1)
__device__ __forceinline__ float sum_bf16x8(bf16x8 x, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, acc, false);
}

// --- wavefront helpers ---
__device__ __forceinline__ float partner_max(float x) {
  // value of lane l^32 combined with our own: permlane32_swap(x, x) returns {x[l], x[l^32]} in some order.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Layout row r (0 or 1) of 128-row query tile t: rows 2t and 2t + 1, or the two rows the planner
// paired for the tile (row_pairs[2t + r]). A row index of nb_q or more names no row.
__device__ __forceinline__ int tile_row(const uint16_t* row_pairs, int t, int r) {
  return row_pairs != nullptr ? (int)row_pairs[2 * t + r] : 2 * t + r;
}

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
// The dispatcher deals workgroup i to XCD i % n_xcd; when the (batch, kv-head) units divide evenly
// over the XCDs, all items of one unit go to one XCD so that its K/V stay in that XCD's L2.
__device__ __forceinline__ Item closed_form_item(int i, int batch, int heads_q, int heads_kv, int n_qtiles,
                                                 bool descending, int n_xcd) {
  const int group = heads_q / heads_kv;
  const int units = batch * heads_kv;
  Item r;
  int rank;
  if (n_xcd > 1 && units % n_xcd == 0) {
    const int xcd = i % n_xcd, slot = i / n_xcd;
    const int per_rank = (units / n_xcd) * group;
    rank = slot / per_rank;
    const int rem = slot - rank * per_rank;
    const int unit = xcd + n_xcd * (rem / group);
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

// Split-KV launches kv_splits workgroups per item. Workgroup w runs on XCD w % n_xcd; the item list
// (closed form or planner) places item i on XCD i % n_xcd. So that all splits of an item share its
// XCD's L2, the workgroups of each XCD take that XCD's items in list order, kv_splits consecutive
// workgroups per item. This is a bijection between workgroups and (item, split) pairs whenever
// n_items divides by n_xcd; otherwise workgroups take items in plain order.
__device__ __forceinline__ void split_item(uint32_t w, int n_items, int kv_splits, int n_xcd, int& item_idx,
                                           int& split) {
  if (kv_splits > 1 && n_xcd > 1 && n_items % n_xcd == 0) {
    const uint32_t xcd = w % (uint32_t)n_xcd, slot = w / (uint32_t)n_xcd;
    item_idx = (int)((slot / (uint32_t)kv_splits) * (uint32_t)n_xcd + xcd);
    split = (int)(slot % (uint32_t)kv_splits);
  } else {
    item_idx = (int)(w / (uint32_t)kv_splits);
    split = (int)(w % (uint32_t)kv_splits);
  }
}

__device__ __forceinline__ int clamp_len(int32_t len, int seq) { return len < 0 ? 0 : (len > seq ? seq : len); }

// A dense mask's bits of one row (or column) for the 64 positions k0 .. k0+63: two 32-bit words,
// 0 past the row's words or for a row past the sequence. The dK/dV kernels load them one step
// ahead of the step that tests them, so that the load's latency is spent under the previous step's
// work; the forward and the dQ pass load them in the step that uses them.
__device__ __forceinline__ void dense_words(const uint32_t* row_bits, bool row_ok, int row_words, int k0,
                                            uint32_t (&w)[2]) {
  const int w0 = k0 >> 5;
  w[0] = (row_ok && w0 < row_words) ? row_bits[w0] : 0u;
  w[1] = (row_ok && w0 + 1 < row_words) ? row_bits[w0 + 1] : 0u;
}


// Writes a wave's 32 output rows of D bf16 columns, held in the MFMA accumulator layout of O^T and
// dQ^T (lane (c, hh) holds row c, columns db*32 + g4*8 + hh*4 + 0..3 in acc[db][g4*4 + 0..3]),
// scaled by the lane's factor f, as whole rows: the rows go to `lds` with a row stride of 2D + 8
// bytes, so that consecutive rows start on different banks (the bank-conflict counter reads about a
// third less than with a stride of 2D + 16, and what remains is under 0.5% of a launch's cycles),
// and come back as 8-byte pairs (rows are 8-byte aligned), one 16-byte store per pair. Rows at or
// past `rows` are not written. `lds` holds 32 * (2D + 8) bytes that no other wave touches
// meanwhile.
template <int D>
__device__ __forceinline__ void write_rows_bf16(char* lds, const f32x16 (&acc)[D / 32], float f, int lane, bf16* out,
                                                int rows) {
  constexpr int DB = D / 32, RBP = 2 * D + 8, CPR = 2 * D / 16;
  const int c = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (bf16)(acc[db][g4 * 4 + e] * f);
      *(bf16x4*)(lds + c * RBP + (db * 32 + g4 * 8 + hh * 4) * 2) = v4;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's rows are in LDS
#pragma unroll
  for (int j = 0; j < 32 * CPR / 64; ++j) {
    const int chunk = j * 64 + lane;
    const int r = chunk / CPR, cc = chunk % CPR;
    const char* src = lds + r * RBP + cc * 16;
    const uint2 lo = *(const uint2*)src, hi = *(const uint2*)(src + 8);
    if (r < rows) *(uint4*)(out + (size_t)r * D + cc * 8) = uint4{lo.x, lo.y, hi.x, hi.y};
  }
}

}  // namespace attn
