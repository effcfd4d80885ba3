// Tile-list scheduler: orders the work items of one call longest-first.
//
// The report on the Xingchen-Cup sparse FlashAttention operator (smzdm.com), section 03, stresses
// that the kept blocks of a sparse (or causal) mask are unevenly spread, so a static split leaves
// cores idle; the fused-attention write-up (zwxr.cn), section 4.2, finds a dynamic hand-out, where
// a core that is done fetches the next block, faster than a static split. Here the items are sorted
// by cost, longest first, and launched as one workgroup each: the hardware dispatcher hands the next
// item in the list to whichever compute unit frees up first, which is that dynamic policy with a
// longest-processing-time order on top. The same report's opening anecdote (147 microseconds of an
// idle chip spent in a clumsy statistics step) warns that a slow prologue can cost more than it
// saves, so this is one short kernel with one workgroup: a cost histogram in LDS, a scan, and a
// scatter.
//
// Items:
//   FWD_Q / BWD_Q: (b, h_q, q-tile of BM rows), cost = number of 64-key tiles the tile visits.
//   BWD_KV:        (b, h_kv, k-tile of BN rows), cost = number of (query head, q-tile) pairs.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

constexpr int NCOST = 1024;   // cost buckets per XCD; larger costs share the top bucket
constexpr int NBUCKET = kMaxXcd * NCOST;
constexpr int THREADS = 1024;

constexpr int MAX_CACHED = 16384;  // items whose cost is kept in LDS between the passes

// Number of kept tiles in the union of `nrows` consecutive layout rows starting at r0. The loads
// are issued 16 at a time so that their latencies overlap (one dependent load per column would
// make this prologue cost tens of microseconds).
__device__ int layout_row_union_count(const uint8_t* lay, int nb_k, int r0, int nrows, int nb_q) {
  int count = 0;
  for (int j = 0; j < nb_k; j += 16) {
    uint32_t keep = 0;
    for (int r = 0; r < nrows; ++r) {
      const int row = r0 + r;
      if (row >= nb_q) break;
      const uint8_t* rp = lay + (size_t)row * nb_k;
      uint8_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = (j + u < nb_k) ? rp[j + u] : (uint8_t)0;
#pragma unroll
      for (int u = 0; u < 16; ++u) keep |= (v[u] != 0 ? 1u : 0u) << u;
    }
    count += __popc(keep);
  }
  return count;
}

// Number of kept tiles in the union of `ncols` consecutive layout columns starting at c0.
__device__ int layout_col_union_count(const uint8_t* lay, int nb_k, int c0, int ncols, int nb_q) {
  int count = 0;
  for (int i = 0; i < nb_q; i += 16) {
    uint32_t keep = 0;
    for (int cc = 0; cc < ncols; ++cc) {
      const int col = c0 + cc;
      if (col >= nb_k) break;
      uint8_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = (i + u < nb_q) ? lay[(size_t)(i + u) * nb_k + col] : (uint8_t)0;
#pragma unroll
      for (int u = 0; u < 16; ++u) keep |= (v[u] != 0 ? 1u : 0u) << u;
    }
    count += __popc(keep);
  }
  return count;
}

constexpr int MAX_UNITS = 4096;   // tiles whose cost is tabulated once in LDS (shared block layouts)
constexpr int MAX_LENGTHS = 4096; // padding lengths cached in LDS

struct alignas(16) PlanShared {
  int unit_cost[MAX_UNITS];       // shared block layout: kept tiles per layout row (or column)
  int lengths[MAX_LENGTHS];
};

// Cost of one item. `tab` says whether sh.unit_cost holds the shared layout's per-row (FWD_Q) or
// per-column (BWD_KV) counts, and whether sh.lengths holds the padding lengths.
__device__ int item_cost(const PlanParams& p, uint32_t item, const PlanShared& sh, bool tab_units, bool tab_len) {
  const int t = (int)(item % (uint32_t)p.n_tiles);
  const uint32_t bh = item / (uint32_t)p.n_tiles;
  const int h = (int)(bh % (uint32_t)p.heads);
  const int b = (int)(bh / (uint32_t)p.heads);
  const int tile = p.tile;
  const int len = (p.mask == MASK_PADDING) ? (tab_len ? sh.lengths[b] : p.lengths[b]) : 0;
  if (p.mode == PLAN_BWD_KV) {
    // key tile t of kv head h
    if (p.mask == MASK_PADDING) {
      const int L = clamp_len(len, p.seq_k);
      const int Lq = clamp_len(len, p.seq_q);
      return (t * tile < L) ? p.group * ((Lq + 63) / 64) : 0;
    }
    if (p.mask == MASK_BLOCK) {
      if (tab_units) return p.group * sh.unit_cost[t];
      int total = 0;
      for (int g = 0; g < p.group; ++g) {
        const int hq = h * p.group + g;
        const uint8_t* lay = p.layout + b * p.layout_stride_b + hq * p.layout_stride_h;
        total += layout_col_union_count(lay, p.nb_k, (t * tile) / 64, tile / 64, p.nb_q);
      }
      return total;
    }
    if (p.mask == MASK_CAUSAL) return p.group * ((p.seq_q - t * tile + 63) / 64);
    return p.group * ((p.seq_q + 63) / 64);
  }
  // query tile t of query head h
  if (p.mask == MASK_PADDING) {
    const int L = clamp_len(len, p.seq_k);
    const int Lq = clamp_len(len, p.seq_q);
    return (t * tile < Lq) ? (L + 63) / 64 : 0;
  }
  if (p.mask == MASK_BLOCK) {
    if (tab_units) return sh.unit_cost[t];
    const uint8_t* lay = p.layout + b * p.layout_stride_b + h * p.layout_stride_h;
    return layout_row_union_count(lay, p.nb_k, (t * tile) / 64, tile > 64 ? tile / 64 : 1, p.nb_q);
  }
  if (p.mask == MASK_CAUSAL) return min((p.seq_k + 63) / 64, (min(t * tile + tile, p.seq_q) - 1) / 64 + 1);
  return (p.seq_k + 63) / 64;
}

// Block-wide exclusive scan of one value per thread (THREADS threads, wave64).
__device__ int block_exclusive_scan(int v, int* wave_sums) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int ws = lane < THREADS / 64 ? wave_sums[lane] : 0;
    int wincl = ws;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(wincl, off, 64);
      if (lane >= off) wincl += o;
    }
    if (lane < THREADS / 64) wave_sums[lane] = wincl - ws;
  }
  __syncthreads();
  return wave_sums[wave] + incl - v;
}

// q = a / b and rem = a % b for 0 <= a < 2^24 and b >= 1, from inv_b = 1/b in float: the product
// a * inv_b is within one of the quotient, which the remainder's range then corrects.
__device__ __forceinline__ int divmod_small(int a, int b, float inv_b, int& rem) {
  int q = (int)((float)a * inv_b);
  int r = a - q * b;
  if (r < 0) {
    --q;
    r += b;
  } else if (r >= b) {
    ++q;
    r -= b;
  }
  rem = r;
  return q;
}

// Closed-form list for a block layout shared by every (batch, head): all units have the same
// per-tile costs, so the tiles are ranked once (longest first, ties by index) and the list is
// rank-major, unit-minor, with unit u on XCD u % n_xcd (list positions slot * n_xcd + xcd). The
// layout is staged in LDS with one coalesced pass; no histogram or scan is needed.
constexpr int MAX_RANKED = 256;                // tiles ranked in closed form (the ranking is quadratic)
constexpr int MAX_STAGED_LAYOUT = 2 * MAX_CACHED;   // layout bytes staged in LDS (the `cached` array)

__device__ __forceinline__ bool closed_form_plan(const PlanParams& p) {
  return p.mask == MASK_BLOCK && p.layout_stride_b == 0 && p.layout_stride_h == 0 && p.tile >= 64 &&
         p.n_tiles <= MAX_RANKED && (int64_t)p.nb_q * p.nb_k <= MAX_STAGED_LAYOUT;
}

// Pairs the nb_q (at most 64) rows of a shared layout into query tiles of two (plan_pairs_rows): in
// rounds, every open row names the open row it shares the most kept tiles with (ties to the lower
// index), and rows that name each other pair. Each round pairs at least one pair (the pair of
// largest overlap with the lowest indices names itself both ways). After MAX_PAIR_ROUNDS rounds,
// or once no pair forms, the open rows pair in index order, an odd last one with "no row" (nb_q).
// Tile t is the pair whose lower row is the t-th lowest; its cost is the number of kept tiles in
// the union of its two rows. Writes p.row_pairs and cost[0, n_tiles).
//
// Lane r of every wave stands for row r. Waves 0-3 (one per SIMD) hold the keys
// (overlap << 16 | 0xffff - t) of their row against sixteen candidates each and, every round, post
// the best open one; after one barrier every wave takes the best of the four posts of each row and
// finds the mutual choices with one lane exchange, so all waves hold the same open rows without a
// second barrier (the posts of consecutive rounds go to alternate buffers).
constexpr int MAX_PAIR_ROUNDS = 6;
constexpr int MAX_PAIR_ROWS = 64;                        // layout rows the pairing handles (plan_pairs_rows)
constexpr int PAIR_WAVES = 4;                            // waves that scan candidates
constexpr int PAIR_CANDS = MAX_PAIR_ROWS / PAIR_WAVES;   // candidates per scanning wave
static_assert(MAX_PAIR_ROWS == 4 * (THREADS / 64), "every wave computes the keys of four candidates");
static_assert(MAX_RANKED + MAX_PAIR_ROWS * MAX_PAIR_ROWS <= NBUCKET, "the keys follow the ranked order in the buckets");

struct PairLds {
  uint64_t mask[MAX_PAIR_ROWS];                  // kept key tiles of each row, one bit each
  int partial[2][PAIR_WAVES][MAX_PAIR_ROWS];     // best key of each row among each wave's candidates
};

__device__ void pair_rows(const PlanParams& p, const uint8_t* lay, bool masks_ready, PairLds& s, int* keys,
                          int* cost) {
  constexpr int NW = THREADS / 64;
  const int nq = p.nb_q;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // row masks (unless the layout copy wrote them): wave w builds rows w + 16 i, one lane per key
  // tile (nb_k <= 64); loads first
  if (!masks_ready) {
    uint8_t kept[MAX_PAIR_ROWS / NW];
#pragma unroll
    for (int i = 0; i < MAX_PAIR_ROWS / NW; ++i) {
      const int r = wave + NW * i;
      kept[i] = (r < nq && lane < p.nb_k) ? lay[r * p.nb_k + lane] : 0;
    }
#pragma unroll
    for (int i = 0; i < MAX_PAIR_ROWS / NW; ++i) {
      const int r = wave + NW * i;
      const uint64_t m = __ballot(kept[i] != 0);
      if (lane == 0 && r < nq) s.mask[r] = m;
    }
    __syncthreads();
  }
  // keys: wave w computes candidates 4w .. 4w + 3 for every row into keys[t][r]; the scanning
  // waves then load their sixteen
  const int r = lane;
  const uint64_t own = r < nq ? s.mask[r] : 0ull;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * wave + j;
    keys[t * MAX_PAIR_ROWS + r] =
        (t < nq && r < nq && t != r) ? (__popcll(own & s.mask[t]) << 16) | (0xffff - t) : -1;
  }
  __syncthreads();
  const bool scan = wave < PAIR_WAVES;
  int key[PAIR_CANDS];
#pragma unroll
  for (int j = 0; j < PAIR_CANDS; ++j) key[j] = scan ? keys[(PAIR_CANDS * wave + j) * MAX_PAIR_ROWS + r] : -1;
  uint64_t open = nq >= 64 ? ~0ull : (1ull << nq) - 1;   // rows not yet paired (the same in every wave)
  int partner = -1;                                       // the row paired with row r
  for (int round = 0; round < MAX_PAIR_ROUNDS; ++round) {
    if (scan) {
      int post = -1;
#pragma unroll
      for (int j = 0; j < PAIR_CANDS; ++j)
        if ((open >> (PAIR_CANDS * wave + j)) & 1) post = max(post, key[j]);
      s.partial[round & 1][wave][r] = post;
    }
    __syncthreads();
    int k = -1;
#pragma unroll
    for (int w = 0; w < PAIR_WAVES; ++w) k = max(k, s.partial[round & 1][w][r]);
    const int b = (((open >> r) & 1) && k >= 0) ? 0xffff - (k & 0xffff) : -1;
    const int bb = __shfl(b, b >= 0 ? b : r, 64);   // the choice of row b
    const bool mutual = b >= 0 && bb == r;
    if (mutual) partner = b;
    open = __ballot(r < nq && partner < 0);
    if (__ballot(mutual) == 0) break;
  }
  if (wave == 0) {
    // the rows still open pair in index order, an odd last one with "no row"
    const uint64_t below = r == 0 ? 0ull : open & (~0ull >> (64 - r));   // open rows under r
    if ((open >> r) & 1) {
      if (__popcll(below) & 1) {
        partner = 63 - __builtin_clzll(below);
      } else {
        const uint64_t above = r == 63 ? 0ull : open & (~0ull << (r + 1));
        partner = above != 0 ? __builtin_ctzll(above) : nq;
      }
    }
    // tiles in order of their lower row
    const bool first = r < nq && partner > r;
    const uint64_t firsts = __ballot(first);
    if (first) {
      const int t = __popcll(r == 0 ? 0ull : firsts & (~0ull >> (64 - r)));
      p.row_pairs[2 * t] = (uint16_t)r;
      p.row_pairs[2 * t + 1] = (uint16_t)partner;
      cost[t] = __popcll(own | (partner < nq ? s.mask[partner] : 0ull));
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void plan_closed_form(const PlanParams& p, uint8_t* lay, int* cost, int* order,
                                                 PairLds& pair_lds) {
  const int nbytes = p.nb_q * p.nb_k;
  const bool aligned = (reinterpret_cast<uintptr_t>(p.layout) & 15) == 0;
  // with row pairing on whole 16-byte row chunks, the copy also writes the rows' kept-tile masks
  // (16 bits per chunk, upper chunks past nb_k zero)
  const bool masks_in_copy = p.row_pairs != nullptr && aligned && (p.nb_k & 15) == 0;
  if (aligned) {
    // 16 bytes per thread (the LDS copy is 16-byte aligned); the tail byte by byte
    const int n16 = nbytes / 16;
    const int chunks = p.nb_k / 16;   // per row, when masks_in_copy
    const float i_chunks = 1.0f / (float)max(chunks, 1);
    uint16_t* mask16 = reinterpret_cast<uint16_t*>(pair_lds.mask);
    for (int i = threadIdx.x; i < n16; i += THREADS) {
      const uint4 v = reinterpret_cast<const uint4*>(p.layout)[i];
      reinterpret_cast<uint4*>(lay)[i] = v;
      if (masks_in_copy) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t bits = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) bits |= (((w[k >> 2] >> ((k & 3) * 8)) & 0xffu) != 0u ? 1u : 0u) << k;
        int chunk;
        const int row = divmod_small(i, chunks, i_chunks, chunk);
        mask16[row * 4 + chunk] = (uint16_t)bits;
        if (chunk == chunks - 1)
          for (int c2 = chunks; c2 < 4; ++c2) mask16[row * 4 + c2] = 0;
      }
    }
    for (int i = n16 * 16 + threadIdx.x; i < nbytes; i += THREADS) lay[i] = p.layout[i];
  } else {
    for (int i = threadIdx.x; i < nbytes; i += THREADS) lay[i] = p.layout[i];
  }
  for (int t = threadIdx.x; t < p.n_tiles; t += THREADS) cost[t] = 0;
  __syncthreads();
  if (p.row_pairs != nullptr) {
    pair_rows(p, lay, masks_in_copy, pair_lds, order + MAX_RANKED, cost);
  } else {
    // kept tiles in the union of each tile's layout rows (columns): one (tile, column) pair per thread
    const int per_unit = p.tile / 64;   // layout rows (query tiles) or columns (key tiles) per tile
    const int n_other = p.mode == PLAN_BWD_KV ? p.nb_q : p.nb_k;
    const int pairs = p.n_tiles * n_other;
    for (int e = threadIdx.x; e < pairs; e += THREADS) {
      const int t = e / n_other, x = e - t * n_other;
      bool keep = false;
      for (int r = 0; r < per_unit; ++r) {
        const int y = t * per_unit + r;
        if (p.mode == PLAN_BWD_KV) keep = keep || (y < p.nb_k && lay[x * p.nb_k + y] != 0);
        else keep = keep || (y < p.nb_q && lay[y * p.nb_k + x] != 0);
      }
      if (keep) atomicAdd(&cost[t], 1);
    }
    __syncthreads();
  }
  // rank of each tile, longest first and ties by index: one wave per tile, 64 comparisons a ballot
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = wave; t < p.n_tiles; t += THREADS / 64) {
    const int c = cost[t];
    int r = 0;
    for (int u0 = 0; u0 < p.n_tiles; u0 += 64) {
      const int u = u0 + lane;
      const bool before = u < p.n_tiles && (cost[u] > c || (cost[u] == c && u < t));
      r += __popcll(__ballot(before));
    }
    if (lane == 0) order[r] = t;
  }
  __syncthreads();
  const int G = p.mode == PLAN_BWD_KV ? 1 : p.group;   // heads per unit
  const int per_unit_items = G * p.n_tiles;
  const int n_units = p.n_items / per_unit_items;
  const int heads_kv = p.heads / G;
  const int n_xcd = (p.n_xcd > 1 && p.n_xcd <= kMaxXcd && n_units % p.n_xcd == 0) ? p.n_xcd : 1;
  const int per_rank = (n_units / n_xcd) * G;
  if (p.n_items < (1 << 24)) {
    // the four divisions by workgroup-uniform divisors through float reciprocals
    const float i_xcd = 1.0f / (float)n_xcd, i_rank = 1.0f / (float)per_rank, i_g = 1.0f / (float)G,
                i_hkv = 1.0f / (float)heads_kv;
    for (int pos = threadIdx.x; pos < p.n_items; pos += THREADS) {
      int x, rem, g, hk;
      const int slot = divmod_small(pos, n_xcd, i_xcd, x);
      const int r = divmod_small(slot, per_rank, i_rank, rem);
      const int u = x + n_xcd * divmod_small(rem, G, i_g, g);
      const int b = divmod_small(u, heads_kv, i_hkv, hk);
      p.items[pos] = (uint32_t)(((int64_t)b * p.heads + hk * G + g) * p.n_tiles + order[r]);
    }
  } else {
    for (int pos = threadIdx.x; pos < p.n_items; pos += THREADS) {
      const int x = pos % n_xcd, slot = pos / n_xcd;
      const int r = slot / per_rank, rem = slot - r * per_rank;
      const int u = x + n_xcd * (rem / G);
      const int b = u / heads_kv, h = (u - b * heads_kv) * G + rem % G;
      p.items[pos] = (uint32_t)(((int64_t)b * p.heads + h) * p.n_tiles + order[r]);
    }
  }
}

__device__ __forceinline__ void plan_items(const PlanParams& p) {
  __shared__ int bucket[NBUCKET];
  __shared__ int wave_sums[THREADS / 64];
  __shared__ __attribute__((aligned(16))) uint16_t cached[MAX_CACHED];
  __shared__ PlanShared sh;
  if (closed_form_plan(p)) {
    // the row pairing works in the padding-length cache
    static_assert(sizeof(PairLds) <= sizeof(sh.lengths) && offsetof(PlanShared, lengths) % 8 == 0, "pairing LDS");
    plan_closed_form(p, (uint8_t*)cached, sh.unit_cost, bucket, *reinterpret_cast<PairLds*>(sh.lengths));
    return;
  }
  const bool cache = p.n_items <= MAX_CACHED;
  // A block layout shared by every (batch, head): the cost of a tile is the number of kept
  // columns (rows) in the union of its layout rows (columns), the same for every (batch, head).
  // Tabulate it once, every thread testing independent (tile, column) pairs of the layout.
  const int per_unit = p.tile / 64;                   // layout rows (columns) per tile
  const int n_other = p.mode == PLAN_BWD_KV ? p.nb_q : p.nb_k;
  const bool tab_units = p.mask == MASK_BLOCK && p.layout_stride_b == 0 && p.layout_stride_h == 0 &&
                         per_unit >= 1 && p.n_tiles <= MAX_UNITS;
  const bool tab_len = p.mask == MASK_PADDING && p.n_items > 0 &&
                       (int64_t)p.n_items / ((int64_t)p.heads * p.n_tiles) <= MAX_LENGTHS;
  for (int i = threadIdx.x; i < NBUCKET; i += THREADS) bucket[i] = 0;
  if (tab_units)
    for (int u = threadIdx.x; u < p.n_tiles; u += THREADS) sh.unit_cost[u] = 0;
  if (tab_len) {
    const int batch = (int)((int64_t)p.n_items / ((int64_t)p.heads * p.n_tiles));
    for (int b = threadIdx.x; b < batch; b += THREADS) sh.lengths[b] = p.lengths[b];
  }
  __syncthreads();
  if (tab_units) {
    const int64_t total = (int64_t)p.n_tiles * n_other;
    for (int64_t e = threadIdx.x; e < total; e += THREADS) {
      const int unit = (int)(e / n_other), x = (int)(e % n_other);
      bool keep = false;
      for (int r = 0; r < per_unit; ++r) {
        const int y = unit * per_unit + r;
        if (p.mode == PLAN_BWD_KV) {
          if (y < p.nb_k && p.layout[(size_t)x * p.nb_k + y] != 0) keep = true;
        } else {
          if (y < p.nb_q && p.layout[(size_t)y * p.nb_k + x] != 0) keep = true;
        }
      }
      if (keep) atomicAdd(&sh.unit_cost[unit], 1);
    }
    __syncthreads();
  }
  // Items of one (batch, kv-head) unit share K and V (forward, dQ) or Q and dO (dK/dV). The
  // dispatcher deals workgroup w to XCD w % n_xcd; when the units divide evenly over the XCDs,
  // unit u goes to XCD u % n_xcd (list positions rank * n_xcd + xcd) so that its data stay in one
  // L2. Within an XCD items are ordered longest first. Bucket xcd * NCOST + (NCOST - 1 - cost).
  const int items_per_unit = p.mode == PLAN_BWD_KV ? p.n_tiles : p.group * p.n_tiles;
  const int n_units = p.n_items / items_per_unit;
  const int n_xcd = p.n_xcd;
  const bool spread = n_xcd > 1 && n_xcd <= kMaxXcd && (n_units % n_xcd) == 0;
  auto xcd_of = [&](int i) { return spread ? (i / items_per_unit) % n_xcd : 0; };
  for (int i = threadIdx.x; i < p.n_items; i += THREADS) {
    const int cost = min(item_cost(p, (uint32_t)i, sh, tab_units, tab_len), NCOST - 1);
    if (cache) cached[i] = (uint16_t)cost;
    atomicAdd(&bucket[xcd_of(i) * NCOST + NCOST - 1 - cost], 1);
  }
  __syncthreads();
  constexpr int PER = NBUCKET / THREADS;
  int local[PER];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    local[k] = bucket[threadIdx.x * PER + k];
    sum += local[k];
  }
  int off = block_exclusive_scan(sum, wave_sums);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    bucket[threadIdx.x * PER + k] = off;
    off += local[k];
  }
  __syncthreads();
  const int per_xcd = spread ? p.n_items / n_xcd : p.n_items;
  for (int i = threadIdx.x; i < p.n_items; i += THREADS) {
    const int cost = cache ? (int)cached[i] : min(item_cost(p, (uint32_t)i, sh, tab_units, tab_len), NCOST - 1);
    const int x = xcd_of(i);
    const int rank = atomicAdd(&bucket[x * NCOST + NCOST - 1 - cost], 1) - x * per_xcd;
    p.items[spread ? rank * n_xcd + x : rank] = (uint32_t)i;
  }
}

__global__ __launch_bounds__(THREADS) void plan_kernel(PlanParams p) { plan_items(p); }

// Several independent item lists in one launch, one workgroup each: the backward's dK/dV and dQ
// lists, and with them the forward's when a forward also plans the backward that follows it. The
// workgroup reads its list's parameters in place from the kernel arguments.
template <int N>
struct PlanList {
  PlanParams p[N];
};
__global__ __launch_bounds__(THREADS) void plan_pair_kernel(PlanList<2> lists) { plan_items(lists.p[blockIdx.x]); }
__global__ __launch_bounds__(THREADS) void plan_triple_kernel(PlanList<3> lists) { plan_items(lists.p[blockIdx.x]); }

}  // namespace

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(THREADS), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_plan_pair(const PlanParams& a, const PlanParams& b, hipStream_t stream) {
  hipLaunchKernelGGL(plan_pair_kernel, dim3(2), dim3(THREADS), 0, stream, PlanList<2>{{a, b}});
  return hipGetLastError();
}

hipError_t launch_plan_triple(const PlanParams& a, const PlanParams& b, const PlanParams& c, hipStream_t stream) {
  hipLaunchKernelGGL(plan_triple_kernel, dim3(3), dim3(THREADS), 0, stream, PlanList<3>{{a, b, c}});
  return hipGetLastError();
}

}  // namespace attn
