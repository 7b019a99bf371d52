// Work scheduler of the native sparse attention forward (gfx950).
//
// The indices are given per query token (`block_indices [B, T, Hkv, S]`,
// `block_counts [B, T, Hkv]`, type annotations of `run` on the ejKernel
// native_sparse_attention API page).  A work item is a tile of up to `tq`
// consecutive tokens of one sequence and one head group.  For every item the
// planner
//   1. reads the first clamp(count, 0, S) entries of each token's row and
//      keeps the entries 0 <= idx <= the token's own block;
//   2. merges the rows into one ascending, duplicate-free block list through
//      a bitmap in LDS, each entry carrying the set of the item's tokens that
//      listed the block (so one gathered block serves every token that
//      selected it);
//   3. weighs the item by its (block, token) pairs.
// All items are then ordered longest-first (a stable counting sort on the
// weight), so the heaviest tiles start first and short ones fill the tail.
#include "nsa_internal.h"

namespace nsa {

namespace {

// Packed sequences: tile_start[s] = first token tile of sequence s;
// tile_start[num_seqs] = total tiles.  (Fixed-length calls need no table:
// every sequence has ceil(T / tq) tiles.)
__global__ void __launch_bounds__(256) init_kernel(const int32_t* __restrict__ cu_seqlens,
                                                   int32_t num_seqs, int32_t tq,
                                                   int32_t* __restrict__ tile_start) {
  __shared__ int32_t part[256];
  int32_t carry = 0;
  for (int32_t base = 0; base <= num_seqs; base += 256) {
    const int32_t s = base + (int32_t)threadIdx.x;
    int32_t tiles = 0;
    if (s < num_seqs) {
      const int32_t len = cu_seqlens[s + 1] - cu_seqlens[s];
      tiles = len > 0 ? (len + tq - 1) / tq : 0;
    }
    part[threadIdx.x] = tiles;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int32_t add = threadIdx.x >= (unsigned)o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (s <= num_seqs) tile_start[s] = carry + part[threadIdx.x] - tiles;
    carry += part[255];
    __syncthreads();
  }
}

struct PlanArgs {
  const int32_t* bi;
  const int32_t* bc;
  const int32_t* cu;
  const int32_t* tile_start;
  ItemHeader* hdr;
  int32_t* bucket;
  int32_t* blocks;      // [n_items * umax]
  uint32_t* masks;      // [n_items * umax][mw]
  uint32_t* units;      // [n_items * umax_units]
  int32_t T, Hkv, S, bs, gpk, tq, num_seqs, n_tiles, n_items, umax, n_chunks;
  int32_t max_pairs;    // tq * min(S, blocks per sequence): the most (block, token) pairs of an item
  int32_t unit_weight;  // weight of a streamed unit in pairs (item_bucket), 0: pairs alone
  int32_t max_weight;   // the heaviest possible item's weight
  int32_t kb, nsb, umax_units, tpw;
  int32_t mw;           // token-mask words per merged entry
  int32_t nbw;          // bitmap words per wave: ceil(blocks per sequence / 32)
  int32_t wave_words;   // LDS words per wave: 2 * nbw + mw * umax
  int32_t qblock;       // rows per query block: [B, Hkv, nqb, S] / [B, Hkv, nqb]
  int32_t nqb;
  int32_t vec4;         // rows are read 16 bytes at a time (S % 4 == 0, indices 16-byte aligned)
};

// An item's weight for the longest-first order.  The forward streams each
// of its U merged entries' units once (the loaders' share) and computes
// each (block, token) pair once (the attention waves' share); a streamed
// unit costs the loaders about as much as kUnitWeight pairs cost the
// attention waves (per-unit and per-pair cycle counts of the ring kernel),
// and the larger share bounds the item.  That weight balances the
// workgroups best where each draws few items; where each draws many, the
// pair count alone (equal for most items of a fixed-count workload, so the
// list keeps token order and neighbouring items share their L2) measured
// faster, and unit_weight is 0.  Scaled so the heaviest possible item lands
// in the top bucket.
constexpr int32_t kUnitWeight = 6;
constexpr int32_t kUnitWeightRounds = 32;   // the unit-aware weight up to this many items per workgroup
__device__ __forceinline__ int32_t item_bucket(const PlanArgs& a, int32_t U, int32_t pairs) {
  const int64_t w = std::max<int64_t>((int64_t)a.unit_weight * U * a.nsb, pairs);
  const int64_t b = (w * (kNumBuckets - 1) + a.max_weight - 1) / a.max_weight;
  return b < kNumBuckets ? (int32_t)b : kNumBuckets - 1;
}

// Sequence s and first position pos0 of token tile `tile` (false past the
// last tile): closed form for fixed-length sequences, the tile table of
// init_kernel for packed ones.
__device__ __forceinline__ bool locate_tile(const PlanArgs& a, int32_t tile, int32_t& s, int32_t& pos0) {
  if (!a.cu) {
    const int32_t tps = (a.T + a.tq - 1) / a.tq;
    if (tile >= a.num_seqs * tps) return false;
    s = tile / tps;
    pos0 = (tile - s * tps) * a.tq;
    return true;
  }
  if (tile >= a.tile_start[a.num_seqs]) return false;
  int32_t lo = 0, hi = a.num_seqs - 1;   // last s with tile_start[s] <= tile
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (a.tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  s = lo;
  pos0 = (tile - a.tile_start[s]) * a.tq;
  return true;
}

// Attention waves that read a sub-block of an entry: wave wc owns the
// item's tokens [wc * tpw, wc * tpw + tpw) and reads the sub-block iff one
// of its tokens listed the block and its last token is at offset >= d (the
// sub-block's first key relative to the item's first position; the caller
// emits only sub-blocks with d < ntok, so a partial last wave qualifies
// whenever its group index does).  Waves below wc_min = d / tpw end too
// early; each tpw-bit group of the token set is folded to its lowest bit and
// counted (tpw is a power of two <= 32).
__device__ __forceinline__ int32_t readers(const uint32_t* tm, int32_t mw, int32_t tpw, int32_t d) {
  const int32_t first_bit = (d > 0 ? d / tpw : 0) * tpw;   // first bit of wave wc_min
  const uint32_t lows = tpw >= 32 ? 1u : 0xFFFFFFFFu / ((1u << tpw) - 1u);   // bit 0 of every group
  int32_t np = 0;
  for (int32_t w = 0; w < mw; w++) {
    uint32_t x = tm[w];
    for (int32_t sh = 1; sh < tpw; sh <<= 1) x |= x >> sh;
    x &= lows;
    const int32_t lo = first_bit - 32 * w;                 // keep groups from bit lo on
    if (lo >= 32) continue;
    if (lo > 0) x &= 0xFFFFFFFFu << lo;
    np += __popc(x);
  }
  return np;
}

// LDS operations of one wave complete in issue order, so ordering the
// compiler's view is all a wave needs between its own LDS writes and reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

constexpr int kPlanBatch = 8;   // index entries per lane loaded before use

// Block listed by entry e of an item (token e / S, position e % S) if the
// entry is kept, else -1.  The count and the index are loaded independently
// (the index row is always inside the tensor), so the two loads overlap.
__device__ __forceinline__ int32_t entry_block(const PlanArgs& a, int32_t e, int32_t nent, int32_t tok0,
                                               int32_t pos0, int32_t h) {
  if (e >= nent) return -1;
  const int32_t tau = e / a.S;
  const int32_t i = e - tau * a.S;
  // row of (token, kv head), or of (sequence, kv head, query block): a token
  // uses the row of the query block that holds it (fixed length only, so the
  // sequence is (tok0 - pos0) / T)
  const int64_t row = a.qblock ? ((int64_t)((tok0 - pos0) / a.T) * a.Hkv + h) * a.nqb + (pos0 + tau) / a.bs
                               : (int64_t)(tok0 + tau) * a.Hkv + h;
  int32_t n = a.bc[row];
  const int32_t idx = a.bi[row * a.S + i];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  return (i < n && idx >= 0 && idx <= (pos0 + tau) / a.bs) ? idx : -1;
}

// kWG false: one wave per item (blockDim.x / 64 items per workgroup, each
// wave with its own slice of the dynamic LDS; the waves never synchronise
// with each other).  kWG true: one workgroup of four waves per item, for
// items with many index entries: the entry passes are spread over all 256
// threads and one wave forms and writes the merged list.
template <bool kWG>
__global__ void __launch_bounds__(256) plan_kernel(PlanArgs a) {
  extern __shared__ uint32_t plan_lds[];
  const int32_t lane = threadIdx.x & 63;
  const int32_t wv = threadIdx.x >> 6;
  const int32_t item = kWG ? (int32_t)blockIdx.x : blockIdx.x * (int32_t)(blockDim.x >> 6) + wv;
  if (item >= a.n_items) return;
  const int32_t tid = kWG ? (int32_t)threadIdx.x : lane;   // this thread among the item's threads
  const int32_t nthr = kWG ? 256 : 64;
  auto item_sync = [&]() {
    if constexpr (kWG) __syncthreads(); else wave_lds_sync();
  };
  uint32_t* bitmap = plan_lds + (kWG ? (size_t)0 : (size_t)wv * a.wave_words);
  int32_t* wbase = reinterpret_cast<int32_t*>(bitmap + a.nbw);
  uint32_t* tmask = bitmap + 2 * a.nbw;   // [umax][mw]

  const int32_t vg = item / a.n_tiles;
  const int32_t tile = item - vg * a.n_tiles;
  const int32_t h = vg / a.gpk;
  int32_t s = 0, pos0 = 0;
  if (!locate_tile(a, tile, s, pos0)) {
    if (tid == 0) {
      a.hdr[item] = ItemHeader{0, 0, 0, 0};
      a.bucket[item] = 0;
    }
    return;
  }
  const int32_t bos = a.cu ? a.cu[s] : s * a.T;
  const int32_t len = a.cu ? (a.cu[s + 1] - a.cu[s]) : a.T;
  const int32_t ntok = min(a.tq, len - pos0);
  const int32_t tok0 = bos + pos0;
  const int32_t own_hi = (pos0 + ntok - 1) / a.bs;
  const int32_t nwords = own_hi / 32 + 1;   // host guarantees <= nbw
  const int32_t nent = ntok * a.S;

  for (int32_t w = tid; w < nwords; w += nthr) bitmap[w] = 0;
  item_sync();
  // Entry e = tau * S + i of the item (token tau, list position i) is kept
  // iff i < clamp(count, 0, S) and 0 <= idx <= tau's own block; the loads of
  // kPlanBatch entries per lane are issued before any of them is used.
  // When the item's entries fit one batch per thread (every item of up to
  // 8 x nthr entries), the first batch stays in registers for the token-set
  // pass below instead of being loaded again.
  const bool one_batch = nent <= nthr * kPlanBatch;
  int32_t keep0[kPlanBatch];
#pragma unroll
  for (int u = 0; u < kPlanBatch; u++) keep0[u] = -1;
  for (int32_t e0 = tid; e0 < nent; e0 += nthr * kPlanBatch) {
    int32_t keep[kPlanBatch];
#pragma unroll
    for (int u = 0; u < kPlanBatch; u++) keep[u] = entry_block(a, e0 + nthr * u, nent, tok0, pos0, h);
#pragma unroll
    for (int u = 0; u < kPlanBatch; u++)
      if (keep[u] >= 0) atomicOr(&bitmap[keep[u] >> 5], 1u << (keep[u] & 31));
    if (e0 == tid) {
#pragma unroll
      for (int u = 0; u < kPlanBatch; u++) keep0[u] = keep[u];
    }
  }
  item_sync();
  // merged-list position of the first block of every bitmap word: each lane
  // counts a contiguous run of words, then a wave scan (every wave computes
  // it, the first one stores it)
  const int32_t per = (nwords + 63) / 64;
  int32_t mine = 0;
  for (int32_t k = 0; k < per; k++) {
    const int32_t w = lane * per + k;
    if (w < nwords) mine += __popc(bitmap[w]);
  }
  const int32_t incl = wave_inclusive_scan(mine);
  const int32_t U = __shfl(incl, 63, 64);
  int32_t run = incl - mine;
  if (wv == 0 || !kWG) {
    for (int32_t k = 0; k < per; k++) {
      const int32_t w = lane * per + k;
      if (w < nwords) {
        wbase[w] = run;
        run += __popc(bitmap[w]);
      }
    }
  }
  for (int32_t c = tid; c < U * a.mw; c += nthr) tmask[c] = 0;
  item_sync();
  // token set of every merged entry
  for (int32_t e0 = tid; e0 < nent; e0 += nthr * kPlanBatch) {
    int32_t keep[kPlanBatch];
#pragma unroll
    for (int u = 0; u < kPlanBatch; u++)
      keep[u] = one_batch ? keep0[u] : entry_block(a, e0 + nthr * u, nent, tok0, pos0, h);
#pragma unroll
    for (int u = 0; u < kPlanBatch; u++) {
      if (keep[u] >= 0) {
        const int32_t idx = keep[u];
        const int32_t tau = (e0 + nthr * u) / a.S;
        const int32_t w = idx >> 5;
        const int32_t cid = wbase[w] + __popc(bitmap[w] & ((1u << (idx & 31)) - 1u));
        atomicOr(&tmask[cid * a.mw + (tau >> 5)], 1u << (tau & 31));
      }
    }
  }
  item_sync();
  if (kWG && wv != 0) return;   // one wave writes the list
  // emit the list: lane-strided over the candidate blocks 0 .. 32 * nwords - 1
  int32_t pairs = 0;
  const int64_t lbase = (int64_t)item * a.umax;
  for (int32_t blk = lane; blk < nwords * 32; blk += 64) {
    const int32_t w = blk >> 5;
    const uint32_t bits = bitmap[w];
    if (((bits >> (blk & 31)) & 1u) == 0u) continue;
    const int32_t cid = wbase[w] + __popc(bits & ((1u << (blk & 31)) - 1u));
    const uint32_t* tm = tmask + cid * a.mw;
    a.blocks[lbase + cid] = blk;
    for (int32_t w2 = 0; w2 < a.mw; w2++) {
      a.masks[(lbase + cid) * a.mw + w2] = tm[w2];
      pairs += __popc(tm[w2]);
    }
    // unit words: which attention waves read each key sub-block
    for (int32_t sb = 0; sb < a.nsb; sb++) {
      const int32_t kstart = blk * a.bs + sb * a.kb;
      uint32_t word = 0u;
      if (kstart <= pos0 + ntok - 1) {
        word = unit_word(blk, readers(tm, a.mw, a.tpw, kstart - pos0));
      }
      a.units[(int64_t)item * a.umax_units + cid * a.nsb + sb] = word;
    }
  }
  pairs = wave_sum(pairs);
  if (lane == 0) {
    a.hdr[item] = ItemHeader{tok0, pos0, ntok, U};
    a.bucket[item] = item_bucket(a, U, pairs);
  }
}

// Lane-per-token planner for sequences of at most 32 * NW blocks (NW <= 16):
// one workgroup of ceil(tq / 64) waves per item, thread tau owning token tau
// of the item.  Each thread reads its token's row (the first clamp(count, 0,
// S) entries) into a register bitmap of the listed blocks it keeps (0 <= idx
// <= its own block); the item's merged list is the OR of those bitmaps, and
// the token set of every merged entry is one wave ballot per 64 tokens.  No
// entry touches shared memory with an atomic, so rows that list the same
// blocks (dense or causal selections) do not serialise.  It writes exactly
// what plan_kernel writes.
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o, 64);
  return v;
}

template <int NW>
__global__ void __launch_bounds__(256) plan_tokens_kernel(PlanArgs a) {
  __shared__ uint32_t s_ibm[NW];                        // the item's listed blocks
  __shared__ int32_t s_blk[32 * NW];                    // merged list
  __shared__ uint32_t s_tm[32 * NW * kMaxMaskWords];    // token set of every entry, [entry][mw]
  __shared__ int32_t s_pairs;
  const int32_t tid = threadIdx.x;
  const int32_t lane = tid & 63;
  const int32_t wv = tid >> 6;
  const int32_t nthr = blockDim.x;
  const int32_t item = blockIdx.x;
  if (item >= a.n_items) return;
  const int32_t vg = item / a.n_tiles;
  const int32_t tile = item - vg * a.n_tiles;
  const int32_t h = vg / a.gpk;
  int32_t s = 0, pos0 = 0;
  if (!locate_tile(a, tile, s, pos0)) {
    if (tid == 0) {
      a.hdr[item] = ItemHeader{0, 0, 0, 0};
      a.bucket[item] = 0;
    }
    return;
  }
  const int32_t bos = a.cu ? a.cu[s] : s * a.T;
  const int32_t len = a.cu ? (a.cu[s + 1] - a.cu[s]) : a.T;
  const int32_t ntok = min(a.tq, len - pos0);
  const int32_t tok0 = bos + pos0;

  if (tid < NW) s_ibm[tid] = 0u;
  if (tid == 0) s_pairs = 0;
  // this thread's token: its kept entries as a bitmap of block ids
  uint32_t bm[NW];
#pragma unroll
  for (int w = 0; w < NW; w++) bm[w] = 0u;
  if (tid < ntok) {
    const int32_t t = pos0 + tid;
    const int64_t row = a.qblock ? ((int64_t)((tok0 - pos0) / a.T) * a.Hkv + h) * a.nqb + t / a.bs
                                 : (int64_t)(tok0 + tid) * a.Hkv + h;
    int32_t n = a.bc[row];
    n = n < 0 ? 0 : (n > a.S ? a.S : n);
    const int32_t own = t / a.bs;
    const int32_t* r = a.bi + row * a.S;
    auto keep = [&](int32_t idx) {
      if (idx >= 0 && idx <= own) {
        const uint32_t bit = 1u << (idx & 31);
        const int32_t w = idx >> 5;
#pragma unroll
        for (int ww = 0; ww < NW; ww++) bm[ww] |= (ww == w) ? bit : 0u;
      }
    };
    // rows are read kRowBatch entries at a time, every load of a batch
    // issued before any is used; the first batch does not wait for the
    // count (every entry of the row is inside the tensor)
    constexpr int kRowBatch = 32;
    if (a.vec4) {
      for (int32_t i0 = 0; i0 < n || i0 == 0; i0 += kRowBatch) {
        int4 e[kRowBatch / 4];
#pragma unroll
        for (int j = 0; j < kRowBatch / 4; j++)
          if (i0 + 4 * j < (i0 == 0 ? a.S : n)) e[j] = *reinterpret_cast<const int4*>(r + i0 + 4 * j);   // inside the row
#pragma unroll
        for (int j = 0; j < kRowBatch / 4; j++) {
          const int32_t i = i0 + 4 * j;
          if (i < n) keep(e[j].x);
          if (i + 1 < n) keep(e[j].y);
          if (i + 2 < n) keep(e[j].z);
          if (i + 3 < n) keep(e[j].w);
        }
      }
    } else {
      for (int32_t i0 = 0; i0 < n || i0 == 0; i0 += kRowBatch) {
        int32_t e[kRowBatch];
#pragma unroll
        for (int j = 0; j < kRowBatch; j++)
          if (i0 + j < (i0 == 0 ? a.S : n)) e[j] = r[i0 + j];
#pragma unroll
        for (int j = 0; j < kRowBatch; j++)
          if (i0 + j < n) keep(e[j]);
      }
    }
  }
  __syncthreads();   // s_ibm cleared
#pragma unroll
  for (int w = 0; w < NW; w++) {
    const uint32_t x = wave_or(bm[w]);
    if (lane == 0 && x != 0u) atomicOr(&s_ibm[w], x);
  }
  __syncthreads();
  // merged-list position of each word's first block
  uint32_t ibm[NW];
  int32_t wbase[NW];
  int32_t U = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    ibm[w] = s_ibm[w];
    wbase[w] = U;
    U += __popc(ibm[w]);
  }
  // token sets: one ballot per (entry, 64 tokens); wave wv owns token words
  // 2 wv and 2 wv + 1
  const int32_t mw = a.mw;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    uint32_t bits = ibm[w];
    while (bits != 0u) {
      const int32_t b = __builtin_ctz(bits);
      bits &= bits - 1u;
      const int32_t cid = wbase[w] + __popc(ibm[w] & ((1u << b) - 1u));
      const uint64_t m = __ballot((bm[w] >> b) & 1u);
      if (lane == 0) {
        if (2 * wv < mw) s_tm[cid * mw + 2 * wv] = (uint32_t)m;
        if (2 * wv + 1 < mw) s_tm[cid * mw + 2 * wv + 1] = (uint32_t)(m >> 32);
        if (wv == 0) s_blk[cid] = w * 32 + b;
      }
    }
  }
  __syncthreads();
  // emit the list, the token sets and the unit words
  int32_t pairs = 0;
  const int64_t lbase = (int64_t)item * a.umax;
  for (int32_t cid = tid; cid < U; cid += nthr) {
    const int32_t blk = s_blk[cid];
    const uint32_t* tm = s_tm + cid * mw;
    a.blocks[lbase + cid] = blk;
    for (int32_t w2 = 0; w2 < mw; w2++) {
      a.masks[(lbase + cid) * mw + w2] = tm[w2];
      pairs += __popc(tm[w2]);
    }
    for (int32_t sb = 0; sb < a.nsb; sb++) {
      const int32_t kstart = blk * a.bs + sb * a.kb;
      uint32_t word = 0u;
      if (kstart <= pos0 + ntok - 1) word = unit_word(blk, readers(tm, mw, a.tpw, kstart - pos0));
      a.units[(int64_t)item * a.umax_units + cid * a.nsb + sb] = word;
    }
  }
  pairs = wave_sum(pairs);
  if (lane == 0 && pairs != 0) atomicAdd(&s_pairs, pairs);
  __syncthreads();
  if (tid == 0) {
    a.hdr[item] = ItemHeader{tok0, pos0, ntok, U};
    a.bucket[item] = item_bucket(a, U, s_pairs);
  }
}

// One workgroup per bucket b: the items of each chunk that fell into b
// (counted from the items' buckets), then the exclusive scan over chunks.
// Workgroup 0 also clears the device status word: the schedule is complete
// before any forward of it runs.
__global__ void __launch_bounds__(256) scan_kernel(const int32_t* __restrict__ bucket, int32_t n_items,
                                                   int32_t* __restrict__ off,
                                                   int32_t* __restrict__ total, int32_t n_chunks,
                                                   int32_t* __restrict__ err) {
  __shared__ int32_t part[256];
  const int b = blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *err = 0;
  int32_t* orow = off + (int64_t)b * n_chunks;
  int32_t carry = 0;
  for (int32_t base = 0; base < n_chunks; base += 256) {
    const int32_t c = base + (int32_t)threadIdx.x;
    int32_t v = 0;
    if (c < n_chunks) {
      const int32_t i0 = c * kChunk, i1 = min(n_items, i0 + kChunk);
      for (int32_t i = i0; i < i1; i++) v += bucket[i] == b ? 1 : 0;
    }
    part[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int32_t add = threadIdx.x >= (unsigned)o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    if (c < n_chunks) orow[c] = carry + part[threadIdx.x] - v;
    carry += part[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) total[b] = carry;
}

// Rank of this lane among the wave's valid lanes holding the same key (lanes
// below it), and how many hold it.  Every valid lane ORs its bit into its
// key's 64-bit word of `sets` (a wave-private LDS table, all zero on entry),
// then reads the word back: the lanes' LDS operations of one instruction all
// complete before the wave's next LDS instruction, so the word then holds
// exactly the lanes that share the key.  The key's lowest lane clears the
// word again afterwards.  Keys are 0 .. kNumBuckets - 1.
__device__ __forceinline__ void same_key_rank(int32_t key, bool valid, uint64_t* sets, int32_t& rank,
                                              int32_t& count) {
  const uint32_t lane = threadIdx.x & 63;
  if (valid) __hip_atomic_fetch_or(&sets[key], 1ull << lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const uint64_t m = valid ? __hip_atomic_load(&sets[key], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) : 0ull;
  rank = (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  count = __popcll(m);
  if (valid && rank == 0) __hip_atomic_store(&sets[key], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Exclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int32_t wave_exclusive_scan(int32_t v) {
  int32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(incl, o, 64);
    if ((threadIdx.x & 63) >= (unsigned)o) incl += y;
  }
  return incl - v;
}

// Start of every bucket in the longest-first list (heavier buckets first),
// from the buckets' totals: one wave, two buckets per lane.
__device__ __forceinline__ void bucket_bases(const int32_t* tot, int32_t* base) {
  static_assert(kNumBuckets == 128, "two buckets per lane");
  const int32_t lane = threadIdx.x & 63;
  const int32_t b0 = kNumBuckets - 1 - 2 * lane;   // the heavier of the lane's two
  const int32_t s0 = tot[b0], s1 = tot[b0 - 1];
  const int32_t excl = wave_exclusive_scan(s0 + s1);
  base[b0] = excl;
  base[b0 - 1] = excl + s0;
}

// One wave per chunk: place every item at
//   (items of heavier buckets) + (same bucket, earlier chunks) + (same bucket, earlier in chunk).
__global__ void __launch_bounds__(64) scatter_kernel(const int32_t* __restrict__ bucket,
                                                     const int32_t* __restrict__ off,
                                                     const int32_t* __restrict__ total,
                                                     int32_t* __restrict__ worklist, int32_t n_items,
                                                     int32_t n_chunks) {
  __shared__ int32_t base[kNumBuckets];
  __shared__ uint64_t sets[kNumBuckets];
  const int chunk = blockIdx.x;
  const int i = threadIdx.x;
  sets[i] = 0ull;
  sets[i + 64] = 0ull;
  bucket_bases(total, base);
  const int32_t item = chunk * kChunk + i;
  const bool valid = item < n_items;
  const int32_t b = valid ? bucket[item] : -1;
  int32_t rank, count;
  __syncthreads();
  same_key_rank(b, valid, sets, rank, count);
  if (valid) worklist[base[b] + off[(int64_t)b * n_chunks + chunk] + rank] = item;
}

// The scan and the scatter in one workgroup, for at most kOrderMaxChunks
// chunks: per-chunk bucket counts into LDS, a scan per bucket over the
// chunks, bucket bases longest-first, then every item placed at the same
// position scan_kernel + scatter_kernel would give it.  Also clears the
// device status word.
constexpr int kOrderMaxChunks = 64;

__global__ void __launch_bounds__(256) order_kernel(const int32_t* __restrict__ bucket, int32_t n_items,
                                                    int32_t n_chunks, int32_t* __restrict__ worklist,
                                                    int32_t* __restrict__ err) {
  // [chunk][bucket]: count, then start offset inside its bucket (a thread
  // per bucket walks the chunks: consecutive buckets, consecutive banks)
  __shared__ int32_t cnt[kOrderMaxChunks][kNumBuckets];
  __shared__ int32_t tot[kNumBuckets];
  __shared__ int32_t base[kNumBuckets];
  __shared__ uint64_t sets[4][kNumBuckets];   // per wave: lanes holding each key
  const int32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) *err = 0;
  for (int32_t i = tid; i < kNumBuckets * kOrderMaxChunks; i += 256) (&cnt[0][0])[i] = 0;
  for (int32_t i = tid; i < 4 * kNumBuckets; i += 256) (&sets[0][0])[i] = 0ull;
  __syncthreads();
  // chunk c by wave c % 4; every bucket load of the wave goes out at once
  constexpr int kPerWave = kOrderMaxChunks / 4;
  int32_t bkt[kPerWave];
#pragma unroll
  for (int j = 0; j < kPerWave; j++) {
    const int32_t item = (wv + 4 * j) * kChunk + lane;
    bkt[j] = item < n_items ? bucket[item] : -1;
  }
  // the first lane of each bucket present in a chunk writes its count
#pragma unroll
  for (int j = 0; j < kPerWave; j++) {
    const int32_t c = wv + 4 * j;
    if (c >= n_chunks) break;
    int32_t rank, count;
    same_key_rank(bkt[j], bkt[j] >= 0, sets[wv], rank, count);
    if (bkt[j] >= 0 && rank == 0) cnt[c][bkt[j]] = count;
  }
  __syncthreads();
  // per bucket, exclusive scan over the chunks (a thread per bucket, the
  // counts held in registers; chunks past the last hold zeros)
  if (tid < kNumBuckets) {
    int32_t v[kOrderMaxChunks];
#pragma unroll
    for (int32_t c = 0; c < kOrderMaxChunks; c++) v[c] = cnt[c][tid];
    int32_t run = 0;
#pragma unroll
    for (int32_t c = 0; c < kOrderMaxChunks; c++) {
      cnt[c][tid] = run;
      run += v[c];
    }
    tot[tid] = run;
  }
  __syncthreads();
  if (wv == 0) bucket_bases(tot, base);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPerWave; j++) {
    const int32_t c = wv + 4 * j;
    if (c >= n_chunks) break;
    int32_t rank, count;
    same_key_rank(bkt[j], bkt[j] >= 0, sets[wv], rank, count);
    if (bkt[j] >= 0) worklist[base[bkt[j]] + cnt[c][bkt[j]] + rank] = c * kChunk + lane;
  }
}

}  // namespace

hipError_t launch_schedule(const Plan& p, const int32_t* block_indices, const int32_t* block_counts,
                           const int32_t* cu_seqlens, char* ws, hipStream_t stream) {
  int32_t* tile_start = reinterpret_cast<int32_t*>(ws + p.off_tile_start);
  if (p.varlen) init_kernel<<<1, 256, 0, stream>>>(cu_seqlens, p.num_seqs, p.tq, tile_start);
  PlanArgs a;
  a.bi = block_indices;
  a.bc = block_counts;
  a.cu = p.varlen ? cu_seqlens : nullptr;
  a.tile_start = tile_start;
  a.hdr = reinterpret_cast<ItemHeader*>(ws + p.off_hdr);
  a.bucket = reinterpret_cast<int32_t*>(ws + p.off_bucket);
  a.blocks = reinterpret_cast<int32_t*>(ws + p.off_blocks);
  a.masks = reinterpret_cast<uint32_t*>(ws + p.off_masks);
  a.mw = p.mw;
  a.T = p.T;
  a.Hkv = p.Hkv;
  a.S = p.S;
  a.bs = p.bs;
  a.gpk = p.gpk;
  a.tq = p.tq;
  a.num_seqs = p.num_seqs;
  a.n_tiles = p.n_tiles;
  a.n_items = p.n_items;
  a.umax = p.umax;
  a.n_chunks = p.n_chunks;
  a.max_pairs = p.tq * (p.S < p.nb_max ? p.S : p.nb_max);
  a.unit_weight = p.n_items <= (int64_t)kUnitWeightRounds * p.nwg ? kUnitWeight : 0;
  const int64_t max_w = std::max<int64_t>((int64_t)a.unit_weight * p.umax * p.nsb, a.max_pairs);
  a.max_weight = max_w > INT32_MAX ? INT32_MAX : (int32_t)max_w;
  a.units = reinterpret_cast<uint32_t*>(ws + p.off_units);
  a.kb = p.kb;
  a.nsb = p.nsb;
  a.umax_units = p.umax_units;
  a.tpw = p.tpw;
  a.nbw = (p.nb_max + 31) / 32;
  a.wave_words = 2 * a.nbw + p.mw * p.umax;
  a.qblock = p.qblock ? 1 : 0;
  a.nqb = p.nqb;
  a.vec4 = (p.S % 4 == 0) && ((reinterpret_cast<uintptr_t>(block_indices) & 15u) == 0) ? 1 : 0;
  const size_t wave_bytes = sizeof(uint32_t) * (size_t)a.wave_words;
  const int nw = (p.nb_max + 31) / 32;   // bitmap words a token's row needs
  const bool many = (int64_t)p.tq * p.S > 64 * 2 * kPlanBatch;   // index entries per item
  if (many && nw <= 16) {
    // wide items (many tokens listing the same blocks: the entry passes of
    // plan_kernel would serialise on a few LDS words): one lane per token,
    // a workgroup of ceil(tq / 64) waves per item
    const dim3 blk(64 * ((p.tq + 63) / 64));
    if (nw <= 1) plan_tokens_kernel<1><<<p.n_items, blk, 0, stream>>>(a);
    else if (nw <= 2) plan_tokens_kernel<2><<<p.n_items, blk, 0, stream>>>(a);
    else if (nw <= 4) plan_tokens_kernel<4><<<p.n_items, blk, 0, stream>>>(a);
    else if (nw <= 8) plan_tokens_kernel<8><<<p.n_items, blk, 0, stream>>>(a);
    else plan_tokens_kernel<16><<<p.n_items, blk, 0, stream>>>(a);
  } else if (many) {
    // many index entries per item: a workgroup per item
    plan_kernel<true><<<p.n_items, 256, wave_bytes, stream>>>(a);
  } else {
    int waves = (int)((64 * 1024) / wave_bytes);   // items per workgroup
    waves = waves < 1 ? 1 : (waves > 4 ? 4 : waves);
    plan_kernel<false><<<(p.n_items + waves - 1) / waves, 64 * waves, wave_bytes * waves, stream>>>(a);
  }
  int32_t* off = reinterpret_cast<int32_t*>(ws + p.off_off);
  int32_t* total = reinterpret_cast<int32_t*>(ws + p.off_total);
  int32_t* err = reinterpret_cast<int32_t*>(ws + p.off_err);
  int32_t* worklist = reinterpret_cast<int32_t*>(ws + p.off_worklist);
  if (p.n_chunks <= kOrderMaxChunks) {
    order_kernel<<<1, 256, 0, stream>>>(a.bucket, p.n_items, p.n_chunks, worklist, err);
  } else {
    scan_kernel<<<kNumBuckets, 256, 0, stream>>>(a.bucket, p.n_items, off, total, p.n_chunks, err);
    scatter_kernel<<<p.n_chunks, 64, 0, stream>>>(a.bucket, off, total, worklist, p.n_items, p.n_chunks);
  }
  return hipGetLastError();
}

}  // namespace nsa
