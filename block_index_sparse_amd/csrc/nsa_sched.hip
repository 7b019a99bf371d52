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

// tile_start[s] = first token tile of sequence s; tile_start[num_seqs] = total
// tiles.  Also clears the weight histogram and the error word.
__global__ void __launch_bounds__(256) init_kernel(const int32_t* __restrict__ cu_seqlens,
                                                   int32_t num_seqs, int32_t T, int32_t tq,
                                                   int32_t* __restrict__ tile_start,
                                                   int32_t* __restrict__ hist, int32_t hist_n,
                                                   int32_t* __restrict__ err) {
  for (int32_t i = threadIdx.x; i < hist_n; i += blockDim.x) hist[i] = 0;
  if (threadIdx.x == 0) *err = 0;
  __shared__ int32_t part[256];
  int32_t carry = 0;
  for (int32_t base = 0; base <= num_seqs; base += 256) {
    const int32_t s = base + (int32_t)threadIdx.x;
    int32_t tiles = 0;
    if (s < num_seqs) {
      const int32_t len = cu_seqlens ? (cu_seqlens[s + 1] - cu_seqlens[s]) : T;
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
  uint4* masks;         // [n_items * umax]
  uint32_t* units;      // [n_items * umax_units]
  int32_t* hist;        // [kNumBuckets][n_chunks]
  int32_t T, Hkv, S, bs, gpk, tq, num_seqs, n_tiles, n_items, umax, n_chunks;
  int32_t max_pairs;    // tq * min(S, blocks per sequence): the heaviest possible item
  int32_t kb, nsb, umax_units, tpw;
};

// Token bits [first, first + count) of a 128-bit set (count a power of two
// dividing 32, first a multiple of count).
__device__ __forceinline__ uint32_t field(const uint32_t* m, int first, int count) {
  const uint32_t sh = m[first >> 5] >> (first & 31);
  return count >= 32 ? sh : (sh & ((1u << count) - 1u));
}

// Block-wide exclusive scan of one value per thread (256 threads).
__device__ int32_t block_exclusive_scan(int32_t v, int32_t* part, int32_t* total) {
  part[threadIdx.x] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int32_t add = threadIdx.x >= (unsigned)o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  const int32_t incl = part[threadIdx.x];
  *total = part[255];
  __syncthreads();
  return incl - v;
}

// One workgroup (256 threads) per item.
__global__ void __launch_bounds__(256) plan_kernel(PlanArgs a) {
  __shared__ uint32_t bitmap[kMaxBitmapWords];
  __shared__ int32_t wbase[kMaxBitmapWords];
  __shared__ uint32_t tmask[kMaxUnion][kMaxMaskWords];
  __shared__ int32_t part[256];
  __shared__ int32_t red[256];

  const int32_t item = blockIdx.x;
  const int32_t vg = item / a.n_tiles;
  const int32_t tile = item - vg * a.n_tiles;
  const int32_t h = vg / a.gpk;
  const int32_t total_tiles = a.tile_start[a.num_seqs];
  const int32_t chunk = item / kChunk;

  if (tile >= total_tiles) {
    if (threadIdx.x == 0) {
      a.hdr[item] = ItemHeader{0, 0, 0, 0};
      a.bucket[item] = 0;
      atomicAdd(&a.hist[chunk], 1);  // bucket 0 row
    }
    return;
  }
  // sequence holding this tile: last s with tile_start[s] <= tile
  int32_t lo = 0, hi = a.num_seqs - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (a.tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int32_t s = lo;
  const int32_t bos = a.cu ? a.cu[s] : s * a.T;
  const int32_t len = a.cu ? (a.cu[s + 1] - a.cu[s]) : a.T;
  const int32_t pos0 = (tile - a.tile_start[s]) * a.tq;
  const int32_t ntok = min(a.tq, len - pos0);
  const int32_t tok0 = bos + pos0;
  const int32_t own_hi = (pos0 + ntok - 1) / a.bs;
  const int32_t nwords = own_hi / 32 + 1;   // host guarantees <= kMaxBitmapWords
  const int32_t nent = ntok * a.S;

  for (int32_t w = threadIdx.x; w < nwords; w += 256) bitmap[w] = 0;
  __syncthreads();
  for (int32_t e = threadIdx.x; e < nent; e += 256) {
    const int32_t tau = e / a.S;
    const int32_t i = e - tau * a.S;
    const int64_t row = (int64_t)(tok0 + tau) * a.Hkv + h;
    int32_t n = a.bc[row];
    n = n < 0 ? 0 : (n > a.S ? a.S : n);
    if (i < n) {
      const int32_t idx = a.bi[row * a.S + i];
      if (idx >= 0 && idx <= (pos0 + tau) / a.bs) atomicOr(&bitmap[idx >> 5], 1u << (idx & 31));
    }
  }
  __syncthreads();
  // compact ids: exclusive prefix of set bits over the words
  const int32_t per = (nwords + 255) / 256;
  int32_t mine = 0;
  for (int32_t k = 0; k < per; k++) {
    const int32_t w = threadIdx.x * per + k;
    if (w < nwords) mine += __popc(bitmap[w]);
  }
  int32_t U;
  int32_t run = block_exclusive_scan(mine, part, &U);
  for (int32_t k = 0; k < per; k++) {
    const int32_t w = threadIdx.x * per + k;
    if (w < nwords) {
      wbase[w] = run;
      run += __popc(bitmap[w]);
    }
  }
  for (int32_t c = threadIdx.x; c < U; c += 256)
    for (int m = 0; m < kMaxMaskWords; m++) tmask[c][m] = 0;
  __syncthreads();
  for (int32_t e = threadIdx.x; e < nent; e += 256) {
    const int32_t tau = e / a.S;
    const int32_t i = e - tau * a.S;
    const int64_t row = (int64_t)(tok0 + tau) * a.Hkv + h;
    int32_t n = a.bc[row];
    n = n < 0 ? 0 : (n > a.S ? a.S : n);
    if (i < n) {
      const int32_t idx = a.bi[row * a.S + i];
      if (idx >= 0 && idx <= (pos0 + tau) / a.bs) {
        const int32_t w = idx >> 5;
        const int32_t cid = wbase[w] + __popc(bitmap[w] & ((1u << (idx & 31)) - 1u));
        atomicOr(&tmask[cid][tau >> 5], 1u << (tau & 31));
      }
    }
  }
  __syncthreads();
  int32_t pairs = 0;
  const int64_t lbase = (int64_t)item * a.umax;
  for (int32_t w = threadIdx.x; w < nwords; w += 256) {
    uint32_t bits = bitmap[w];
    int32_t cid = wbase[w];
    while (bits) {
      const int32_t b = __ffs(bits) - 1;
      bits &= bits - 1u;
      a.blocks[lbase + cid] = w * 32 + b;
      uint4 mk;
      mk.x = tmask[cid][0];
      mk.y = tmask[cid][1];
      mk.z = tmask[cid][2];
      mk.w = tmask[cid][3];
      a.masks[lbase + cid] = mk;
      pairs += __popc(mk.x) + __popc(mk.y) + __popc(mk.z) + __popc(mk.w);
      // unit words: which attention waves read each key sub-block
      const int32_t blk = w * 32 + b;
      for (int32_t sb = 0; sb < a.nsb; sb++) {
        const int32_t kstart = blk * a.bs + sb * a.kb;
        uint32_t word = 0u;
        if (kstart <= pos0 + ntok - 1) {
          int32_t np = 0;
          for (int32_t wv = 0; wv < kConsumers; wv++) {
            const int32_t first = wv * a.tpw;
            if (first >= ntok) break;
            const int32_t last_pos = pos0 + min(first + a.tpw, ntok) - 1;
            if (field(tmask[cid], first, a.tpw) != 0u && kstart <= last_pos) np++;
          }
          word = unit_word(blk, np);
        }
        a.units[(int64_t)item * a.umax_units + cid * a.nsb + sb] = word;
      }
      cid++;
    }
  }
  // weight = (block, token) pairs, scaled so the heaviest possible item lands
  // in the top bucket
  red[threadIdx.x] = pairs;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < (unsigned)o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.hdr[item] = ItemHeader{tok0, pos0, ntok, U};
    const int64_t wgt = ((int64_t)red[0] * (kNumBuckets - 1) + a.max_pairs - 1) / a.max_pairs;
    const int32_t b = wgt < kNumBuckets ? (int32_t)wgt : kNumBuckets - 1;
    a.bucket[item] = b;
    atomicAdd(&a.hist[(int64_t)b * a.n_chunks + chunk], 1);
  }
}

// One workgroup per bucket: exclusive scan over chunks.
__global__ void __launch_bounds__(256) scan_kernel(const int32_t* __restrict__ hist,
                                                   int32_t* __restrict__ off,
                                                   int32_t* __restrict__ total, int32_t n_chunks) {
  __shared__ int32_t part[256];
  const int b = blockIdx.x;
  const int32_t* hrow = hist + (int64_t)b * n_chunks;
  int32_t* orow = off + (int64_t)b * n_chunks;
  int32_t carry = 0;
  for (int32_t base = 0; base < n_chunks; base += 256) {
    const int32_t c = base + (int32_t)threadIdx.x;
    const int32_t v = c < n_chunks ? hrow[c] : 0;
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

// One wave per chunk: place every item at
//   (items of heavier buckets) + (same bucket, earlier chunks) + (same bucket, earlier in chunk).
__global__ void __launch_bounds__(64) scatter_kernel(const int32_t* __restrict__ bucket,
                                                     const int32_t* __restrict__ off,
                                                     const int32_t* __restrict__ total,
                                                     int32_t* __restrict__ worklist, int32_t n_items,
                                                     int32_t n_chunks) {
  __shared__ int32_t base[kNumBuckets];
  __shared__ int32_t bk[kChunk];
  const int chunk = blockIdx.x;
  const int i = threadIdx.x;
  if (i == 0) {
    int32_t acc = 0;
    for (int b = kNumBuckets - 1; b >= 0; b--) {
      base[b] = acc;
      acc += total[b];
    }
  }
  const int32_t item = chunk * kChunk + i;
  const int32_t b = item < n_items ? bucket[item] : -1;
  bk[i] = b;
  __syncthreads();
  if (item < n_items) {
    int32_t rank = 0;
    for (int j = 0; j < i; j++) rank += (bk[j] == b) ? 1 : 0;
    worklist[base[b] + off[(int64_t)b * n_chunks + chunk] + rank] = item;
  }
}

}  // namespace

hipError_t launch_schedule(const Plan& p, const int32_t* block_indices, const int32_t* block_counts,
                           const int32_t* cu_seqlens, char* ws, hipStream_t stream) {
  int32_t* tile_start = reinterpret_cast<int32_t*>(ws + p.off_tile_start);
  int32_t* hist = reinterpret_cast<int32_t*>(ws + p.off_hist);
  init_kernel<<<1, 256, 0, stream>>>(p.varlen ? cu_seqlens : nullptr, p.num_seqs, p.T, p.tq,
                                     tile_start, hist, kNumBuckets * p.n_chunks,
                                     reinterpret_cast<int32_t*>(ws + p.off_err));
  PlanArgs a;
  a.bi = block_indices;
  a.bc = block_counts;
  a.cu = p.varlen ? cu_seqlens : nullptr;
  a.tile_start = tile_start;
  a.hdr = reinterpret_cast<ItemHeader*>(ws + p.off_hdr);
  a.bucket = reinterpret_cast<int32_t*>(ws + p.off_bucket);
  a.blocks = reinterpret_cast<int32_t*>(ws + p.off_blocks);
  a.masks = reinterpret_cast<uint4*>(ws + p.off_masks);
  a.hist = hist;
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
  a.units = reinterpret_cast<uint32_t*>(ws + p.off_units);
  a.kb = p.kb;
  a.nsb = p.nsb;
  a.umax_units = p.umax_units;
  a.tpw = p.tpw;
  plan_kernel<<<p.n_items, 256, 0, stream>>>(a);
  int32_t* off = reinterpret_cast<int32_t*>(ws + p.off_off);
  int32_t* total = reinterpret_cast<int32_t*>(ws + p.off_total);
  scan_kernel<<<kNumBuckets, 256, 0, stream>>>(hist, off, total, p.n_chunks);
  scatter_kernel<<<p.n_chunks, 64, 0, stream>>>(a.bucket, off, total,
                                                reinterpret_cast<int32_t*>(ws + p.off_worklist),
                                                p.n_items, p.n_chunks);
  return hipGetLastError();
}

}  // namespace nsa
