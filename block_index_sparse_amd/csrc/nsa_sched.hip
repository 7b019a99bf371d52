// Work scheduler of the native sparse attention forward (gfx950).
//
// The indices are given per query token (`block_indices [B, T, Hkv, S]`,
// `block_counts [B, T, Hkv]`, type annotations of `run` on the ejKernel
// native_sparse_attention API page).  A work item is a tile of up to `tpi`
// consecutive tokens of one sequence and one kv head.  For every item the
// scheduler
//   1. reads the first clamp(count, 0, S) entries of each token's row, keeps
//      the entries 0 <= idx <= own block, and merges the rows into one
//      ascending, duplicate-free block list where each entry carries the set
//      of the item's tokens that listed the block;
//   2. weighs the item by the (block, column tile) pairs the forward kernel
//      will compute;
//   3. orders all items longest-first (a stable counting sort on the weight),
//      so that the heaviest tiles start first and the short ones fill the
//      tail of the grid.
#include "nsa_internal.h"

namespace nsa {

namespace {

constexpr int kInfIdx = 0x7fffffff;

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o, 64);
  return v;
}

// tile_start[s] = first token tile of sequence s; tile_start[num_seqs] = total tiles.
__global__ void __launch_bounds__(256) tile_start_kernel(const int32_t* __restrict__ cu_seqlens,
                                                         int32_t num_seqs, int32_t T, int32_t tpi,
                                                         int32_t* __restrict__ tile_start) {
  __shared__ int32_t part[256];
  int32_t carry = 0;
  for (int32_t base = 0; base <= num_seqs; base += 256) {
    const int32_t s = base + (int32_t)threadIdx.x;
    int32_t tiles = 0;
    if (s < num_seqs) {
      int32_t len = cu_seqlens ? (cu_seqlens[s + 1] - cu_seqlens[s]) : T;
      tiles = len > 0 ? (len + tpi - 1) / tpi : 0;
    }
    part[threadIdx.x] = tiles;
    __syncthreads();
    // inclusive Hillis-Steele scan
    for (int o = 1; o < 256; o <<= 1) {
      int32_t add = threadIdx.x >= (unsigned)o ? part[threadIdx.x - o] : 0;
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
  BlockEntry* lists;
  int32_t* hist;  // [kNumBuckets][n_chunks]
  int32_t T, Hkv, S, bs, G, nt, tpt, tpi, num_seqs, n_tiles, n_items, umax, n_chunks, epl;
};

// One wave per item; a workgroup of 4 waves covers one chunk of kChunk items.
__global__ void __launch_bounds__(256) plan_kernel(PlanArgs a) {
  __shared__ int32_t hist[kNumBuckets];
  for (int i = threadIdx.x; i < kNumBuckets; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x;
  const int32_t total_tiles = a.tile_start[a.num_seqs];

  for (int it = wave; it < kChunk; it += 4) {
    const int32_t item = chunk * kChunk + it;
    if (item >= a.n_items) break;
    const int32_t h = item / a.n_tiles;
    const int32_t tile = item - h * a.n_tiles;
    ItemHeader hd = {0, 0, 0, 0};
    int32_t weight = 0;
    if (tile < total_tiles) {
      // sequence holding this tile: last s with tile_start[s] <= tile
      int32_t lo = 0, hi = a.num_seqs - 1;
      while (lo < hi) {
        int32_t mid = (lo + hi + 1) >> 1;
        if (a.tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
      }
      const int32_t s = lo;
      const int32_t bos = a.cu ? a.cu[s] : s * a.T;
      const int32_t len = a.cu ? (a.cu[s + 1] - a.cu[s]) : a.T;
      const int32_t pos0 = (tile - a.tile_start[s]) * a.tpi;
      const int32_t ntok = min(a.tpi, len - pos0);
      hd.tok0 = bos + pos0;
      hd.pos0 = pos0;
      hd.ntok = ntok;

      int vals[kMaxEntriesPerLane];
      int taus[kMaxEntriesPerLane];
#pragma unroll
      for (int r = 0; r < kMaxEntriesPerLane; r++) {
        vals[r] = kInfIdx;
        taus[r] = 0;
        if (r < a.epl) {
          const int e = r * 64 + lane;
          const int tau = e / a.S;
          const int i = e - tau * a.S;
          taus[r] = tau;
          if (tau < ntok) {
            const int64_t row = (int64_t)(hd.tok0 + tau) * a.Hkv + h;
            int n = a.bc[row];
            n = n < 0 ? 0 : (n > a.S ? a.S : n);
            if (i < n) {
              const int idx = a.bi[row * a.S + i];
              const int own = (pos0 + tau) / a.bs;
              if (idx >= 0 && idx <= own) vals[r] = idx;
            }
          }
        }
      }
      // column tiles' token sets
      int32_t u = 0;
      while (true) {
        int lm = kInfIdx;
#pragma unroll
        for (int r = 0; r < kMaxEntriesPerLane; r++) lm = min(lm, vals[r]);
        const int m = wave_min(lm);
        if (m == kInfIdx) break;
        uint32_t bits = 0;
#pragma unroll
        for (int r = 0; r < kMaxEntriesPerLane; r++) {
          if (vals[r] == m) {
            bits |= 1u << taus[r];
            vals[r] = kInfIdx;
          }
        }
        const uint32_t tm = wave_or(bits);
        if (lane == 0) {
          BlockEntry be;
          be.block = m;
          be.tokmask = tm;
          a.lists[(int64_t)item * a.umax + u] = be;
        }
        // (block, column tile) pairs this entry costs
        if (a.G <= 16) {
          for (int n = 0; n < a.nt; n++) {
            const uint32_t tmask = ((1u << a.tpt) - 1u) << (n * a.tpt);
            weight += (tm & tmask) ? 1 : 0;
          }
        } else {
          weight += a.nt;
        }
        u++;
      }
      hd.nunion = u;
    }
    const int32_t b = weight < kNumBuckets ? weight : kNumBuckets - 1;
    if (lane == 0) {
      a.hdr[item] = hd;
      a.bucket[item] = b;
      atomicAdd(&hist[b], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kNumBuckets; i += blockDim.x)
    a.hist[(int64_t)i * a.n_chunks + chunk] = hist[i];
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
      int32_t add = threadIdx.x >= (unsigned)o ? part[threadIdx.x - o] : 0;
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
  tile_start_kernel<<<1, 256, 0, stream>>>(p.varlen ? cu_seqlens : nullptr, p.num_seqs, p.T, p.tpi,
                                           tile_start);
  PlanArgs a;
  a.bi = block_indices;
  a.bc = block_counts;
  a.cu = p.varlen ? cu_seqlens : nullptr;
  a.tile_start = tile_start;
  a.hdr = reinterpret_cast<ItemHeader*>(ws + p.off_hdr);
  a.bucket = reinterpret_cast<int32_t*>(ws + p.off_bucket);
  a.lists = reinterpret_cast<BlockEntry*>(ws + p.off_lists);
  a.hist = reinterpret_cast<int32_t*>(ws + p.off_hist);
  a.T = p.T;
  a.Hkv = p.Hkv;
  a.S = p.S;
  a.bs = p.bs;
  a.G = p.G;
  a.nt = p.nt;
  a.tpt = p.tpt;
  a.tpi = p.tpi;
  a.num_seqs = p.num_seqs;
  a.n_tiles = p.n_tiles;
  a.n_items = p.n_items;
  a.umax = p.umax;
  a.n_chunks = p.n_chunks;
  a.epl = (p.tpi * p.S + 63) / 64;
  plan_kernel<<<p.n_chunks, 256, 0, stream>>>(a);
  int32_t* off = reinterpret_cast<int32_t*>(ws + p.off_off);
  int32_t* total = reinterpret_cast<int32_t*>(ws + p.off_total);
  scan_kernel<<<kNumBuckets, 256, 0, stream>>>(a.hist, off, total, p.n_chunks);
  scatter_kernel<<<p.n_chunks, 64, 0, stream>>>(a.bucket, off, total,
                                                reinterpret_cast<int32_t*>(ws + p.off_worklist),
                                                p.n_items, p.n_chunks);
  return hipGetLastError();
}

}  // namespace nsa
