// Internal declarations shared by the host API and the gfx950 kernels of the
// native sparse attention forward.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsa {

// Work item: up to `tpi` consecutive query tokens of one sequence and one kv
// head.  Items are numbered item = kv_head * n_tiles + tile, where tiles
// enumerate the sequences' token tiles back to back.
struct ItemHeader {
  int32_t tok0;   // packed row of the item's first token
  int32_t pos0;   // position of that token inside its sequence
  int32_t ntok;   // valid tokens in the item (0 = padding item, nothing to do)
  int32_t nunion; // entries of the item's block list
};

// One entry of an item's block list: a block id (relative to the sequence
// start) and the bit set of the item's tokens that selected it.
struct BlockEntry {
  int32_t block;
  uint32_t tokmask;
};

constexpr int kNumBuckets = 128;   // LPT weight buckets (weights clamp to 127)
constexpr int kChunk = 64;         // items per scheduler chunk
constexpr int kMaxEntriesPerLane = 16;
constexpr int kWaves = 4;          // waves per forward workgroup

// Everything the host derives from the call arguments.
struct Plan {
  // problem
  int32_t B, T, Hq, Hkv, D, S, bs, G;
  int32_t num_seqs;          // sequences (B for fixed length)
  bool varlen;
  bool bf16;
  // tiling
  int32_t nt;                // MFMA column tiles (16 columns each) per item
  int32_t tpt;               // tokens per column tile (G <= 16), else 1
  int32_t tpi;               // tokens per item
  int32_t ncols;             // columns used per item (tpi * G)
  int32_t n_tiles;           // upper bound on token tiles over all sequences
  int32_t n_items;           // n_tiles * Hkv
  int32_t umax;              // max block-list entries per item
  int32_t n_chunks;          // ceil(n_items / kChunk)
  int32_t nb_max;            // upper bound on blocks per sequence
  // workspace layout (byte offsets)
  size_t off_tile_start, off_hdr, off_bucket, off_lists, off_hist, off_off, off_total,
      off_worklist, bytes;
};

// Launchers (defined in the .hip files).
hipError_t launch_schedule(const Plan& p, const int32_t* block_indices, const int32_t* block_counts,
                           const int32_t* cu_seqlens, char* ws, hipStream_t stream);
hipError_t launch_fwd(const Plan& p, const void* q, const void* k, const void* v, float scale,
                      void* out, float* lse, char* ws, hipStream_t stream);

}  // namespace nsa
