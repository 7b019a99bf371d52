// Internal declarations shared by the host API and the gfx950 kernels of the
// native sparse attention forward.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nsa {

// A work item is a tile of up to `tq` consecutive query tokens of one
// sequence and one head group (the G query heads of a kv head, or a group of
// 16 of them when G > 16).  item = head_group * n_tiles + tile, where tiles
// enumerate the sequences' token tiles back to back.
struct ItemHeader {
  int32_t tok0;   // packed row of the item's first token
  int32_t pos0;   // position of that token inside its sequence
  int32_t ntok;   // valid tokens in the item (0 = padding item, nothing to do)
  int32_t nunion; // entries of the item's merged block list
};

constexpr int kNumBuckets = 128;    // longest-first weight buckets
constexpr int kChunk = 64;          // items per scheduler chunk
constexpr int kMaxMaskWords = 8;    // token bit set of one list entry: up to 256 tokens
constexpr int kMaxTileTokens = 32 * kMaxMaskWords;
constexpr int kMaxTileTokensF32 = 128;   // tokens per item of the fp32 path
constexpr int kMaxBitmapWords = 2048;   // blocks per sequence the planner can merge: 65536
constexpr int kMaxUnion = 2048;         // entries of one item's merged list
constexpr int kConsumers = 12;      // attention waves per forward workgroup
constexpr int kProducers = 4;       // loader waves per forward workgroup
constexpr int kXcds = 8;            // XCDs of an MI355X

// Unit-table word: one per streamed unit (list entry x key sub-block).
//   bit 31     unit is live (block in range, first key not past the item's last token)
//   bits 24-27 attention waves that read the unit
//   bits 0-23  block id
__host__ __device__ constexpr uint32_t unit_word(int32_t block, int32_t npart) {
  return 0x80000000u | ((uint32_t)npart << 24) | (uint32_t)block;
}

// Everything the host derives from the call arguments.
struct Plan {
  // problem
  int32_t B, T, Hq, Hkv, D, S, bs, G;
  int32_t num_seqs;          // sequences (B for fixed length)
  bool varlen;
  bool qblock;               // indices per query block: [B, Hkv, nqb, S], counts [B, Hkv, nqb]
  int32_t nqb;               // query blocks per sequence (qblock layout)
  bool bf16;
  // head groups: G <= 16 -> one group of G heads per kv head; G = 32, 64 ->
  // G/16 groups of 16 heads sharing the kv head
  int32_t gv;                // heads per group
  int32_t gpk;               // groups per kv head
  int32_t hv;                // groups in total (Hkv * gpk)
  // tiling
  int32_t tpt;               // tokens per 16-column MFMA tile
  int32_t ntpw;              // column tiles per attention wave
  int32_t tpw;               // tokens per attention wave
  int32_t tq;                // tokens per item (at most kConsumers * tpw)
  int32_t mw;                // token-mask words per merged-list entry (ceil(tq / 32))
  int32_t kb;                // keys per streamed unit (min(bs, 64))
  int32_t nsb;               // streamed units per listed block (bs / kb)
  int32_t umax_units;        // unit-table stride per item (umax * nsb rounded up to 16)
  int32_t n_tiles;           // upper bound on token tiles over all sequences
  int32_t n_items;           // n_tiles * hv
  int32_t umax;              // max merged-list entries per item
  int32_t n_chunks;          // ceil(n_items / kChunk)
  int32_t nb_max;            // upper bound on blocks per sequence
  int32_t nwg;               // persistent forward workgroups
  // workspace layout (byte offsets)
  size_t off_tile_start, off_hdr, off_bucket, off_blocks, off_masks, off_units, off_hist, off_off,
      off_total, off_worklist, off_err, bytes;
};

// Decode (one query token per sequence against a KV cache): derived sizes.
struct DecodePlan {
  int32_t B, Smax, Hq, Hkv, D, S, bs, G;
  int32_t gv, gpk;           // heads per group (<= 16), groups per kv head
};

// Backward: sizes of a call (fixed-length sequences, bf16).
struct BwdPlan {
  int32_t B, T, Hq, Hkv, D, S, bs, G;
  int32_t gv, gpk;
};

// Launchers (defined in the .hip files).
hipError_t launch_schedule(const Plan& p, const int32_t* block_indices, const int32_t* block_counts,
                           const int32_t* cu_seqlens, char* ws, hipStream_t stream);
hipError_t launch_fwd(const Plan& p, const void* q, const void* k, const void* v, float scale,
                      void* out, float* lse, char* ws, hipStream_t stream);
hipError_t launch_decode(const DecodePlan& p, const void* q, const void* k, const void* v,
                         const int32_t* seq_lens, const int32_t* block_indices,
                         const int32_t* block_counts, float scale, void* out, float* lse,
                         hipStream_t stream);
size_t bwd_workspace_bytes(const BwdPlan& p);   // Delta, then the reader bitmaps
hipError_t launch_bwd(const BwdPlan& p, const void* q, const void* k, const void* v, const void* out,
                      const float* lse, const void* dout, const int32_t* block_indices,
                      const int32_t* block_counts, float scale, float* dq, float* dk, float* dv,
                      float* delta, hipStream_t stream);
int device_cu_count();

}  // namespace nsa
