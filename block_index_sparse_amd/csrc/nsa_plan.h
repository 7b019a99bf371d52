// Host-side plan arithmetic of the native sparse attention library: the
// tiling, work-item and workspace layout of the forward and the decode step
// (the backward's sizes are in nsa_bwd_plan.h).  Plain C++ with no HIP dependency, so it also builds with the
// host compiler alone (the sanitizer build of the tests exercises it on
// hostile dims).  Internal, not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "nsa.h"

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
  size_t off_tile_start, off_hdr, off_bucket, off_blocks, off_masks, off_units, off_off, off_total,
      off_worklist, off_err, bytes;
};

// Decode (one query token per sequence against a KV cache): derived sizes.
struct DecodePlan {
  int32_t B, Smax, Hq, Hkv, D, S, bs, G;
  int32_t gv, gpk;           // heads per group (<= 16), groups per kv head
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// a * b * c <= limit for non-negative factors, without overflowing.
inline bool product_le(int64_t a, int64_t b, int64_t c, int64_t limit) {
  if (a == 0 || b == 0 || c == 0) return true;
  if (a > limit / b) return false;
  return a * b <= limit / c;
}

// Derive tiling and workspace layout.  Returns NSA_SUCCESS or an error.
// small_units: 32-key units where a block holds 64 keys of D = 128 (the
// ring then holds 8 units instead of 4; the gradient mode of the ring, whose
// waves keep a unit longer, gains more from the deeper ring than it loses to
// the per-unit handshakes, the forward does not).
inline nsa_status make_plan(const nsa_dims* d, int32_t block_size, int32_t num_seqs, bool varlen, Plan* p,
                            bool qblock, int cus, bool small_units = false) {
  if (!d) return NSA_ERROR_INVALID_VALUE;
  if (d->batch <= 0 || d->seqlen <= 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 ||
      d->head_dim <= 0 || d->num_selected <= 0 || block_size <= 0)
    return NSA_ERROR_INVALID_VALUE;
  if (d->num_q_heads % d->num_kv_heads) return NSA_ERROR_INVALID_VALUE;
  if (varlen && (d->batch != 1 || num_seqs <= 0)) return NSA_ERROR_INVALID_VALUE;
  if (varlen && qblock) return NSA_ERROR_NOT_SUPPORTED;
  if (d->dtype != NSA_DTYPE_F32 && d->dtype != NSA_DTYPE_BF16) return NSA_ERROR_NOT_SUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return NSA_ERROR_NOT_SUPPORTED;
  if (block_size != 32 && block_size != 64 && block_size != 128) return NSA_ERROR_NOT_SUPPORTED;
  const int64_t rows = (int64_t)d->batch * d->seqlen;
  if (rows > INT32_MAX / 2 || !product_le(rows, d->num_q_heads, d->head_dim, INT64_C(1) << 40))
    return NSA_ERROR_NOT_SUPPORTED;

  Plan& P = *p;
  P = Plan{};
  P.B = d->batch;
  P.T = d->seqlen;
  P.Hq = d->num_q_heads;
  P.Hkv = d->num_kv_heads;
  P.D = d->head_dim;
  P.S = d->num_selected;
  P.bs = block_size;
  P.G = P.Hq / P.Hkv;
  P.varlen = varlen;
  P.qblock = qblock;
  P.nqb = (P.T + P.bs - 1) / P.bs;
  P.num_seqs = varlen ? num_seqs : P.B;
  P.bf16 = d->dtype == NSA_DTYPE_BF16;
  // head groups of at most 16 heads (one MFMA column tile)
  if (P.G <= 16) {
    P.gv = P.G;
    P.gpk = 1;
  } else if (P.G % 16 == 0 && P.G <= 1024) {
    P.gv = 16;
    P.gpk = P.G / 16;
  } else {
    return NSA_ERROR_NOT_SUPPORTED;
  }
  P.hv = P.Hkv * P.gpk;
  // tokens per 16-column tile: the largest power of two with tpt * gv <= 16
  P.tpt = 1;
  while (P.tpt * 2 * P.gv <= 16) P.tpt *= 2;
  P.ntpw = P.bf16 ? 1 : ((P.tpt * 2 * kConsumers <= kMaxTileTokensF32) ? 2 : 1);
  P.tpw = P.tpt * P.ntpw;
  P.kb = P.bs < 64 ? P.bs : 64;
  if (small_units && P.bs == 64 && P.D == 128 && P.bf16) P.kb = 32;
  P.nsb = P.bs / P.kb;
  const int64_t nb_max = (P.T + P.bs - 1) / P.bs;  // a sequence is at most T long
  if (nb_max > (int64_t)kMaxBitmapWords * 32) return NSA_ERROR_NOT_SUPPORTED;
  // Tokens per item: one tile per attention wave (bf16 up to 256 tokens,
  // fp32 up to 128).  An item wider than 128 tokens is used only where its
  // merged list and token masks fit the scheduler's 64 KB of LDS per wave;
  // otherwise the item falls back to 128 tokens.
  const int64_t nbw = (nb_max + 31) / 32;
  int64_t umax = 1;
  auto size_for = [&](int32_t tq) {
    P.tq = tq;
    P.mw = (tq + 31) / 32;
    umax = std::max<int64_t>(1, std::min<int64_t>((int64_t)tq * P.S, nb_max));
  };
  size_for(std::min(kConsumers * P.tpw, P.bf16 ? kMaxTileTokens : kMaxTileTokensF32) / P.tpw *
           P.tpw);
  if (P.tq > 128 &&
      (umax > kMaxUnion || (2 * nbw + (int64_t)P.mw * umax) * (int64_t)sizeof(uint32_t) > 64 * 1024))
    size_for(std::min(kConsumers * P.tpw, 128) / P.tpw * P.tpw);
  if (umax > kMaxUnion) return NSA_ERROR_NOT_SUPPORTED;
  const int64_t Ttot = rows;
  const int64_t n_tiles =
      varlen ? Ttot / P.tq + P.num_seqs : (int64_t)P.B * ((P.T + P.tq - 1) / P.tq);
  const int64_t n_items = n_tiles * P.hv;
  if (n_items > INT32_MAX / 2) return NSA_ERROR_NOT_SUPPORTED;
  P.n_tiles = (int32_t)n_tiles;
  P.n_items = (int32_t)n_items;
  P.nb_max = (int32_t)nb_max;
  P.umax = (int32_t)umax;
  P.umax_units = (int32_t)((umax * P.nsb + 15) / 16 * 16);
  P.n_chunks = (int32_t)((n_items + kChunk - 1) / kChunk);
  if (cus <= 0) cus = 256;
  const int64_t wg = std::min<int64_t>(n_items, cus);
  P.nwg = (int32_t)((wg + kXcds - 1) / kXcds * kXcds);

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  P.off_tile_start = take(sizeof(int32_t) * (P.num_seqs + 1));
  P.off_hdr = take(sizeof(ItemHeader) * n_items);
  P.off_bucket = take(sizeof(int32_t) * n_items);
  P.off_blocks = take(sizeof(int32_t) * n_items * P.umax);
  P.off_masks = take(sizeof(uint32_t) * P.mw * n_items * P.umax);
  P.off_units = take(sizeof(uint32_t) * n_items * P.umax_units);
  P.off_off = take(sizeof(int32_t) * (size_t)kNumBuckets * P.n_chunks);
  P.off_total = take(sizeof(int32_t) * kNumBuckets);
  P.off_worklist = take(sizeof(int32_t) * n_items);
  P.off_err = take(sizeof(int32_t) * 4);
  P.bytes = off;
  return NSA_SUCCESS;
}

}  // namespace nsa
