// Host-side plan arithmetic of the backward pass of the native sparse
// attention library: the sizes of a call, its tiles, grids and workspace.
// Plain C++ with no HIP dependency, so it also builds with the host compiler
// alone (the sanitizer build of the tests exercises it on hostile dims).
// Internal, not part of the C ABI.
#pragma once

#include "nsa_plan.h"

namespace nsa {

// Backward: sizes of a call (fixed-length sequences, bf16).
struct BwdPlan {
  int32_t B, T, Hq, Hkv, D, S, bs, G;
  int32_t gv, gpk;
  // dQ runs as the gradient mode of the forward's ring kernel, over the
  // forward's own schedule of the same indices (its plan of the same dims);
  // the schedule sits in the workspace after the dK / dV partial sums
  Plan fp;
};

// Work-items of the backward's kernels.
constexpr int kBwdKvThreads = 256;   // dk/dv workgroup: four 16-key tile waves

// readers per dk/dv unit: a kv head's query heads (gv of them) fill gv of
// the 16 MFMA rows, so 16 / gv tokens share one unit; with more than 16
// heads per kv head (gpk > 1) a unit is one token's group of 16
inline int bwd_unit_readers(const BwdPlan& p) { return p.gpk == 1 ? 16 / p.gv : 1; }

constexpr int kBwdSegMax = 4096;   // tokens of one segment (the dk/dv kernel's LDS reader list)

// The token segment of a dk/dv workgroup: 512 tokens up to T = 4096, then
// 1024, 2048 past 8192 and 4096 past 16384 (fewer workgroups and partial sums
// where every segment still has many workgroups; short segments bound the
// longest workgroup, that of a block every token reads), times the readers
// per unit (a workgroup's work follows its units, not its tokens), at most
// kBwdSegMax and at most T.  One segment (ns = 1): the dk/dv kernel writes
// the final sums itself and no partial sums are kept.
inline int seg_tokens(int T, int readers_per_unit) {
  const int64_t base = T > 16384 ? 4096 : (T > 8192 ? 2048 : (T > 4096 ? 1024 : 512));
  return (int)std::min<int64_t>(std::min<int64_t>(base * readers_per_unit, kBwdSegMax), std::max(T, 1));
}
inline int bwd_seg_tokens(const BwdPlan& p) { return seg_tokens(p.T, bwd_unit_readers(p)); }
inline int bwd_segments(const BwdPlan& p) { return (p.T + bwd_seg_tokens(p) - 1) / bwd_seg_tokens(p); }

// r / gv for 0 <= r < 16 as (r * bwd_gv_magic(p)) >> 16 (the kernels split a
// unit's 16 rows into (reader, head) without an integer division)
inline int bwd_gv_magic(const BwdPlan& p) { return (1 << 16) / p.gv + 1; }

struct BwdGrids {
  int64_t dkdv, reduce, clear_words;
};

inline BwdGrids bwd_grids(const BwdPlan& p) {
  const int64_t ns = bwd_segments(p);
  const int64_t nb = (p.T + p.bs - 1) / p.bs, nw = (p.T + 31) / 32;
  BwdGrids g;
  g.dkdv = (int64_t)p.B * p.Hkv * ((p.T + 63) / 64) * ns;
  g.reduce = ((int64_t)p.B * p.T * p.Hkv * p.D / 4 + 255) / 256;
  g.clear_words = (int64_t)p.B * p.Hkv * nb * nw;
  return g;
}

inline size_t bwd_delta_bytes(const BwdPlan& p) {
  return ((size_t)p.B * p.T * p.Hq * sizeof(float) + 255) / 256 * 256;
}

inline size_t bwd_readers_bytes(const BwdPlan& p) {
  const size_t nb = (size_t)(p.T + p.bs - 1) / p.bs, nw = (size_t)(p.T + 31) / 32;
  return ((size_t)p.B * p.Hkv * nb * nw * sizeof(uint32_t) + 255) / 256 * 256;
}

inline size_t bwd_part_bytes(const BwdPlan& p) {
  const size_t ns = (size_t)bwd_segments(p);
  return ns > 1 ? ns * 2 * (size_t)p.B * p.T * p.Hkv * p.D * sizeof(float) : 0;
}

// byte offset of the forward's schedule in the backward's workspace
inline size_t bwd_schedule_offset(const BwdPlan& p) {
  return bwd_delta_bytes(p) + bwd_readers_bytes(p) + align_up(bwd_part_bytes(p), 256);
}

inline size_t bwd_workspace_bytes(const BwdPlan& p) { return bwd_schedule_offset(p) + p.fp.bytes; }

// cus: compute units of the device (the forward plan's grid; the layout of
// the workspace does not depend on it)
inline nsa_status make_bwd_plan(const nsa_dims* d, int32_t block_size, BwdPlan* p, int cus = 256) {
  if (!d) return NSA_ERROR_INVALID_VALUE;
  if (d->batch <= 0 || d->seqlen <= 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 ||
      d->head_dim <= 0 || d->num_selected <= 0 || block_size <= 0)
    return NSA_ERROR_INVALID_VALUE;
  if (d->num_q_heads % d->num_kv_heads) return NSA_ERROR_INVALID_VALUE;
  if (d->dtype != NSA_DTYPE_BF16) return NSA_ERROR_NOT_SUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return NSA_ERROR_NOT_SUPPORTED;
  if (block_size != 32 && block_size != 64 && block_size != 128) return NSA_ERROR_NOT_SUPPORTED;
  if (d->num_selected > 64) return NSA_ERROR_NOT_SUPPORTED;
  p->B = d->batch;
  p->T = d->seqlen;
  p->Hq = d->num_q_heads;
  p->Hkv = d->num_kv_heads;
  p->D = d->head_dim;
  p->S = d->num_selected;
  p->bs = block_size;
  p->G = p->Hq / p->Hkv;
  if (p->G <= 16) {
    p->gv = p->G;
    p->gpk = 1;
  } else if (p->G % 16 == 0 && p->G <= 1024) {
    p->gv = 16;
    p->gpk = p->G / 16;
  } else {
    return NSA_ERROR_NOT_SUPPORTED;
  }
  const int64_t rows = (int64_t)p->B * p->T;
  if (!product_le(rows, p->Hq, p->D, INT64_C(1) << 40) || !product_le(rows, p->Hkv, p->gpk, INT32_MAX / 2))
    return NSA_ERROR_NOT_SUPPORTED;
  // every launch of the backward must stay inside the 2^32 work-items a
  // grid dimension holds
  const BwdGrids g = bwd_grids(*p);
  if (g.dkdv * kBwdKvThreads >= (INT64_C(1) << 32) ||
      g.reduce * 256 >= (INT64_C(1) << 32))
    return NSA_ERROR_NOT_SUPPORTED;
  // the forward's plan of the same call (the backward needs its out and lse)
  const nsa_status fs = make_plan(d, block_size, 0, false, &p->fp, false, cus, true);
  if (fs != NSA_SUCCESS) return fs;
  if (!p->fp.bf16 || p->fp.ntpw != 1) return NSA_ERROR_NOT_SUPPORTED;
  return NSA_SUCCESS;
}

}  // namespace nsa
