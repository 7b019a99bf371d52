// Backward pass of the native sparse attention forward for gfx950: the
// gradients dQ, dK, dV of the operation of the ejKernel
// native_sparse_attention API page (module description and "Parameters").
// With P_s = exp(scale q.k_s - lse) over the token's visible keys:
//   Delta = dO . O,   dP_s = dO . v_s,   dS_s = P_s (dP_s - Delta)
//   dQ    = scale sum_s dS_s k_s
//   dK_s  = scale sum_{t, hq} dS_s q,    dV_s = sum_{t, hq} P_s dO
// (the chain rule through the masked softmax; the forward's lse is reused).
//
// dQ (with Delta = dO . O and the reader bitmaps of the dk/dv kernel) is the
// gradient mode of the forward's ring kernel (nsa_fwd.hip), run over the
// forward's own schedule of the same indices: it gathers every kept unit
// once per item, as the forward does.  The reader bitmaps hold, per
// (sequence, kv head, key block), a bit per token that keeps the block (from
// the row's first clamp(count, 0, S) entries 0 <= j <= own; atomic OR, so
// repeats and order do not matter).
//
// dkdv kernel: one workgroup per (sequence, kv head, 64-key chunk, token
// segment), one wave per 16-key tile, two workgroups per CU.  Wave 0 turns
// the chunk's reader bitmaps into a list of the segment's reader tokens, in
// token order (so the sums are deterministic).  The workgroup then walks the
// list kStepUnits units per step, a unit being tpt consecutive readers of
// the list x one head group (16 rows of (reader, query head)): all its
// lanes load the step's Q_t, dO_t, lse and Delta rows once into registers
// two steps ahead and store them into one of two LDS buffers, and each wave
// takes every unit of the step, one after the other: it forms S = Q K^T and
// dP = dO V^T for its 16 keys (K and V rows in registers as B operands), P
// and dS (a row sees a key iff its reader reads the key's block and the key
// is not past the reader), and accumulates dV += P^T dO and dK += dS^T Q
// with 16x16x16 MFMAs whose B operands (dO and Q, rows x d) are read
// transposed from the buffer.  The segments' partial sums are added in
// segment order by the reduce kernel; where one segment covers the sequence
// the kernel writes the final dK and dV itself and no reduce runs.  Every
// key row gets written (zeros where no token reads the block).
#include <utility>

#include "nsa.h"
#include "nsa_internal.h"
#include "nsa_device.h"

namespace nsa {

namespace {

using namespace dev;

constexpr int kKvTiles = kBwdKvThreads / 64;    // 16-key tiles per dk/dv workgroup (a 64-key chunk)
constexpr int kStepUnits = 2;  // units of 16 (reader, head) rows per dk/dv step, taken by every tile wave
constexpr int kSegMax = kBwdSegMax;   // readers of a chunk are split into token segments of at most this many tokens


struct BwdArgs {
  const void* q;          // [B, T, Hq, D] bf16
  const void* k;          // [B, T, Hkv, D]
  const void* v;
  const float* lse;       // [B, T, Hq]
  const void* dout;       // [B, T, Hq, D]
  float* dk;              // [B, T, Hkv, D]
  float* dv;
  float* delta;           // [B, T, Hq] workspace
  uint32_t* readers;      // [B, Hkv, nb, nw] workspace: bit t of block j = token t reads j
  float* part;            // [ns][2][B, T, Hkv, D] workspace: per token segment, dK (unscaled) and dV
  int32_t B, T, Hq, Hkv, bs, gv, gpk, nb, nw, ns, seg;   // seg: tokens per segment
  int32_t tpt;            // readers per dk/dv unit (16 / gv if gpk == 1, else 1)
  int32_t gv_magic;       // (1 << 16) / gv + 1: r / gv = (r * gv_magic) >> 16 for 0 <= r < 16
  float scale;
  float scale_log2;
};

// ---------------------------------------------------------------------------
// the reader bitmaps start cleared (the dq ring sets their bits)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_clear_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}


// ---------------------------------------------------------------------------
// dk, dv
// ---------------------------------------------------------------------------
// one unit of 16 (reader token, query head) rows as staged in LDS: the Q
// and dO rows, lse and Delta of each row, each row's last visible key of
// the chunk for each of the chunk's blocks, and the unit's header (the OR
// of its readers' block bits, its last reader)
template <int D>
struct KvUnit {
  static constexpr int kRow = D * 2;                  // bytes of one head's row
  static constexpr int kRows = 16 * kRow;             // Q (or dO) rows of 16 heads
  static constexpr int kLse = 2 * kRows;              // lse[16], then Delta[16]
  static constexpr int kLim = kLse + 2 * 64;          // int8 lim[2][16]
  static constexpr int kHdr = kLim + 64;              // int bits, int last token
  static constexpr int kBytes = kHdr + 64;
  static constexpr int kChunks = kRows / 16;          // 16-byte chunks of Q (or dO)
  static constexpr int kStepChunks = kStepUnits * 2 * kChunks;
  static constexpr int kThreads = 64 * kKvTiles;
  static constexpr int kLoads = kStepChunks / kThreads;   // 16-byte loads per lane per step
  static_assert(kStepChunks % kThreads == 0, "a step's chunks spread evenly over the workgroup");
};

// the next step's Q_t / dO_t chunks and one lse or Delta value, in flight
// in registers while the current step computes
template <int D>
struct KvStage {
  u32x4 v[KvUnit<D>::kLoads];
  float f;
};

// Row r of unit u.  Packed (tpt > 1 readers per unit, then gpk = 1): reader
// u tpt + r / gv of the list, query head h gv + r % gv; the row exists if
// r < tpt gv and its reader is on the list.  Otherwise: reader u / gpk,
// query head (h gpk + u % gpk) gv + r; the row exists if r < gv.  (r / gv
// as (r * gv_magic) >> 16, exact for r < 16.)
template <bool kPacked>
__device__ __forceinline__ int row_reader(const BwdArgs& a, int u, int r) {
  return kPacked ? u * a.tpt + ((r * a.gv_magic) >> 16) : u / a.gpk;
}
template <bool kPacked>
__device__ __forceinline__ int row_head(const BwdArgs& a, int h, int u, int r) {
  return kPacked ? h * a.gv + (r - ((r * a.gv_magic) >> 16) * a.gv) : (h * a.gpk + u % a.gpk) * a.gv + min(r, a.gv - 1);
}
template <bool kPacked>
__device__ __forceinline__ bool row_exists(const BwdArgs& a, int u, int r, int nread) {
  return kPacked ? (r < a.tpt * a.gv && row_reader<true>(a, u, r) < nread) : r < a.gv;
}

template <int D, bool kPacked>
__device__ __forceinline__ void kv_stage_load(const BwdArgs& a, const uint16_t* rlist, int nunits, int nread,
                                              int seg_lo, int64_t tok_base, int h, int tid, int step,
                                              KvStage<D>& st) {
  using U = KvUnit<D>;
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ dO = reinterpret_cast<const __bf16*>(a.dout);
#pragma unroll
  for (int l = 0; l < U::kLoads; l++) {
    const int gi = l * U::kThreads + tid;
    const int unit = gi / (2 * U::kChunks);
    const int rem = gi % (2 * U::kChunks);
    const int row = (rem % U::kChunks) / (D / 8);
    const int ck = rem % (D / 8);
    // past the last unit or reader: a clamped in-bounds address (the value
    // is replaced by zeros or never read)
    const int u = min(kStepUnits * step + unit, nunits - 1);
    const int t = seg_lo + (rlist[min(row_reader<kPacked>(a, u, row), nread - 1)] & 4095);
    const int hq = row_head<kPacked>(a, h, u, row);
    const __bf16* src = rem < U::kChunks ? Q : dO;
    st.v[l] = *reinterpret_cast<const u32x4*>(src + ((tok_base + t) * a.Hq + hq) * D + ck * 8);
  }
  // lanes 0 .. 32 kStepUnits - 1: unit tid / 32, lse or Delta ((tid / 16) % 2), row tid % 16
  const int unit = (tid >> 5) % kStepUnits;
  const int u = min(kStepUnits * step + unit, nunits - 1);
  const int t = seg_lo + (rlist[min(row_reader<kPacked>(a, u, tid & 15), nread - 1)] & 4095);
  const int hq = row_head<kPacked>(a, h, u, tid & 15);
  st.f = ((tid >> 4) & 1 ? a.delta : a.lse)[(tok_base + t) * a.Hq + hq];
}

template <int D, bool kPacked>
__device__ __forceinline__ void kv_stage_store(const BwdArgs& a, const uint16_t* rlist, int nunits, int nread,
                                               int seg_lo, int kbase, NSA_LDS char* buf, int tid, int step,
                                               const KvStage<D>& st) {
  using U = KvUnit<D>;
#pragma unroll
  for (int l = 0; l < U::kLoads; l++) {
    const int gi = l * U::kThreads + tid;
    const int unit = gi / (2 * U::kChunks);
    const int rem = gi % (2 * U::kChunks);
    const int row = (rem % U::kChunks) / (D / 8);
    const int ck = rem % (D / 8);
    const int u = min(kStepUnits * step + unit, nunits - 1);
    // rows that do not exist are zero (their P and dS are zero too, and 0
    // times a stale value could be NaN)
    const u32x4 z = {0u, 0u, 0u, 0u};
    // row-major 16-byte chunks XOR-swizzled by row, as in the forward's V
    // slot: the A-operand reads and the transposed reads are conflict-free
    *(NSA_LDS u32x4*)(buf + unit * U::kBytes + (rem < U::kChunks ? 0 : U::kRows) + row * U::kRow +
                      ((ck ^ v_swizzle<D>(row)) * 16)) = row_exists<kPacked>(a, u, row, nread) ? st.v[l] : z;
  }
  if (tid < 32 * kStepUnits) {
    const int unit = tid >> 5;
    const int which = (tid >> 4) & 1;
    const int r = tid & 15;
    const int u = min(kStepUnits * step + unit, nunits - 1);
    // a row that does not exist: lse = +inf makes its P zero, Delta = 0
    const float val = row_exists<kPacked>(a, u, r, nread) ? st.f : (which ? 0.f : INFINITY);
    *(NSA_LDS float*)(buf + unit * U::kBytes + U::kLse + which * 64 + r * 4) = val;
  } else if (kPacked && tid < 128) {
    // wave 1, 16 lanes per unit: for each row and each block of the chunk,
    // the offset from the chunk's first key (kbase) of the last key the
    // row sees, clamped to [-1, 63] (-1: none: the row's reader does not
    // read that block or the row does not exist); and the unit's header:
    // the block bits of any of its readers and its last reader's token (the
    // list is in token order, rows that do not exist hold entry 0)
    static_assert(kStepUnits <= 4, "16 lanes of wave 1 per unit");
    const int unit = (tid >> 4) & 3;
    const int r = tid & 15;
    const int u = min(kStepUnits * step + unit, nunits - 1);
    const int e = row_exists<kPacked>(a, u, r, nread) ? (int)rlist[row_reader<kPacked>(a, u, r)] : 0;
    const uint64_t any0 = __ballot(((e >> 12) & 1) != 0);
    const uint64_t any1 = __ballot(((e >> 13) & 1) != 0);
    const int last = rlist[min(row_reader<kPacked>(a, u, 0) + a.tpt, nread) - 1] & 4095;
    if (unit < kStepUnits) {
      const int off = row_exists<kPacked>(a, u, r, nread) ? min(max(seg_lo + (e & 4095) - kbase, -1), 63) : -1;
#pragma unroll
      for (int tb = 0; tb < 2; tb++)
        *(NSA_LDS signed char*)(buf + unit * U::kBytes + U::kLim + tb * 16 + r) =
            (signed char)(((e >> (12 + tb)) & 1) ? off : -1);
      if (r == 0) {
        // lanes 16 unit .. 16 unit + 15 of the wave are the unit's rows
        const int bits = (((any0 >> (16 * unit)) & 0xFFFFull) != 0ull ? 1 : 0) |
                         (((any1 >> (16 * unit)) & 0xFFFFull) != 0ull ? 2 : 0);
        *(NSA_LDS int*)(buf + unit * U::kBytes + U::kHdr) = bits;
        *(NSA_LDS int*)(buf + unit * U::kBytes + U::kHdr + 4) = last;
      }
    }
  }
}

// LDS writes of every wave done and visible before any wave goes on; global
// loads in flight stay in flight (no vector-memory wait)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// kPacked: tpt > 1 readers share a unit's 16 rows; each row then carries its
// own reader's token and block bits
template <int D, bool kPacked>
__global__ void __launch_bounds__(64 * kKvTiles) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dkdv_kernel(BwdArgs a) {
  using U = KvUnit<D>;
  constexpr int KT = D / 32;   // k-steps of S = Q K^T over d
  constexpr int DT = D / 16;   // 16-column d tiles of dK, dV
  constexpr int kRow = U::kRow;
  // two step buffers of kStepUnits units each
  __shared__ __attribute__((aligned(1024))) char slot[2][kStepUnits * U::kBytes];
  // the chunk's readers in the segment: token - segment start (bits 0..11),
  // and which of the chunk's key blocks the token reads (bits 12, 13)
  __shared__ uint16_t rlist[kSegMax];
  __shared__ int nread_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15;
  const int g = lane >> 4;
  const int nchunk = (a.T + 63) / 64;
  // workgroup order: first chunk 0 of every (sequence, kv head, segment):
  // block 0 is read by most tokens under attention-sink selections, so the
  // longest workgroups start first; then segment-major, the chunks of one
  // token segment in a row, so the Q_t and dO_t rows those workgroups
  // gather come from HBM about once and then from the last-level cache
  const int nbhs = a.B * a.Hkv * a.ns;
  int chunk, r;
  if ((int)blockIdx.x < nbhs) {
    chunk = 0;
    r = blockIdx.x;
  } else {
    const int rest = max(nchunk - 1, 1);
    const int i = blockIdx.x - nbhs;
    chunk = 1 + i % rest;
    r = i / rest;
  }
  const int seg = r % a.ns;                    // token segment [seg * a.seg, + a.seg)
  const int bh = r / a.ns;
  const int seg_lo = seg * a.seg;
  const int seg_hi = min(seg_lo + a.seg, a.T);
  // a segment that ends at or before the chunk's first key has no reader:
  // the whole workgroup leaves (and the reduction skips it by the same rule)
  if (seg_hi <= chunk * 64) return;
  const int h = bh % a.Hkv;
  const int b = bh / a.Hkv;
  const int tile = wave;                       // 16-key tile of the chunk
  const int key0 = chunk * 64 + tile * 16;     // the tile's first key (position in the sequence)
  const bool active = key0 < a.T;              // every wave reaches the barriers below
  const int blk0 = chunk * 64 / a.bs;          // the chunk's first key block
  const int nblk = a.bs >= 64 ? 1 : 64 / a.bs; // key blocks in the chunk (bs = 32: two)
  const int tblk = a.bs >= 64 ? 0 : tile * 16 / a.bs;   // the tile's block among them
  const int64_t tok_base = (int64_t)b * a.T;

  // the reader list: tokens t >= the chunk's first key in the segment that
  // read any of the chunk's blocks, in token order (wave 0; <= 128 words)
  if (wave == 0) {
    const int t_lo = max(chunk * 64, seg_lo);  // a multiple of 32
    const int w_lo = t_lo / 32;
    const int nwd = (seg_hi + 31) / 32 - w_lo;
    const uint32_t* rb = a.readers + (((int64_t)b * a.Hkv + h) * a.nb + blk0) * a.nw;
    int base = 0;                              // readers listed by earlier passes
    for (int w0 = 0; w0 < nwd; w0 += 64) {     // 64 words (2048 tokens) per pass
      const int wi = w_lo + w0 + lane;
      uint32_t per0 = 0u, per1 = 0u;           // the words of the chunk's first and second block
      if (w0 + lane < nwd) {
        per0 = rb[wi];
        if (nblk > 1 && blk0 + 1 < a.nb) per1 = rb[a.nw + wi];
        if (wi == (seg_hi - 1) / 32 && (seg_hi & 31) != 0) {
          const uint32_t m = 0xFFFFFFFFu >> (32 - (seg_hi & 31));
          per0 &= m;
          per1 &= m;
        }
      }
      uint32_t any = per0 | per1;
      const int cnt = __builtin_popcount(any);
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      int pos = base + incl - cnt;
      while (any != 0u) {
        const int bit = __builtin_ctz(any);
        any &= any - 1u;
        const int t = wi * 32 + bit;
        rlist[pos++] = (uint16_t)((t - seg_lo) | (((per0 >> bit) & 1u) << 12) | (((per1 >> bit) & 1u) << 13));
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) nread_s = base;
  }
  __syncthreads();
  const int nread = nread_s;
  // units of tpt readers x one head group, reader-major
  const int nunits = (nread + a.tpt - 1) / a.tpt * a.gpk;
  const int nsteps = (nunits + kStepUnits - 1) / kStepUnits;

  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) {
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (nsteps > 0) {
    // K and V rows of the tile as B operands (lane (c, g): key row c, d = 32 kk + 8 g)
    const __bf16* __restrict__ Kp = reinterpret_cast<const __bf16*>(a.k);
    const __bf16* __restrict__ Vp = reinterpret_cast<const __bf16*>(a.v);
    const int key = key0 + c;
    const bool kvalid = active && key < a.T;
    const int64_t krow = ((tok_base + (kvalid ? key : 0)) * a.Hkv + h) * D;
    bf16x8 kf[KT], vf[KT];
#pragma unroll
    for (int kk = 0; kk < KT; kk++) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(Kp + krow + kk * 32 + g * 8);
      vf[kk] = *reinterpret_cast<const bf16x8*>(Vp + krow + kk * 32 + g * 8);
    }
    const float sl = a.scale_log2;
    const int kofs = tile * 16 + c;               // this lane's key, from the chunk's first key

    // unit j of a step: unit kStepUnits * step + j, if it exists, reads the
    // tile's block and reaches the tile's first key
    auto compute = [&](NSA_LDS const char* buf, int step, int j) __attribute__((always_inline)) {
      const int slot_unit = j;
      const int u = kStepUnits * step + slot_unit;
      if (u >= nunits) return;
      NSA_LDS const char* qs = buf + slot_unit * U::kBytes;
      NSA_LDS const char* ds = qs + U::kRows;
      // skip the unit if none of its readers reads the tile's block or the
      // tile starts past its last reader
      int t = 0;   // the unit's reader (one reader per unit)
      if constexpr (kPacked) {
        const int ubits = __builtin_amdgcn_readfirstlane(*(NSA_LDS const int*)(qs + U::kHdr));
        const int ulast = seg_lo + __builtin_amdgcn_readfirstlane(*(NSA_LDS const int*)(qs + U::kHdr + 4));
        if (!active || !((ubits >> tblk) & 1) || key0 > ulast) return;
      } else {
        const int e = rlist[u / a.gpk];
        t = seg_lo + (e & 4095);
        if (!active || !((e >> (12 + tblk)) & 1) || key0 > t) return;
      }
      // every LDS read of the step goes out first, so their latencies
      // overlap: Q_t, dO_t of the group's heads as A operands (lane (c, g):
      // head c, d = 32 kk + 8 g), lse and Delta of heads 4 g .. 4 g + 3, and
      // the B operands of dV and dK (heads 4 g .. + 3 at d = 16 dt + c)
      // read transposed
      bf16x8 qa[KT], da[KT];
#pragma unroll
      for (int kk = 0; kk < KT; kk++) {
        const int ch = (kk * 4 + g) ^ v_swizzle<D>(c);
        qa[kk] = *(NSA_LDS const bf16x8*)(qs + c * kRow + ch * 16);
        da[kk] = *(NSA_LDS const bf16x8*)(ds + c * kRow + ch * 16);
      }
      const f32x4 l4 = *(NSA_LDS const f32x4*)(qs + U::kLse + g * 16);
      const f32x4 d4 = *(NSA_LDS const f32x4*)(qs + U::kLse + 64 + g * 16);
      // rows 4 g .. 4 g + 3: last visible key of the tile's block, from the chunk's first key
      const int lim4 = kPacked ? *(NSA_LDS const int*)(qs + U::kLim + tblk * 16 + g * 4) : 0;
      bf16x4 qb[DT], db[DT];
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        const int row = g * 4 + (c >> 2);
        const int d0 = dt * 16 + (c & 3) * 4;
        const int off = row * kRow + ((d0 >> 3) ^ v_swizzle<D>(row)) * 16 + (d0 & 7) * 2;
        qb[dt] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((NSA_LDS s16x4*)(qs + off)));
        db[dt] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((NSA_LDS s16x4*)(ds + off)));
      }
      __builtin_amdgcn_sched_barrier(0);
      // S = Q K^T and dP = dO V^T: lane (c, g) holds heads 4 g + jj of key c
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f}, pacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KT; kk++) {
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], kf[kk], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(da[kk], vf[kk], pacc, 0, 0, 0);
      }
      bf16x4 pa, sa;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const bool see = kPacked ? kofs <= (int)(signed char)(lim4 >> (8 * jj)) : key <= t;
        const float p = see ? fast_exp2(__builtin_fmaf(sacc[jj], sl, -l4[jj] * 1.4426950408889634f)) : 0.f;
        pa[jj] = (__bf16)p;
        sa[jj] = (__bf16)(p * (pacc[jj] - d4[jj]));
      }
      // dV += P^T dO, dK += dS^T Q
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        dv[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, db[dt], dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(sa, qb[dt], dk[dt], 0, 0, 0);
      }
    };

    // software pipeline over steps: the workgroup loads step s + 2 into
    // registers while it computes step s from one LDS buffer, then stores
    // step s + 1 into the other; one barrier per step of kStepUnits units
    NSA_LDS char* buf0 = (NSA_LDS char*)&slot[0][0];
    NSA_LDS char* buf1 = (NSA_LDS char*)&slot[1][0];
    KvStage<D> s0, s1;
    kv_stage_load<D, kPacked>(a, rlist, nunits, nread, seg_lo, tok_base, h, tid, 0, s0);
    kv_stage_load<D, kPacked>(a, rlist, nunits, nread, seg_lo, tok_base, h, tid, 1, s1);
    kv_stage_store<D, kPacked>(a, rlist, nunits, nread, seg_lo, chunk * 64, buf0, tid, 0, s0);
    lds_barrier();
    for (int step = 0; step < nsteps; step += 2) {
      kv_stage_load<D, kPacked>(a, rlist, nunits, nread, seg_lo, tok_base, h, tid, step + 2, s0);
#pragma unroll
      for (int j = 0; j < kStepUnits; j++) compute(buf0, step, j);
      kv_stage_store<D, kPacked>(a, rlist, nunits, nread, seg_lo, chunk * 64, buf1, tid, step + 1, s1);
      lds_barrier();
      kv_stage_load<D, kPacked>(a, rlist, nunits, nread, seg_lo, tok_base, h, tid, step + 3, s1);
#pragma unroll
      for (int j = 0; j < kStepUnits; j++) compute(buf1, step + 1, j);
      kv_stage_store<D, kPacked>(a, rlist, nunits, nread, seg_lo, chunk * 64, buf0, tid, step + 2, s0);
      lds_barrier();
    }
  }
  if (!active) return;

  // the segment's partial sum dS^T Q and P^T dO; lane (c, g) holds keys 4 g + jj at d = 16 dt + c
  // (with one segment the sums are final: dK = scale dS^T Q, dV = P^T dO
  // go straight to the outputs)
  const int64_t plane = (int64_t)a.B * a.T * a.Hkv * D;
  const bool whole = a.ns == 1;
  float* pk = whole ? a.dk : a.part + (int64_t)seg * 2 * plane;
  float* pv = whole ? a.dv : pk + plane;
  const float ks = whole ? a.scale : 1.f;
#pragma unroll
  for (int jj = 0; jj < 4; jj++) {
    const int kr = key0 + g * 4 + jj;
    if (kr >= a.T) continue;
    const int64_t o = ((tok_base + kr) * a.Hkv + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      pk[o + dt * 16 + c] = dk[dt][jj] * ks;
      pv[o + dt * 16 + c] = dv[dt][jj];
    }
  }
}

// dK = scale * sum over the key's segments, dV = sum over them, in segment
// order; segments that end at or before the key's 64-key chunk hold nothing
// (their workgroups left without writing)
template <int D>
__global__ void __launch_bounds__(256) bwd_reduce_kernel(BwdArgs a) {
  const int64_t plane = (int64_t)a.B * a.T * a.Hkv * D;
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;   // float4 index into a plane
  if (i4 * 4 >= plane) return;
  const int64_t rowi = i4 * 4 / D;                               // (b * T + key) * Hkv + h
  const int key = (int)((rowi / a.Hkv) % a.T);
  const int seg0 = (key / 64) * 64 / a.seg;                 // first segment ending after the chunk start
  f32x4 sk = f32x4{0.f, 0.f, 0.f, 0.f}, sv = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sgi = seg0; sgi < a.ns; sgi++) {
    const float* pk = a.part + (int64_t)sgi * 2 * plane;
    sk += *reinterpret_cast<const f32x4*>(pk + i4 * 4);
    sv += *reinterpret_cast<const f32x4*>(pk + plane + i4 * 4);
  }
  *reinterpret_cast<f32x4*>(a.dk + i4 * 4) = sk * a.scale;
  *reinterpret_cast<f32x4*>(a.dv + i4 * 4) = sv;
}

}  // namespace

hipError_t launch_bwd(const BwdPlan& p, const void* q, const void* k, const void* v, const void* out,
                      const float* lse, const void* dout, const int32_t* block_indices,
                      const int32_t* block_counts, float scale, float* dq, float* dk, float* dv,
                      float* delta, hipStream_t stream) {
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.lse = lse;
  a.dout = dout;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.B = p.B;
  a.T = p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.bs = p.bs;
  a.gv = p.gv;
  a.gpk = p.gpk;
  a.tpt = bwd_unit_readers(p);
  a.gv_magic = bwd_gv_magic(p);
  a.nb = (p.T + p.bs - 1) / p.bs;
  a.nw = (p.T + 31) / 32;
  a.readers = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(delta) + bwd_delta_bytes(p));
  a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(a.readers) + bwd_readers_bytes(p));
  a.seg = bwd_seg_tokens(p);
  a.ns = bwd_segments(p);
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  const BwdGrids gr = bwd_grids(p);   // make_bwd_plan kept every grid inside 2^32 work-items
  hipLaunchKernelGGL(bwd_clear_kernel, dim3((unsigned)std::min<int64_t>((gr.clear_words + 255) / 256, 4096)),
                     dim3(256), 0, stream, a.readers, gr.clear_words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dQ, Delta and the reader bitmaps from the forward's ring over its own
  // schedule of the indices, then dK / dV and their segment sums; a launch
  // that fails leaves the later ones unlaunched
  char* fws = reinterpret_cast<char*>(delta) + bwd_schedule_offset(p);   // delta opens the workspace
  e = launch_schedule(p.fp, block_indices, block_counts, nullptr, fws, stream);
  if (e != hipSuccess) return e;
  e = launch_dq_ring(p.fp, q, k, v, out, lse, dout, scale, dq, delta, a.readers, a.nb, a.nw, fws, stream);
  if (e != hipSuccess) return e;
  auto two = [&](auto kv_fn, auto red_fn) -> hipError_t {
    hipLaunchKernelGGL(kv_fn, dim3((unsigned)gr.dkdv), dim3(kBwdKvThreads), 0, stream, a);
    hipError_t r = hipGetLastError();
    if (r != hipSuccess || a.ns == 1) return r;   // one segment: dk, dv are written already
    hipLaunchKernelGGL(red_fn, dim3((unsigned)gr.reduce), dim3(256), 0, stream, a);
    return hipGetLastError();
  };
  const bool packed = a.tpt > 1;
  if (p.D == 64)
    return packed ? two(bwd_dkdv_kernel<64, true>, bwd_reduce_kernel<64>)
                  : two(bwd_dkdv_kernel<64, false>, bwd_reduce_kernel<64>);
  if (p.D == 128)
    return packed ? two(bwd_dkdv_kernel<128, true>, bwd_reduce_kernel<128>)
                  : two(bwd_dkdv_kernel<128, false>, bwd_reduce_kernel<128>);
  return hipErrorInvalidValue;
}

}  // namespace nsa
