// Native sparse attention forward kernels for gfx950 (CDNA4).
//
// Operation (ejKernel native_sparse_attention API page, module description
// and "Parameters"): for each query token, the query heads of kv head h
// attend to the keys of the blocks listed for (token, h), causal inside the
// token's own block; softmax(scale * q.k) weighted sum of v, plus the
// log-sum-exp of the scores.
//
// bf16 kernel: persistent workgroups of 16 waves, one per CU.
//  * 4 loader waves stream the K and V rows of each item's merged block list
//    (ascending block order, `kb` keys per unit) into a ring of R LDS slots.
//    Loader p owns the units v = p (mod 4).  Once every attention wave that
//    reads the slot's occupant has released its K rows, it sends the new K
//    rows straight to LDS with 16-byte buffer loads and publishes them when
//    they have landed; then, once the V rows are released too, it sends the
//    new V rows the same way and publishes them.  A unit's V loads are
//    issued only after its K rows have landed: the memory pipeline serves a
//    CU's loads in order, and V queued ahead of another loader's K would
//    delay the scores every reader waits for first.
//  * 12 attention waves each own a fixed set of the item's tokens and walk
//    the same unit sequence without any barrier: a wave waits only for the
//    unit's data, computes its own tokens that selected the block, releases
//    the slot and moves on, so tokens with different block lists do not
//    hold each other up.  A gathered block feeds every token of the item
//    that listed it, and every query head of those tokens.
//  * Matrix work, per 16 query columns (the G heads of one token, or 16/G
//    tokens x G heads when G < 16):
//        S^T (keys x cols) = K (keys x D) . Q^T (D x cols)     A = K rows
//        O^T (D x cols)   += V^T (D x keys) . P^T (keys x cols)
//    with v_mfma_f32_16x16x32_bf16.  In this orientation the fp32 S^T
//    accumulator layout (lane = column, four consecutive keys per lane group)
//    is exactly the B-operand layout of P^T, so P stays in registers.  K
//    fragments are ds_read_b128 from the slot; V^T fragments come from
//    ds_read_b64_tr_b16, the gfx950 transposing LDS read (lanes 4r..4r+3 of a
//    16-lane group supply row r of a 4 x 16 tile, lane i receives column i).
//    Both slot halves are XOR-swizzled by 16-byte chunk so these reads are
//    free of bank conflicts.
//  * fp32 online softmax in the log2 domain: scores scaled by scale*log2(e),
//    v_exp_f32 for 2^x, running max and normaliser per column (the
//    (output, max, normaliser) carry of a flash-attention block step, as in
//    `flash_attention_block` on the ejKernel ragged-decode page); masks are
//    evaluated only on units that hold a token's own block or that not every
//    token of the tile selected.
//  * Every wait is a bounded spin: a wave that waits too long sets the
//    status word in the workspace and leaves, so the grid always drains.
//
// fp32 kernel: one wave per (item, token group) reading K and V straight
// from global memory, v_mfma_f32_16x16x4_f32, P kept in fp32.
#include <cstdlib>
#include <utility>

#include "nsa.h"
#include "nsa_internal.h"
#include "nsa_device.h"

namespace nsa {

namespace {

using namespace dev;

// Schedule reads go through the constant address space: with a wave-uniform
// address they become scalar loads, which keeps the vector-memory counter
// free for the loader waves' own direct-to-LDS traffic.
template <typename T>
__device__ __forceinline__ T ld_const(const T* p, int64_t i) {
#if defined(__HIP_DEVICE_COMPILE__)
  return ((const NSA_CONST T*)p)[i];
#else
  return p[i];
#endif
}

constexpr int kMaxSpin = 1 << 22;        // polls before a wait is declared stuck
constexpr int32_t kErrStuck = NSA_DEVICE_WAIT_EXPIRED;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const ItemHeader* hdr;
  const int32_t* blocks;
  const uint32_t* masks;   // [n_items * umax][mw] token bits of each merged entry
  const uint32_t* units;
  const int32_t* worklist;
  int32_t* err;
  int32_t Ttot;     // packed token rows
  int32_t Hq, Hkv, G, gv, gpk, tpt, tpw, tq, mw, n_tiles, n_items, umax, umax_units, bs, nwg;
  float scale_log2;  // scale * log2(e)
  int32_t split_release;   // attention waves release a slot's K rows after S^T
  int32_t serial;          // debug: one unit in the ring at a time (NSA_DEBUG=1)
  // the gradient mode of the ring kernel (dq): its inputs and outputs
  const void* dout;        // [rows, Hq, D] bf16
  const void* fwd_out;     // [rows, Hq, D] bf16, the forward's output
  const float* lse_in;     // [rows, Hq] natural-log lse of the forward
  float* dq;               // [rows, Hq, D] fp32
  float* delta;            // [rows, Hq] fp32: dO . O
  uint32_t* readers;       // [B, Hkv, nb, nw]: bit t of block j = token t keeps j
  int32_t rd_nb, rd_nw;
  int32_t T;               // tokens per sequence (fixed-length sequences)
  float scale;
};

// A header is used only if it stays inside the tensors: a workspace that does
// not hold a matching schedule then cannot make the kernels touch memory
// outside their arguments.
__device__ __forceinline__ bool header_ok(ItemHeader& hd, const FwdArgs& a) {
  if (hd.ntok <= 0 || hd.ntok > a.tq || hd.pos0 < 0 || hd.tok0 < hd.pos0) return false;
  if (hd.tok0 + hd.ntok > a.Ttot) return false;
  hd.nunion = min(max(hd.nunion, 0), a.umax);
  return true;
}

// Column c of a 16-column tile whose first token is `tok_base` -> token
// offset, head inside the group, valid.
__device__ __forceinline__ void column_of(int c, int gv, int tpt, int tok_base, int ntok, int& tau,
                                          int& head, bool& valid) {
  const int lt = c / gv;
  tau = tok_base + lt;
  head = c - lt * gv;
  valid = (lt < tpt) && (tau < ntok);
}

// `count` token bits from bit `first` of an entry's token set, given the
// set's word that holds them (word first / 32: count is a power of two <= 32
// and first a multiple of it, so the field never straddles words).
__device__ __forceinline__ uint32_t mask_field(uint32_t word, int first, int count) {
  const uint32_t sh = word >> (first & 31);
  return count >= 32 ? sh : (sh & ((1u << count) - 1u));
}

// Ring counters live in LDS and are accessed with relaxed atomics; ordering
// is made explicit so that no wait covers more than it must (an acquire or
// release at workgroup scope would also drain the loader waves' in-flight
// direct-to-LDS loads):
//  * a loader publishes a unit after s_waitcnt vmcnt has retired that unit's
//    own loads (their data is then in LDS);
//  * an attention wave releases a slot after an LDS-only release fence
//    (s_waitcnt lgkmcnt(0): its reads of the slot have returned);
//  * reads of a slot are issued only after the counter that allows them was
//    observed (control dependence, plus a compiler fence).
__device__ __forceinline__ uint64_t lds_poll2(int* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_poll(int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Loader-side counter accesses.  The compiler cannot tell the ring slots
// (written by direct-to-LDS loads) from the counters, and would retire every
// in-flight load before touching a counter; written as plain LDS
// instructions they wait only for themselves.
__device__ __forceinline__ uint32_t lds_offset(int* p) {
  return (uint32_t)(uintptr_t)((NSA_LDS int*)p);
}
__device__ __forceinline__ int loader_poll(int* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_offset(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);   // the same value in every lane
}
// One increment per wave: only lane 0 adds (every active lane of an LDS
// atomic would otherwise add its own 1).
__device__ __forceinline__ void loader_bump(int* p) {
  if ((threadIdx.x & 63) == 0)
    asm volatile("ds_add_u32 %0, %1" : : "v"(lds_offset(p)), "v"(1) : "memory");
}
// An attention wave's release: its LDS reads have returned (release fence),
// then lane 0 adds one with a plain ds_add (no return value, no lane
// reduction around it).
__device__ __forceinline__ void lds_release_bump(int* p) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  if ((threadIdx.x & 63) == 0) asm volatile("ds_add_u32 %0, %1" : : "v"(lds_offset(p)), "v"(1) : "memory");
}

// Item of round r for workgroup g: each XCD takes a contiguous stretch of
// the longest-first list per round, so neighbouring items (same head group,
// adjacent tokens, shared sink/local blocks) meet in one L2.  Odd rounds
// walk the round's stretch in reverse (a snake over the workgroups), so the
// workgroup that drew one of the heaviest items of a round draws one of the
// lightest of the next: with few rounds (short workloads) the workgroups'
// totals stay close.
__device__ __forceinline__ int list_position(int g, int round, int nwg) {
  const int per = nwg / kXcds;
  const int p = (g % kXcds) * per + g / kXcds;
  return round * nwg + ((round & 1) ? nwg - 1 - p : p);
}

// Item walk shared by every wave of a workgroup: rounds of the
// longest-first list, skipping items whose header is out of range.
struct ItemCursor {
  int round;
  int item;
  ItemHeader hd;
  bool valid;
};

__device__ __forceinline__ void next_item(ItemCursor& cs, const FwdArgs& a) {
  while (true) {
    const int pos = list_position(blockIdx.x, cs.round, a.nwg);
    if (pos >= a.n_items) {
      cs.valid = false;
      return;
    }
    cs.round++;
    const int item = ld_const(a.worklist, pos);
    if (item < 0 || item >= a.n_items) continue;
    const int32_t* hw = reinterpret_cast<const int32_t*>(a.hdr) + (int64_t)item * 4;
    ItemHeader hd{ld_const(hw, 0), ld_const(hw, 1), ld_const(hw, 2), ld_const(hw, 3)};
    if (!header_ok(hd, a)) continue;
    cs.item = item;
    cs.hd = hd;
    cs.valid = true;
    return;
  }
}

// ---------------------------------------------------------------------------
// bf16 ring kernel
//
// Units: every item contributes nunion * (bs / kb) units, numbered
// v = (units of earlier items of this workgroup) + u * (bs / kb) + sb, in the
// same order on every wave; unit v lives in slot v % R.  A unit is "live" if
// its block is in range and its first key is not past the item's last token.
// An attention wave reads a unit iff the unit is live, one of the wave's
// tokens listed the block and the unit's first key is not past the wave's
// last token; the number of such waves is the unit's participant count,
// computed by the scheduler into the unit's word.
//  * ready2[s][0] / ready2[s][1] count publications of the K rows / V rows
//    of the units of slot s (one each per unit, live or not, in unit order):
//    the K rows of unit v are readable once ready2[v % R][0] >= v / R + 1,
//    its V rows once ready2[v % R][1] >= v / R + 1.  An attention wave reads
//    both counters with one 8-byte load when it waits for the K rows, and
//    polls the V counter again only if the V rows were not yet published.
//  * done[s] counts participant releases of slot s after their V reads: the
//    loader may overwrite slot s once done[s] has reached the participant
//    total of all earlier occupants.  With split releases (few readers per
//    unit) done_k[s] also counts releases after the S^T reads, and the K rows
//    may be replaced as soon as done_k[s] reaches that total.  A wave can only reach a later occupant after it was
//    published, which already required every reader of the earlier one to
//    have released it, so the counts of successive occupants never mix.
// Waves therefore touch only the units they compute.
// ---------------------------------------------------------------------------
template <int D, int KB>
struct RingCfg {
  static constexpr int kSlotBytes = 2 * KB * D * 2;              // K then V
  static constexpr int kR0 = (128 * 1024) / kSlotBytes;
  static constexpr int R = kR0 > 8 ? 8 : kR0;                    // ring slots
  static constexpr int kLoadsKV = (KB * D * 2) / 1024;           // 1 KB loads per K (or V) unit
  static constexpr int kRowsPerLoad = 1024 / (D * 2);
  static_assert(R % kProducers == 0, "slots per loader");
  static_assert(kLoadsKV <= 16, "at most 16 loads per K (or V) half of a unit");
};

// kPosScale: the softmax scale is > 0, so max(scale * s) = scale * max(s) and
// masked scores (-inf) stay -inf through the scaling FMA; otherwise each
// score is scaled and tested on its own.
// kDq: the gradient dQ of the same gather (same items, units and ring): per
// (token, unit) pair S^T = K Q^T, P = 2^(scale log2e S - lse log2e), dP^T =
// V dO^T, dS = P (dP - Delta), dQ^T += K^T dS^T; the V rows are stored
// row-swizzled like the K rows (both are read as rows), K is read again
// transposed for dQ, so a slot is released once, after the last reads.
template <int D, int KB, int NTPW, bool kPosScale, bool kDq>
__global__ void __launch_bounds__(64 * (kConsumers + kProducers), 1) fwd_bf16_ring_kernel(FwdArgs a) {
  static_assert(64 * (kConsumers + kProducers) <= 1024, "workgroup size");
  static_assert(NTPW == 1, "the ring kernel runs one 16-column tile per attention wave");
  using C = RingCfg<D, KB>;
  constexpr int R = C::R;
  constexpr int KT = D / 32;   // k-steps of S^T = K Q^T
  constexpr int MT = KB / 16;  // 16-key row tiles of S^T
  constexpr int KQ = KB / 32;  // 32-key k-steps of O^T += V^T P^T
  constexpr int DT = D / 16;   // 16-row tiles of O^T
  constexpr int CH = D / 8;    // 16-byte chunks per row

  __shared__ __attribute__((aligned(1024))) char ring[R][C::kSlotBytes];
  // the K and V publication counters of a slot side by side: one 8-byte read polls both
  __shared__ __attribute__((aligned(8))) int ready2[R][2];
  __shared__ int done_k[R];
  __shared__ int done[R];
  __shared__ int serial_done;   // debug mode: units fully released so far

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar control flow
  if (threadIdx.x < R) {
    ready2[threadIdx.x][0] = 0;
    ready2[threadIdx.x][1] = 0;
    done_k[threadIdx.x] = 0;
    done[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) serial_done = 0;
  __syncthreads();

  const int nsb = a.bs / KB;  // units per listed block
  ItemCursor cs;
  cs.round = 0;
  next_item(cs, a);

  if (wave >= kConsumers) {
    // ------------------------------------------------------------ loader
    // Loader p owns the units v with v % kProducers == p, and the slots
    // those units map to; it places its units one after another.
    const char* __restrict__ K = reinterpret_cast<const char*>(a.k);
    const char* __restrict__ V = reinterpret_cast<const char*>(a.v);
    const int p = wave - kConsumers;
    const int row_bytes = a.Hkv * D * 2;      // stride between key rows of one kv head
    // Per-lane byte offsets of the unit's loads from the unit's first row.
    // Load ld (of K, or of V) covers rows ld * kRowsPerLoad .. + kRowsPerLoad
    // - 1, lane l writing the 16 bytes at l * 16 of the load's 1 KB of LDS.
    // The chunk swizzles repeat every four loads, so load 4 g + j is the
    // offset of load j plus g groups of rows; only the row base changes
    // between units.
    static_assert(C::kLoadsKV % 4 == 0, "loads come in groups of four");
    const uint32_t grp_bytes = (uint32_t)(4 * C::kRowsPerLoad * row_bytes);
    uint32_t koff[4], voff[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int r = j * C::kRowsPerLoad + lane / CH;
      koff[j] = (uint32_t)(r * row_bytes + ((lane % CH) ^ k_swizzle<D>(r)) * 16);
      voff[j] = (uint32_t)(r * row_bytes + ((lane % CH) ^ (kDq ? k_swizzle<D>(r) : v_swizzle<D>(r))) * 16);
    }
    constexpr int kOwn = R / kProducers;    // ring slots each loader owns
    int tgt[kOwn];                          // participant releases owed to each own slot
#pragma unroll
    for (int j = 0; j < kOwn; j++) tgt[j] = 0;
    // The K rows go straight from memory to LDS as soon as the slot's K
    // half is free (its readers have formed S^T), so their latency overlaps
    // the earlier occupant's softmax and PV; the V rows follow once the K
    // rows have landed and the V half is free.
    // the item holding the next unit to locate: its first stream index, units, kv head
    int it_v0 = 0;
    int it_n = cs.valid ? cs.hd.nunion * nsb : 0;
    int it_h = cs.valid ? __builtin_amdgcn_readfirstlane(cs.item / a.n_tiles / a.gpk) : 0;
    // Find own unit v and read its word: participants and the byte offset of
    // its first row (kv head included).  False once the stream is over.
    auto locate = [&](int v, int& np, int64_t& rb) -> bool {
      while (cs.valid && v - it_v0 >= it_n) {
        it_v0 += it_n;
        next_item(cs, a);
        it_n = cs.valid ? cs.hd.nunion * nsb : 0;
        it_h = cs.valid ? __builtin_amdgcn_readfirstlane(cs.item / a.n_tiles / a.gpk) : 0;
      }
      if (!cs.valid) return false;
      const int uu = v - it_v0;
      const uint32_t word = ld_const(a.units, (int64_t)cs.item * a.umax_units + uu);
      np = (word >> 31) != 0u ? (int)((word >> 24) & 15u) : 0;
      const int kstart = (int)(word & 0xFFFFFFu) * a.bs + (uu & (nsb - 1)) * KB;   // nsb is 1 or 2
      const int row0 = cs.hd.tok0 - cs.hd.pos0 + kstart;
      rb = ((int64_t)row0 * a.Hkv + it_h) * (D * 2);
      return true;
    };
    // Buffer loads of a unit: each group of four loads gets a scalar resource
    // based at its own first row whose record count ends at the tensor's
    // end, so the rows of a unit that runs past the last row read as zero
    // (they are masked by causality); the lane offsets stay the four koff /
    // voff values.
    const int64_t kv_bytes = (int64_t)a.Ttot * a.Hkv * (D * 2);
    auto issue_k = [&](int64_t rb, NSA_LDS char* kdst) {
      [&]<int... LI>(std::integer_sequence<int, LI...>) {
        (__builtin_amdgcn_raw_ptr_buffer_load_lds(group_rsrc(K, rb + (int64_t)(LI / 4) * grp_bytes, kv_bytes),
                                                  (NSA_LDS void*)(kdst + LI * 1024), 16, koff[LI % 4], 0, 0, 0),
         ...);
      }(std::make_integer_sequence<int, C::kLoadsKV>{});
    };
    auto issue_v = [&](int64_t rb, NSA_LDS char* vdst) {
      [&]<int... LI>(std::integer_sequence<int, LI...>) {
        (__builtin_amdgcn_raw_ptr_buffer_load_lds(group_rsrc(V, rb + (int64_t)(LI / 4) * grp_bytes, kv_bytes),
                                                  (NSA_LDS void*)(vdst + LI * 1024), 16, voff[LI % 4], 0, 0, 0),
         ...);
      }(std::make_integer_sequence<int, C::kLoadsKV>{});
    };
    // Bounded wait until the release counter reaches t; false if it expired.
    auto wait_free = [&](int* ctr, int t) -> bool {
      int spins = 0;
      while (loader_poll(ctr) < t) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kMaxSpin) return false;
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      return true;
    };
    // Each pass places own unit v_cur: K loads into the slot, the next
    // unit's word, K landed -> publish K, V half free -> V loads into the
    // slot, V landed -> publish V.
    int v_cur = p;
    int np = 0;               // participants of v_cur
    int64_t rb = 0;           // byte offset of v_cur's first row
    bool have = locate(v_cur, np, rb);
    bool stuck = false;
    while (have) {
      const int slot = v_cur % R;
      const int js = (v_cur / kProducers) % kOwn;   // which of this loader's slots
      int t = 0;
#pragma unroll
      for (int j = 0; j < kOwn; j++) t = (j == js) ? tgt[j] : t;
      NSA_LDS char* kdst = (NSA_LDS char*)&ring[slot][0];
      // debug mode: unit v_cur enters the ring only once every earlier unit
      // of the workgroup has been read by all its readers
      if (a.serial && !wait_free(&serial_done, v_cur)) {
        stuck = true;
        break;
      }
      if (np > 0) {
        // With split releases the K half may be refilled once the readers of
        // the slot's earlier occupants have formed S^T; otherwise the whole
        // slot waits for their V reads.
        if (!wait_free(a.split_release ? &done_k[slot] : &done[slot], t)) {
          stuck = true;
          break;
        }
        issue_k(rb, kdst);
      }
      int np_n = 0;
      int64_t rb_n = 0;
      const bool have_n = locate(v_cur + kProducers, np_n, rb_n);
      if (np > 0) {
        wait_vmcnt<0>();   // the K rows have landed
        loader_bump(&ready2[slot][0]);
        if (a.split_release && !wait_free(&done[slot], t)) {
          stuck = true;
          break;
        }
        issue_v(rb, kdst + KB * D * 2);
        wait_vmcnt<0>();   // the V rows have landed
        loader_bump(&ready2[slot][1]);
#pragma unroll
        for (int j = 0; j < kOwn; j++) tgt[j] += (j == js) ? np : 0;
        if (a.serial) {
          if (!wait_free(&done[slot], t + np)) {
            stuck = true;
            break;
          }
          loader_bump(&serial_done);
        }
      } else {
        loader_bump(&ready2[slot][0]);   // no attention wave reads this unit: nothing to load
        loader_bump(&ready2[slot][1]);
        if (a.serial) loader_bump(&serial_done);
      }
      v_cur += kProducers;
      np = np_n;
      rb = rb_n;
      have = have_n;
    }
    if (stuck) atomicOr(a.err, kErrStuck);
    return;
  }

  // ------------------------------------------------------------ attention
  const int c = lane & 15;
  const int g = lane >> 4;
  const int tpw = a.tpw;
  const int tok_first = wave * tpw;   // this wave's first token inside an item
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q);
  __bf16* __restrict__ Out = reinterpret_cast<__bf16*>(a.out);
  int v_base = 0;
  bool stuck = false;
  while (cs.valid && !stuck) {
    const int item = cs.item;
    const ItemHeader hd = cs.hd;
    const int vg = item / a.n_tiles;
    const int my_ntok = min(max(hd.ntok - tok_first, 0), tpw);
    const int my_tmin = hd.pos0 + tok_first;
    const int my_tmax = my_tmin + my_ntok - 1;
    const int nunits = hd.nunion * nsb;

    int tau[NTPW], hq[NTPW], tcol[NTPW];
    uint32_t tvalid[NTPW];
    bool cvalid[NTPW];
    bf16x8 qf[NTPW][KT];
    f32x4 o[NTPW][DT];
    float mrun[NTPW], lrun[NTPW];
    bf16x8 dof[NTPW][KT];       // gradient mode: dO^T fragments, like qf
    float lse2[NTPW], dlt[NTPW];   // gradient mode: per column lse log2e and Delta
#pragma unroll
    for (int n = 0; n < NTPW; n++) {
      int head;
      column_of(c, a.gv, a.tpt, tok_first + n * a.tpt, hd.ntok, tau[n], head, cvalid[n]);
      hq[n] = vg * a.gv + head;
      tcol[n] = hd.pos0 + tau[n];
      {
        // tokens of tile n (bits relative to tok_first) that exist
        const int t0 = n * a.tpt;
        const int nv = min(max(my_ntok - t0, 0), a.tpt);
        tvalid[n] = nv >= 32 ? 0xFFFFFFFFu : (((1u << nv) - 1u) << t0);
      }
      const int64_t qrow = ((int64_t)(hd.tok0 + (cvalid[n] ? tau[n] : 0)) * a.Hq + hq[n]) * D;
#pragma unroll
      for (int kk = 0; kk < KT; kk++) {
        if (cvalid[n])
          qf[n][kk] = *reinterpret_cast<const bf16x8*>(Q + qrow + kk * 32 + g * 8);
        else
          qf[n][kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int dt = 0; dt < DT; dt++) o[n][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      mrun[n] = -INFINITY;
      lrun[n] = 0.f;
      if constexpr (kDq) {
        // dO^T fragments; Delta = dO . O of the column (each lane holds 32
        // of its D products, the four lane groups are summed); the lse in
        // the log2 domain (0 where the row saw no key: its scores are all
        // masked, so every P of it is 0)
        const __bf16* __restrict__ dO = reinterpret_cast<const __bf16*>(a.dout);
        const __bf16* __restrict__ Ofw = reinterpret_cast<const __bf16*>(a.fwd_out);
        float part = 0.f;
#pragma unroll
        for (int kk = 0; kk < KT; kk++) {
          if (cvalid[n]) {
            dof[n][kk] = *reinterpret_cast<const bf16x8*>(dO + qrow + kk * 32 + g * 8);
            const bf16x8 ov = *reinterpret_cast<const bf16x8*>(Ofw + qrow + kk * 32 + g * 8);
#pragma unroll
            for (int e = 0; e < 8; e++) part = __builtin_fmaf((float)dof[n][kk][e], (float)ov[e], part);
          } else {
            dof[n][kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
          }
        }
        dlt[n] = sum_over_groups(part);
        const int64_t lrow = (int64_t)(hd.tok0 + (cvalid[n] ? tau[n] : 0)) * a.Hq + hq[n];
        const float lv = cvalid[n] ? a.lse_in[lrow] : 0.f;
        lse2[n] = (lv == -INFINITY || lv != lv) ? 0.f : lv * 1.4426950408889634f;
        if (cvalid[n] && g == 0) a.delta[lrow] = dlt[n];
      }
    }

    // find this wave's units 64 at a time: lane i examines unit cbase + i
    for (int cbase = 0; cbase < nunits && my_ntok > 0 && !stuck; cbase += 64) {
      const int uu = cbase + lane;
      int lj = -1;
      uint32_t lbits = 0u;
      bool part = false;
      if (uu < nunits) {
        const int u = uu >> (nsb - 1);   // nsb is 1 or 2
        const int sb = uu & (nsb - 1);
        // the unit word and the entry's token bits load side by side (both
        // inside the item's tables), so a new item waits one memory latency
        const uint32_t word = a.units[(int64_t)item * a.umax_units + uu];
        const uint32_t mk = a.masks[((int64_t)item * a.umax + u) * a.mw + (tok_first >> 5)];
        lj = (int)(word & 0xFFFFFFu);
        const int ks = lj * a.bs + sb * KB;
        if ((word >> 31) != 0u && ks <= my_tmax) {
          lbits = mask_field(mk, tok_first, tpw);
          part = lbits != 0u;
        }
      }
      uint64_t todo = __ballot(part);
      while (todo != 0ull && !stuck) {
        const int b = __builtin_ctzll(todo);
        todo &= todo - 1ull;
        const int uu_b = cbase + b;
        const int j = __builtin_amdgcn_readlane(lj, b);
        const uint32_t mine = (uint32_t)__builtin_amdgcn_readlane((int)lbits, b);
        const int kstart = j * a.bs + (uu_b & (nsb - 1)) * KB;   // nsb is 1 or 2
        const int v = v_base + uu_b;
        const int slot = v % R;
        const int need = v / R + 1;
        int spins = 0;
        uint64_t rw = lds_poll2(&ready2[slot][0]);
        while ((int)(uint32_t)rw < need) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kMaxSpin) {
            stuck = true;
            break;
          }
          rw = lds_poll2(&ready2[slot][0]);
        }
        // the V rows may already be published with the K rows' counter
        const bool v_ready = (int)(uint32_t)(rw >> 32) >= need;
        if (stuck) break;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const bool diag = (kstart + KB - 1) > my_tmin;
        NSA_LDS const char* kl = (NSA_LDS const char*)&ring[slot][0];
        NSA_LDS const char* vl = kl + KB * D * 2;
        constexpr int n = 0;   // one 16-column tile per attention wave
        const uint32_t tbits = mine;
        const bool sel = cvalid[n] && ((mine >> (tau[n] - tok_first)) & 1u);
        if constexpr (kDq) {
          // rows of K (then of V) one 16-key tile at a time: A operands
          auto read_rows = [&](NSA_LDS const char* base, bf16x8 (&kf)[KT], int mt) {
            const int row = mt * 16 + c;
#pragma unroll
            for (int kk = 0; kk < KT; kk++) {
              const int pc = (kk * 4 + g) ^ k_swizzle<D>(row);
              kf[kk] = *(NSA_LDS const bf16x8*)(base + row * (D * 2) + pc * 16);
            }
          };
          f32x4 s[MT];
#pragma unroll
          for (int mt = 0; mt < MT; mt++) {
            bf16x8 kf[KT];
            read_rows(kl, kf, mt);
            s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KT; kk++) s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[n][kk], s[mt], 0, 0, 0);
          }
          // P = 2^(scale log2e s - lse log2e), 0 where masked
          const bool need_mask = diag || (tbits != tvalid[n]);
          const int lim = sel ? tcol[n] - kstart - g * 4 : -1;
          const float sc = a.scale_log2;
#pragma unroll
          for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
              const bool vis = !need_mask || (mt * 16 + jj <= lim);
              s[mt][jj] = vis ? fast_exp2(__builtin_fmaf(s[mt][jj], sc, -lse2[n])) : 0.f;
            }
          // the V rows
          spins = 0;
          while (!v_ready && lds_poll(&ready2[slot][1]) < need) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kMaxSpin) {
              stuck = true;
              break;
            }
          }
          if (stuck) break;
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          // dP^T = V dO^T one 16-key tile at a time, then dS = P (dP - Delta)
          // as the bf16 B operand of dQ^T += K^T dS^T
          bf16x8 dsf[KQ];
#pragma unroll
          for (int mt = 0; mt < MT; mt++) {
            bf16x8 vf[KT];
            read_rows(vl, vf, mt);
            f32x4 dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KT; kk++) dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[kk], dof[n][kk], dp, 0, 0, 0);
#pragma unroll
            for (int jj = 0; jj < 4; jj++) dsf[mt >> 1][(mt & 1) * 4 + jj] = (__bf16)(s[mt][jj] * (dp[jj] - dlt[n]));
          }
          // dQ^T += K^T dS^T: K read transposed, one 16-row tile of dQ^T at a
          // time, the reads of the next tile issued before the MFMAs of this one
          auto read_kt = [&](bf16x8 (&kt)[KQ], int dt) {
#pragma unroll
            for (int kq = 0; kq < KQ; kq++)
#pragma unroll
              for (int half = 0; half < 2; half++) {
                const int key = kq * 32 + half * 16 + g * 4 + (c >> 2);
                const int d0 = dt * 16 + (c & 3) * 4;
                const int pc = (d0 >> 3) ^ k_swizzle<D>(key);
                const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (NSA_LDS s16x4*)(kl + key * (D * 2) + pc * 16 + (d0 & 7) * 2));
                const bf16x4 tb = __builtin_bit_cast(bf16x4, t);
#pragma unroll
                for (int e = 0; e < 4; e++) kt[kq][half * 4 + e] = tb[e];
              }
          };
          auto mm = [&](const bf16x8 (&kt)[KQ], int dt) {
#pragma unroll
            for (int kq = 0; kq < KQ; kq++)
              o[n][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt[kq], dsf[kq], o[n][dt], 0, 0, 0);
          };
          {
            bf16x8 ka[KQ], kb[KQ];
            read_kt(ka, 0);
#pragma unroll
            for (int dt = 0; dt < DT; dt += 2) {
              read_kt(kb, dt + 1);
              mm(ka, dt);
              if (dt + 2 < DT) read_kt(ka, dt + 2);
              else lds_release_bump(&done[slot]);   // the last reads of the slot have returned
              mm(kb, dt + 1);
            }
          }
          continue;
        }
        // S^T = K Q^T; K fragments read from the slot half a unit at a time
        // (one LDS round trip per half), then the MFMAs
        f32x4 s[MT];
#pragma unroll
        for (int mt = 0; mt < MT; mt++) s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // one 16-key row tile of K at a time, two in flight: the reads of
        // tile mt + 2 are issued before the MFMAs of tile mt + 1
        auto read_k = [&](bf16x8 (&kf)[KT], int mt) {
          const int row = mt * 16 + c;
#pragma unroll
          for (int kk = 0; kk < KT; kk++) {
            const int pc = (kk * 4 + g) ^ k_swizzle<D>(row);
            kf[kk] = *(NSA_LDS const bf16x8*)(kl + row * (D * 2) + pc * 16);
          }
        };
        auto qk = [&](const bf16x8 (&kf)[KT], int mt) {
#pragma unroll
          for (int kk = 0; kk < KT; kk++)
            s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kk], qf[n][kk], s[mt], 0, 0, 0);
        };
        {
          static_assert(MT == 2 || MT == 4, "units of 32 or 64 keys");
          bf16x8 ka[KT], kb[KT];
          read_k(ka, 0);
          read_k(kb, 1);
          qk(ka, 0);
          if constexpr (MT == 4) read_k(ka, 2);
          qk(kb, 1);
          if constexpr (MT == 4) {
            read_k(kb, 3);
            qk(ka, 2);
            qk(kb, 3);
          }
        }
        if (a.split_release) lds_release_bump(&done_k[slot]);   // the K reads have returned
        // V^T fragments, a quarter of the row tiles at a time (lane (c, g)
        // reads keys 4g + c/4 of each 16-key half, columns 4 (c % 4) .. + 3)
        constexpr int DQ = DT / 4;
        auto read_v = [&](bf16x8 (&vf)[DQ][KQ], int qb) {
#pragma unroll
          for (int dd = 0; dd < DQ; dd++) {
            const int dt = qb * DQ + dd;
#pragma unroll
            for (int kq = 0; kq < KQ; kq++) {
#pragma unroll
              for (int half = 0; half < 2; half++) {
                const int key = kq * 32 + half * 16 + g * 4 + (c >> 2);
                const int d0 = dt * 16 + (c & 3) * 4;
                const int pc = (d0 >> 3) ^ v_swizzle<D>(key);
                const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (NSA_LDS s16x4*)(vl + key * (D * 2) + pc * 16 + (d0 & 7) * 2));
                const bf16x4 tb = __builtin_bit_cast(bf16x4, t);
#pragma unroll
                for (int e = 0; e < 4; e++) vf[dd][kq][half * 4 + e] = tb[e];
              }
            }
          }
        };
        // mask (only where some column of the tile must not see some key),
        // online softmax in the log2 domain.  Lane (c, g) holds keys
        // 16*mt + 4*g + jj of column c.
        const bool need_mask = diag || (tbits != tvalid[n]);
        if (need_mask) {
          // key kstart + 16 mt + 4 g + jj is visible iff 16 mt + jj <= lim
          const int lim = sel ? tcol[n] - kstart - g * 4 : -1;
#pragma unroll
          for (int mt = 0; mt < MT; mt++) {
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
              if (mt * 16 + jj > lim) s[mt][jj] = -INFINITY;
            }
          }
        }
        float mx = -INFINITY;
        const float sc = a.scale_log2;
        if constexpr (kPosScale) {
          // a v_max3 tree over the lane's 4 MT scores
          float m3[MT];
#pragma unroll
          for (int mt = 0; mt < MT; mt++) m3[mt] = max3_raw(s[mt][0], s[mt][1], max_raw(s[mt][2], s[mt][3]));
          if constexpr (MT == 4) {
            mx = max3_raw(m3[0], m3[1], max_raw(m3[2], m3[3]));
          } else {
            mx = max_raw(m3[0], m3[1]);
          }
          mx = max_over_groups(mx) * sc;
        } else {
#pragma unroll
          for (int mt = 0; mt < MT; mt++) {
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
              s[mt][jj] = s[mt][jj] == -INFINITY ? -INFINITY : s[mt][jj] * sc;
              mx = fmaxf(mx, s[mt][jj]);
            }
          }
          mx = max_over_groups(mx);
        }
        // The running max moves only when a score exceeds it by more than
        // 2^8: p = 2^(x - m) then stays <= 256, exact enough in fp32 and
        // bf16, and the O rescale is skipped on most units.
        const bool raise = mx > mrun[n] + 8.f;
        const float mnew = raise ? mx : mrun[n];
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        // four partial sums (a short dependency chain), each starting at its
        // first term rather than at zero (0 + p costs an add)
        float rsum[4];
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            const float pv = kPosScale ? fast_exp2(__builtin_fmaf(s[mt][jj], sc, -muse))
                                       : fast_exp2(s[mt][jj] - muse);
            s[mt][jj] = pv;
            rsum[jj] = mt == 0 ? pv : rsum[jj] + pv;
          }
        }
        float rs = (rsum[0] + rsum[1]) + (rsum[2] + rsum[3]);
        rs = sum_over_groups(rs);
        if (__ballot(raise) != 0ull) {
          const float alpha = raise ? fast_exp2(mrun[n] - muse) : 1.f;
          lrun[n] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; dt++) o[n][dt] *= alpha;
        }
        lrun[n] += rs;
        mrun[n] = mnew;
        bf16x8 pf[KQ];
#pragma unroll
        for (int kq = 0; kq < KQ; kq++) {
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            pf[kq][jj] = (__bf16)s[2 * kq][jj];
            pf[kq][4 + jj] = (__bf16)s[2 * kq + 1][jj];
          }
        }
        // O^T += V^T P^T, one quarter of the row tiles at a time; the reads
        // of the next quarter are issued before the MFMAs of the current one,
        // and the slot is released as soon as the last reads have returned
        auto pv = [&](bf16x8 (&vf)[DQ][KQ], int qb) {
#pragma unroll
          for (int dd = 0; dd < DQ; dd++) {
#pragma unroll
            for (int kq = 0; kq < KQ; kq++)
              o[n][qb * DQ + dd] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dd][kq], pf[kq], o[n][qb * DQ + dd], 0, 0, 0);
          }
        };
        // the V rows of the unit may land after its K rows (they were issued
        // after them): wait for them only now, after the softmax
        spins = 0;
        while (!v_ready && lds_poll(&ready2[slot][1]) < need) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > kMaxSpin) {
            stuck = true;
            break;
          }
        }
        if (stuck) break;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        bf16x8 va[DQ][KQ], vb[DQ][KQ];
        read_v(va, 0);
        read_v(vb, 1);
        pv(va, 0);
        read_v(va, 2);
        pv(vb, 1);
        read_v(vb, 3);
        lds_release_bump(&done[slot]);
        pv(va, 2);
        pv(vb, 3);
      }
      if constexpr (kDq) {
        // the reader bitmap of the dk/dv kernel: this wave's tokens that keep
        // the lane's block (first sub-block; the first head group of the kv
        // head writes it), one atomic OR per lane for the chunk
        if (part && (uu & (nsb - 1)) == 0 && vg % a.gpk == 0) {
          const int tt = my_tmin;   // position of the wave's first token
          const int64_t rbase = ((int64_t)((hd.tok0 - hd.pos0) / a.T) * a.Hkv + vg / a.gpk) * a.rd_nb + lj;
          const uint32_t live = lbits & ((1u << my_ntok) - 1u);   // my_ntok <= 16
          const uint64_t bits = (uint64_t)live << (tt & 31);
          atomicOr(&a.readers[rbase * a.rd_nw + (tt >> 5)], (uint32_t)bits);
          if ((uint32_t)(bits >> 32) != 0u) atomicOr(&a.readers[rbase * a.rd_nw + (tt >> 5) + 1], (uint32_t)(bits >> 32));
        }
      }
    }
    if (stuck) break;

    if constexpr (kDq) {
      // dq = scale dQ^T, fp32 rows
#pragma unroll
      for (int n = 0; n < NTPW; n++) {
        if (!cvalid[n]) continue;
        const int64_t orow = ((int64_t)(hd.tok0 + tau[n]) * a.Hq + hq[n]) * D;
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
          *reinterpret_cast<f32x4*>(a.dq + orow + dt * 16 + g * 4) = o[n][dt] * a.scale;
      }
      v_base += nunits;
      next_item(cs, a);
      continue;
    }
    // epilogue: out = O / l (bf16, round to nearest even), lse = ln 2 * (m + log2 l)
#pragma unroll
    for (int n = 0; n < NTPW; n++) {
      if (!cvalid[n]) continue;
      const float l = lrun[n];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int64_t orow = ((int64_t)(hd.tok0 + tau[n]) * a.Hq + hq[n]) * D;
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
        bf16x4 ov;
#pragma unroll
        for (int jj = 0; jj < 4; jj++) ov[jj] = (__bf16)(o[n][dt][jj] * inv);
        *reinterpret_cast<bf16x4*>(Out + orow + dt * 16 + g * 4) = ov;
      }
      if (a.lse && g == 0) {
        const float lv = l > 0.f ? (mrun[n] + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
        a.lse[(int64_t)(hd.tok0 + tau[n]) * a.Hq + hq[n]] = lv;
      }
    }
    v_base += nunits;
    next_item(cs, a);
  }
  if (stuck) atomicOr(a.err, kErrStuck);
}

// ---------------------------------------------------------------------------
// fp32: one wave per (item, token group of `tpw` tokens), no LDS
// ---------------------------------------------------------------------------
template <int D, int KB, int NTPW>
__global__ void __launch_bounds__(256, 2) fwd_f32_kernel(FwdArgs a) {
  constexpr int KT = D / 4;
  constexpr int MT = KB / 16;
  constexpr int DT = D / 16;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);   // global wave id
  const int pos = gw / kConsumers;
  const int part = gw % kConsumers;
  if (pos >= a.n_items) return;
  const int item = a.worklist[pos];
  if (item < 0 || item >= a.n_items) return;
  ItemHeader hd = a.hdr[item];
  if (!header_ok(hd, a)) return;
  const int vg = item / a.n_tiles;
  const int h = vg / a.gpk;
  const int tpw = a.tpw;
  const int tok_first = part * tpw;
  const int my_ntok = min(max(hd.ntok - tok_first, 0), tpw);
  if (my_ntok == 0) return;
  const int my_tmin = hd.pos0 + tok_first;
  const int my_tmax = my_tmin + my_ntok - 1;
  const int bos = hd.tok0 - hd.pos0;
  const float* __restrict__ Q = reinterpret_cast<const float*>(a.q);
  const float* __restrict__ K = reinterpret_cast<const float*>(a.k);
  const float* __restrict__ V = reinterpret_cast<const float*>(a.v);

  int tau[NTPW], hq[NTPW], tcol[NTPW];
  bool cvalid[NTPW];
  float qf[NTPW][KT];
  f32x4 o[NTPW][DT];
  float mrun[NTPW], lrun[NTPW];
#pragma unroll
  for (int n = 0; n < NTPW; n++) {
    int head;
    column_of(c, a.gv, a.tpt, tok_first + n * a.tpt, hd.ntok, tau[n], head, cvalid[n]);
    hq[n] = vg * a.gv + head;
    tcol[n] = hd.pos0 + tau[n];
    const int64_t qrow = ((int64_t)(hd.tok0 + (cvalid[n] ? tau[n] : 0)) * a.Hq + hq[n]) * D;
#pragma unroll
    for (int kk = 0; kk < KT; kk++) qf[n][kk] = cvalid[n] ? Q[qrow + kk * 4 + g] : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) o[n][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mrun[n] = -INFINITY;
    lrun[n] = 0.f;
  }
  for (int u = 0; u < hd.nunion; u++) {
    const int j = a.blocks[(int64_t)item * a.umax + u];
    if (j < 0 || j > my_tmax / a.bs) continue;
    const uint32_t mk = a.masks[((int64_t)item * a.umax + u) * a.mw + (tok_first >> 5)];
    const uint32_t mine = mask_field(mk, tok_first, tpw);
    if (mine == 0u) continue;
    for (int sb = 0; sb < a.bs / KB; sb++) {
      const int kstart = j * a.bs + sb * KB;
      if (kstart > my_tmax) break;
      const bool diag = (kstart + KB - 1) > my_tmin;
      const int row0 = bos + kstart;
#pragma unroll
      for (int n = 0; n < NTPW; n++) {
        const uint32_t tbits = (mine >> (n * a.tpt)) & ((1u << a.tpt) - 1u);
        if (tbits == 0u) continue;
        const bool sel = cvalid[n] && ((mine >> (tau[n] - tok_first)) & 1u);
        f32x4 s[MT];
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
          int grow = row0 + mt * 16 + c;
          grow = grow < a.Ttot ? grow : a.Ttot - 1;
          const float* kp = K + ((int64_t)grow * a.Hkv + h) * D + g;
          s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KT; kk++)
            s[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kp[kk * 4], qf[n][kk], s[mt], 0, 0, 0);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            float x = s[mt][jj] * a.scale_log2;
            const int kp = kstart + mt * 16 + g * 4 + jj;
            if (!sel || (diag && kp > tcol[n])) x = -INFINITY;
            s[mt][jj] = x;
            mx = fmaxf(mx, x);
          }
        }
        mx = max_over_groups(mx);
        const float mnew = fmaxf(mrun[n], mx);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(mrun[n] - muse);
        float rs = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            const float pv = fast_exp2(s[mt][jj] - muse);
            s[mt][jj] = pv;
            rs += pv;
          }
        }
        rs = sum_over_groups(rs);
        lrun[n] = lrun[n] * alpha + rs;
        mrun[n] = mnew;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
          f32x4 acc = o[n][dt] * alpha;
#pragma unroll
          for (int mt = 0; mt < MT; mt++) {
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
              int grow = row0 + mt * 16 + g * 4 + jj;
              grow = grow < a.Ttot ? grow : a.Ttot - 1;
              const float vv = V[((int64_t)grow * a.Hkv + h) * D + dt * 16 + c];
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, s[mt][jj], acc, 0, 0, 0);
            }
          }
          o[n][dt] = acc;
        }
      }
    }
  }
  float* __restrict__ Out = reinterpret_cast<float*>(a.out);
#pragma unroll
  for (int n = 0; n < NTPW; n++) {
    if (!cvalid[n]) continue;
    const float l = lrun[n];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t orow = ((int64_t)(hd.tok0 + tau[n]) * a.Hq + hq[n]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      const f32x4 ov = o[n][dt] * inv;
      *reinterpret_cast<f32x4*>(Out + orow + dt * 16 + g * 4) = ov;
    }
    if (a.lse && g == 0) {
      const float lv = l > 0.f ? (mrun[n] + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
      a.lse[(int64_t)(hd.tok0 + tau[n]) * a.Hq + hq[n]] = lv;
    }
  }
}

// NSA_DEBUG=1 (read at every launch): the ring holds one unit at a time, so
// no load overlaps any read of another unit; results must equal the
// overlapped ring's bit for bit.
bool debug_serial() {
  const char* e = getenv("NSA_DEBUG");
  return e && e[0] && e[0] != '0';
}

typedef void (*KernelFn)(FwdArgs);

template <int D, int KB>
KernelFn pick_ntpw(bool bf16, int ntpw, bool pos_scale) {
  if (bf16) {
    if (ntpw == 1)
      return pos_scale ? fwd_bf16_ring_kernel<D, KB, 1, true, false> : fwd_bf16_ring_kernel<D, KB, 1, false, false>;
  } else {
    switch (ntpw) {
      case 1: return fwd_f32_kernel<D, KB, 1>;
      case 2: return fwd_f32_kernel<D, KB, 2>;
    }
  }
  return nullptr;
}

KernelFn pick(bool bf16, int D, int KB, int ntpw, bool pos_scale) {
  if (D == 64) return KB == 32 ? pick_ntpw<64, 32>(bf16, ntpw, pos_scale) : pick_ntpw<64, 64>(bf16, ntpw, pos_scale);
  if (D == 128)
    return KB == 32 ? pick_ntpw<128, 32>(bf16, ntpw, pos_scale) : pick_ntpw<128, 64>(bf16, ntpw, pos_scale);
  return nullptr;
}

}  // namespace

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

hipError_t launch_fwd(const Plan& p, const void* q, const void* k, const void* v, float scale,
                      void* out, float* lse, char* ws, hipStream_t stream) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.hdr = reinterpret_cast<const ItemHeader*>(ws + p.off_hdr);
  a.blocks = reinterpret_cast<const int32_t*>(ws + p.off_blocks);
  a.masks = reinterpret_cast<const uint32_t*>(ws + p.off_masks);
  a.tq = p.tq;
  a.mw = p.mw;
  a.units = reinterpret_cast<const uint32_t*>(ws + p.off_units);
  a.umax_units = p.umax_units;
  a.worklist = reinterpret_cast<const int32_t*>(ws + p.off_worklist);
  a.err = reinterpret_cast<int32_t*>(ws + p.off_err);
  a.Ttot = p.B * p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.gv = p.gv;
  a.gpk = p.gpk;
  a.tpt = p.tpt;
  a.tpw = p.tpw;
  a.n_tiles = p.n_tiles;
  a.n_items = p.n_items;
  a.umax = p.umax;
  a.bs = p.bs;
  a.nwg = p.nwg;
  a.scale_log2 = scale * 1.4426950408889634f;
  // Split releases pay where a unit has few readers (one token per wave);
  // with many readers per unit the second release atomic costs more.
  a.split_release = p.tpw == 1 ? 1 : 0;
  a.serial = debug_serial() ? 1 : 0;
  KernelFn fn = pick(p.bf16, p.D, p.kb, p.ntpw, a.scale_log2 > 0.f);
  if (!fn) return hipErrorInvalidValue;
  if (p.bf16) {
    hipLaunchKernelGGL(fn, dim3(p.nwg), dim3(64 * (kConsumers + kProducers)), 0, stream, a);
  } else {
    const int waves = p.n_items * kConsumers;
    hipLaunchKernelGGL(fn, dim3((waves + 3) / 4), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_dq_ring(const Plan& p, const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, float scale, float* dq, float* delta,
                          uint32_t* readers, int32_t rd_nb, int32_t rd_nw, char* ws, hipStream_t stream) {
  if (!p.bf16 || p.ntpw != 1) return hipErrorInvalidValue;
  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = nullptr;
  a.lse = nullptr;
  a.hdr = reinterpret_cast<const ItemHeader*>(ws + p.off_hdr);
  a.blocks = reinterpret_cast<const int32_t*>(ws + p.off_blocks);
  a.masks = reinterpret_cast<const uint32_t*>(ws + p.off_masks);
  a.units = reinterpret_cast<const uint32_t*>(ws + p.off_units);
  a.worklist = reinterpret_cast<const int32_t*>(ws + p.off_worklist);
  a.err = reinterpret_cast<int32_t*>(ws + p.off_err);
  a.Ttot = p.B * p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.gv = p.gv;
  a.gpk = p.gpk;
  a.tpt = p.tpt;
  a.tpw = p.tpw;
  a.tq = p.tq;
  a.mw = p.mw;
  a.n_tiles = p.n_tiles;
  a.n_items = p.n_items;
  a.umax = p.umax;
  a.umax_units = p.umax_units;
  a.bs = p.bs;
  a.nwg = p.nwg;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.split_release = 0;   // K is read again for dQ: one release per slot
  a.serial = debug_serial() ? 1 : 0;
  a.dout = dout;
  a.fwd_out = out;
  a.lse_in = lse;
  a.dq = dq;
  a.delta = delta;
  a.readers = readers;
  a.rd_nb = rd_nb;
  a.rd_nw = rd_nw;
  a.T = p.T;
  a.scale = scale;
  KernelFn fn = nullptr;
  if (p.D == 64) fn = p.kb == 32 ? fwd_bf16_ring_kernel<64, 32, 1, true, true> : fwd_bf16_ring_kernel<64, 64, 1, true, true>;
  if (p.D == 128)
    fn = p.kb == 32 ? fwd_bf16_ring_kernel<128, 32, 1, true, true> : fwd_bf16_ring_kernel<128, 64, 1, true, true>;
  if (!fn) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3(p.nwg), dim3(64 * (kConsumers + kProducers)), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nsa
