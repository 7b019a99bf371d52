// Decode step of the native sparse attention library for gfx950: the
// newest token of each sequence against its KV cache, with the block
// selection of the ejKernel native_sparse_attention API page applied.
#include <utility>

#include "nsa.h"
#include "nsa_internal.h"
#include "nsa_device.h"

namespace nsa {

namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// bf16 decode: one query token per sequence against its KV cache
//
// The query of sequence b sits at position t = len_b - 1 and attends to the
// keys of the blocks listed in its row (same rules as the forward: entries
// past the count, negative or beyond t's own block contribute nothing, a
// repeated block counts once, keys after t inside the own block are masked).
// One workgroup of kDecWaves waves per (sequence, kv head, group of <= 16
// query heads); two workgroups share a CU, so one's index loads overlap the
// other's K/V traffic.  The kept blocks' units (KB = 32 keys, so that a
// unit's K and V registers and the next unit's fit two waves per SIMD) are
// dealt round robin to the waves, and every wave works alone on its units:
//  * K rows are loaded straight into registers in the MFMA A-operand layout
//    (lane (c, g): key row c of a 16-key tile, 16 bytes at d = 32 kk + 8 g);
//  * V rows are loaded into registers row by row, written to the wave's own
//    LDS slot (XOR-swizzled 16-byte chunks) and read back transposed with
//    ds_read_b64_tr_b16 as the A operand of O^T += V^T P^T;
//  * the next unit's K loads are issued as soon as S^T has consumed the K
//    registers and its V loads as soon as the V rows are in LDS, so they
//    travel while the current unit's softmax and PV run.
// Every wait is the compiler's own: there are no cross-wave counters and no
// loads that write LDS directly.  The waves' partial (max, normaliser, O)
// are merged through LDS at the end, as the flash-attention carry is merged
// on the ragged-decode page.
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 4;   // two workgroups per CU (two waves per SIMD), all resident at once

struct DecArgs {
  const void* q;          // [B, Hq, D]
  const void* k;          // [B, Smax, Hkv, D]
  const void* v;
  const int32_t* seq_lens;   // [B]
  const int32_t* bi;         // [B, Hkv, S]
  const int32_t* bc;         // [B, Hkv]
  void* out;              // [B, Hq, D]
  float* lse;             // [B, Hq]
  int32_t B, Smax, Hq, Hkv, S, bs, G, gv, gpk;
  float scale_log2;
};

template <int D, int KB>
__global__ void __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(2)))
decode_bf16_kernel(DecArgs a) {
  constexpr int KT = D / 32;   // k-steps of S^T = K Q^T
  constexpr int MT = KB / 16;  // 16-key row tiles
  constexpr int KQ = KB / 32;  // 32-key k-steps of O^T += V^T P^T
  constexpr int DT = D / 16;   // 16-row tiles of O^T
  constexpr int CH = D / 8;    // 16-byte chunks per row
  constexpr int kHalf = KB * D * 2;            // bytes of the V rows of a unit
  constexpr int kLoads = kHalf / 1024;         // 1 KB row loads of V per unit
  constexpr int kRowsPerLoad = 1024 / (D * 2);
  static_assert(kLoads % 4 == 0 && kLoads <= 16, "loads per unit");
  static_assert(16 * D * 4 <= kHalf, "the merge buffer fits a V slot");
  __shared__ __attribute__((aligned(1024))) char vslot[kDecWaves][kHalf];
  __shared__ float mw_lds[kDecWaves][16];
  __shared__ float lw_lds[kDecWaves][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int g = lane >> 4;
  const int wg = blockIdx.x;
  const int grp = wg % a.gpk;
  const int bh = wg / a.gpk;
  const int h = bh % a.Hkv;
  const int b = bh / a.Hkv;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > a.Smax ? a.Smax : len);
  len = __builtin_amdgcn_readfirstlane(len);
  const int t = len - 1;                       // query position
  const int own = t >= 0 ? t / a.bs : -1;
  const int nsb = a.bs / KB;                   // units per block (1 or 2)

  // kept entries of the row: lane i holds entry i (S <= 64); an entry is
  // dropped if an earlier valid entry lists the same block
  const int64_t row = (int64_t)b * a.Hkv + h;
  // the count and the row are loaded independently (the row lies inside the
  // tensor whatever the count), so the two loads overlap
  int n = a.bc[row];
  const int idx = lane < a.S ? a.bi[row * a.S + lane] : -1;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  n = __builtin_amdgcn_readfirstlane(n);
  bool keep = lane < n && idx >= 0 && idx <= own;
  const uint64_t valid = __ballot(keep);
  for (int j = 0; j < n; j++) {
    if (((valid >> j) & 1ull) == 0ull) continue;
    const int vj = __builtin_amdgcn_readlane(idx, j);
    if (lane > j && idx == vj) keep = false;
  }
  const uint64_t kept = __ballot(keep);
  // this wave's units: lane k holds the first key of its k-th unit
  int my_ks = 0;
  int my_n = 0;
  {
    int u = 0;
    uint64_t m = kept;
    while (m != 0ull) {
      const int j = __builtin_ctzll(m);
      m &= m - 1ull;
      const int blk = __builtin_amdgcn_readlane(idx, j);
      for (int sb = 0; sb < nsb; sb++) {
        const int ks = blk * a.bs + sb * KB;
        if (ks > t) continue;                  // only the own block's tail can start past t
        if (u % kDecWaves == wave) {
          my_ks = (lane == my_n) ? ks : my_ks;
          my_n++;
        }
        u++;
      }
    }
  }

  // Q^T fragments (B operand): lane (c, g) holds q[b, hq = group head c,
  // d = 32 kk + 8 g .. + 7]; columns past the group's heads are zero
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q);
  const int hq = (h * a.gpk + grp) * a.gv + c;
  const bool cvalid = c < a.gv;
  bf16x8 qf[KT];
#pragma unroll
  for (int kk = 0; kk < KT; kk++) {
    if (cvalid)
      qf[kk] = *reinterpret_cast<const bf16x8*>(Q + ((int64_t)b * a.Hq + hq) * D + kk * 32 + g * 8);
    else
      qf[kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }

  // Buffer loads of a unit's rows; each group of four rows-loads (and each
  // 16-key tile of K) gets a scalar resource based at its own first row whose
  // record count ends at the cache's end, so rows past it read as zero (they
  // are masked by causality).
  const char* __restrict__ Kc = reinterpret_cast<const char*>(a.k);
  const char* __restrict__ Vc = reinterpret_cast<const char*>(a.v);
  const int row_bytes = a.Hkv * D * 2;
  const int64_t kv_bytes = (int64_t)a.B * a.Smax * row_bytes;
  const uint32_t vgrp_bytes = (uint32_t)(4 * kRowsPerLoad * row_bytes);
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int r = j * kRowsPerLoad + lane / CH;
    voff[j] = (uint32_t)(r * row_bytes + ((lane % CH) ^ v_swizzle<D>(r)) * 16);
  }
  const uint32_t koff = (uint32_t)(c * row_bytes + g * 16);   // + 64 kk bytes per k-step
  auto unit_base = [&](int ks) -> int64_t { return (((int64_t)b * a.Smax + ks) * a.Hkv + h) * (D * 2); };
  u32x4 kreg[MT * KT];
  u32x4 vreg[kLoads];
  auto load_k = [&](int64_t rb) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const __amdgpu_buffer_rsrc_t rs = group_rsrc(Kc, rb + (int64_t)mt * 16 * row_bytes, kv_bytes);
#pragma unroll
      for (int kk = 0; kk < KT; kk++)
        kreg[mt * KT + kk] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(koff + kk * 64), 0, 0);
    }
  };
  auto load_v = [&](int64_t rb) {
    [&]<int... LI>(std::integer_sequence<int, LI...>) {
      ((vreg[LI] = __builtin_amdgcn_raw_buffer_load_b128(
            group_rsrc(Vc, rb + (int64_t)(LI / 4) * vgrp_bytes, kv_bytes), (int)voff[LI % 4], 0, 0)),
       ...);
    }(std::make_integer_sequence<int, kLoads>{});
  };
  NSA_LDS char* vl = (NSA_LDS char*)&vslot[wave][0];

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;
  const float sc = a.scale_log2;

  // One unit: kMore says whether a next unit follows, whose loads are then
  // issued inside the step.  The last unit is peeled off the loop so that
  // every pass of the loop issues the same loads in the same order (V, then
  // K), which lets the compiler wait for exactly the loads each use needs.
  auto step = [&]<bool kMore>(int i) __attribute__((always_inline)) {
    const int ks = __builtin_amdgcn_readlane(my_ks, i);
    const int64_t rb_n = kMore ? unit_base(__builtin_amdgcn_readlane(my_ks, i + 1)) : 0;
    // V rows into the wave's slot (its previous contents were read by the
    // previous unit's PV, whose reads the compiler has waited for)
    {
      NSA_LDS char* dst = vl + lane * 16;
#pragma unroll
      for (int li = 0; li < kLoads; li++) *(NSA_LDS u32x4*)(dst + li * 1024) = vreg[li];
    }
    if constexpr (kMore) load_v(rb_n);
    // S^T = K Q^T from the K registers
    f32x4 s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KT; kk++)
        s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[mt * KT + kk]), qf[kk],
                                                        s[mt], 0, 0, 0);
    }
    if constexpr (kMore) load_k(rb_n);
    // scale, causal mask inside the own block, online softmax (log2 domain);
    // lane (c, g) holds keys ks + 16 mt + 4 g + jj of column c
    const bool diag = ks + KB - 1 > t;
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        float x = s[mt][jj] * sc;
        if (diag && ks + mt * 16 + g * 4 + jj > t) x = -INFINITY;
        s[mt][jj] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = max_over_groups(mx);
    const float mnew = fmaxf(mrun, mx);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = fast_exp2(mrun - muse);
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
    lrun = lrun * alpha + rs;
    mrun = mnew;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) o[dt] *= alpha;
    bf16x8 pf[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; kq++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        pf[kq][jj] = (__bf16)s[2 * kq][jj];
        pf[kq][4 + jj] = (__bf16)s[2 * kq + 1][jj];
      }
    }
    // O^T += V^T P^T, V^T fragments read transposed from the slot
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
#pragma unroll
      for (int kq = 0; kq < KQ; kq++) {
        bf16x8 vf;
#pragma unroll
        for (int half = 0; half < 2; half++) {
          const int key = kq * 32 + half * 16 + g * 4 + (c >> 2);
          const int d0 = dt * 16 + (c & 3) * 4;
          const int pc = (d0 >> 3) ^ v_swizzle<D>(key);
          const s16x4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (NSA_LDS s16x4*)(vl + key * (D * 2) + pc * 16 + (d0 & 7) * 2));
          const bf16x4 tb = __builtin_bit_cast(bf16x4, tv);
#pragma unroll
          for (int e = 0; e < 4; e++) vf[half * 4 + e] = tb[e];
        }
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[kq], o[dt], 0, 0, 0);
      }
    }
  };
  if (my_n > 0) {
    const int64_t rb0 = unit_base(__builtin_amdgcn_readlane(my_ks, 0));
    load_v(rb0);
    load_k(rb0);
    for (int i = 0; i + 1 < my_n; i++) step.template operator()<true>(i);
    step.template operator()<false>(my_n - 1);
  }

  // merge the waves' partial results through LDS (the V slots hold O)
  __syncthreads();
  // [d tile][lane group][column] float4s: lane (c, g) writes and reads 16
  // consecutive bytes, lanes side by side (no bank conflicts)
  float* ow = reinterpret_cast<float*>(&vslot[wave][0]);
#pragma unroll
  for (int dt = 0; dt < DT; dt++) *reinterpret_cast<f32x4*>(ow + ((dt * 4 + g) * 16 + c) * 4) = o[dt];
  if (g == 0) {
    mw_lds[wave][c] = mrun;
    lw_lds[wave][c] = lrun;
  }
  __syncthreads();
  float mall = -INFINITY;
#pragma unroll
  for (int w = 0; w < kDecWaves; w++) mall = fmaxf(mall, mw_lds[w][c]);
  const float mu = mall == -INFINITY ? 0.f : mall;
  float wgt[kDecWaves];
  float lall = 0.f;
#pragma unroll
  for (int w = 0; w < kDecWaves; w++) {
    wgt[w] = fast_exp2(mw_lds[w][c] - mu);
    lall += lw_lds[w][c] * wgt[w];
  }
  const float inv = lall > 0.f ? 1.f / lall : 0.f;
  __bf16* __restrict__ Out = reinterpret_cast<__bf16*>(a.out);
  // wave w writes the d tiles dt = w (mod kDecWaves) of every column
  for (int dt = wave; dt < DT; dt += kDecWaves) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kDecWaves; w++)
      acc += *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(&vslot[w][0]) +
                                             ((dt * 4 + g) * 16 + c) * 4) * wgt[w];
    bf16x4 ov;
#pragma unroll
    for (int jj = 0; jj < 4; jj++) ov[jj] = (__bf16)(acc[jj] * inv);
    if (cvalid) *reinterpret_cast<bf16x4*>(Out + ((int64_t)b * a.Hq + hq) * D + dt * 16 + g * 4) = ov;
  }
  if (a.lse && wave == 0 && g == 0 && cvalid)
    a.lse[(int64_t)b * a.Hq + hq] = lall > 0.f ? (mall + __log2f(lall)) * 0.69314718055994530942f : -INFINITY;
}

typedef void (*DecFn)(DecArgs);

DecFn pick_decode(int D, int KB) {
  if (KB != 32) return nullptr;
  if (D == 64) return decode_bf16_kernel<64, 32>;
  if (D == 128) return decode_bf16_kernel<128, 32>;
  return nullptr;
}

}  // namespace

hipError_t launch_decode(const DecodePlan& p, const void* q, const void* k, const void* v,
                         const int32_t* seq_lens, const int32_t* block_indices,
                         const int32_t* block_counts, float scale, void* out, float* lse,
                         hipStream_t stream) {
  DecArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.seq_lens = seq_lens;
  a.bi = block_indices;
  a.bc = block_counts;
  a.out = out;
  a.lse = lse;
  a.B = p.B;
  a.Smax = p.Smax;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.S = p.S;
  a.bs = p.bs;
  a.G = p.G;
  a.gv = p.gv;
  a.gpk = p.gpk;
  a.scale_log2 = scale * 1.4426950408889634f;
  // 32-key units: a 64-key unit's K and V registers plus the next unit's
  // would not fit the 256 VGPRs of two waves per SIMD
  DecFn fn = pick_decode(p.D, 32);
  if (!fn) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3(p.B * p.Hkv * p.gpk), dim3(64 * kDecWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nsa
