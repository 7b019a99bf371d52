// Backward pass of the native sparse attention forward for gfx950: the
// gradients dQ, dK, dV of the operation of the ejKernel
// native_sparse_attention API page (module description and "Parameters").
// With P_s = exp(scale q.k_s - lse) over the token's visible keys:
//   Delta = dO . O,   dP_s = dO . v_s,   dS_s = P_s (dP_s - Delta)
//   dQ    = scale sum_s dS_s k_s
//   dK_s  = scale sum_{t, hq} dS_s q,    dV_s = sum_{t, hq} P_s dO
// (the chain rule through the masked softmax; the forward's lse is reused).
//
// dq kernel: one workgroup of kBwdWaves waves per (token, kv head, group of
// <= 16 query heads), the token's kept blocks dealt in 32-key units to the
// waves like the decode kernel: K and V rows go straight into registers as
// the A operands of S^T = K Q^T and dP^T = V dO^T, the K rows are also
// written to the wave's LDS slot and read back transposed (ds_read_b64_tr_b16)
// as the A operand of dQ^T += K^T dS^T.  The waves' partial dQ are summed
// through LDS.  The kernel also writes Delta for the dk/dv kernel.
//
// dkdv kernel: one workgroup per (sequence, kv head, key block), one wave per
// 16-key tile of the block.  The block's readers are found by scanning the
// rows of the tokens at or after the block (a token reads the block iff it
// is among its first clamp(count, 0, S) entries; repeats do not matter for
// membership); for each reader token and head group the wave forms
// S = Q K^T and dP = dO V^T for its 16 keys (K and V rows in registers as
// B operands), P and dS, and accumulates dV += P^T dO and dK += dS^T Q with
// 16x16x16 MFMAs whose B operands (dO and Q, heads x d) are read transposed
// from LDS.  Every key row of every block gets written (zeros where no token
// reads the block).
#include <utility>

#include "nsa.h"
#include "nsa_internal.h"
#include "nsa_device.h"

namespace nsa {

namespace {

using namespace dev;

constexpr int kBwdWaves = 4;

struct BwdArgs {
  const void* q;          // [B, T, Hq, D] bf16
  const void* k;          // [B, T, Hkv, D]
  const void* v;
  const void* out;        // [B, T, Hq, D] forward output
  const float* lse;       // [B, T, Hq]
  const void* dout;       // [B, T, Hq, D]
  const int32_t* bi;      // [B, T, Hkv, S]
  const int32_t* bc;      // [B, T, Hkv]
  float* dq;              // [B, T, Hq, D]
  float* dk;              // [B, T, Hkv, D]
  float* dv;
  float* delta;           // [B, T, Hq] workspace
  int32_t B, T, Hq, Hkv, S, bs, G, gv, gpk, nb;
  float scale;
  float scale_log2;
};

// ---------------------------------------------------------------------------
// dq (and Delta)
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64 * kBwdWaves) __attribute__((amdgpu_waves_per_eu(2)))
bwd_dq_kernel(BwdArgs a) {
  constexpr int KB = 32;
  constexpr int KT = D / 32;
  constexpr int MT = KB / 16;
  constexpr int KQ = KB / 32;
  constexpr int DT = D / 16;
  constexpr int kHalf = KB * D * 2;
  static_assert(16 * D * 4 <= kHalf, "the merge buffer fits a slot");
  __shared__ __attribute__((aligned(1024))) char kslot[kBwdWaves][kHalf];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int g = lane >> 4;
  const int wg = blockIdx.x;
  const int grp = wg % a.gpk;
  const int rest = wg / a.gpk;
  const int h = rest % a.Hkv;
  const int bt = rest / a.Hkv;           // packed token b * T + t
  const int t = bt % a.T;
  const int own = t / a.bs;
  const int nsb = a.bs / KB;

  // kept entries of the token's row (S <= 64): first occurrences of entries
  // 0 <= idx <= own among the first clamp(count, 0, S)
  const int64_t row = (int64_t)bt * a.Hkv + h;
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
        if (ks > t) continue;
        if (u % kBwdWaves == wave) {
          my_ks = (lane == my_n) ? ks : my_ks;
          my_n++;
        }
        u++;
      }
    }
  }

  // Q^T and dO^T fragments (B operands), Delta and lse of column c
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ dO = reinterpret_cast<const __bf16*>(a.dout);
  const __bf16* __restrict__ O = reinterpret_cast<const __bf16*>(a.out);
  const int hq = (h * a.gpk + grp) * a.gv + c;
  const bool cvalid = c < a.gv;
  const int64_t qrow = ((int64_t)bt * a.Hq + (cvalid ? hq : 0)) * D;
  bf16x8 qf[KT], df[KT];
  float dpart = 0.f;
#pragma unroll
  for (int kk = 0; kk < KT; kk++) {
    if (cvalid) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(Q + qrow + kk * 32 + g * 8);
      df[kk] = *reinterpret_cast<const bf16x8*>(dO + qrow + kk * 32 + g * 8);
      const bf16x8 of = *reinterpret_cast<const bf16x8*>(O + qrow + kk * 32 + g * 8);
#pragma unroll
      for (int e = 0; e < 8; e++) dpart += (float)df[kk][e] * (float)of[e];
    } else {
      qf[kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
      df[kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  const float delta = sum_over_groups(dpart);
  const float lse2 = cvalid ? a.lse[(int64_t)bt * a.Hq + hq] * 1.4426950408889634f : INFINITY;
  if (wave == 0 && g == 0 && cvalid) a.delta[(int64_t)bt * a.Hq + hq] = delta;

  const char* __restrict__ Kc = reinterpret_cast<const char*>(a.k);
  const char* __restrict__ Vc = reinterpret_cast<const char*>(a.v);
  const int row_bytes = a.Hkv * D * 2;
  const int64_t kv_bytes = (int64_t)a.B * a.T * row_bytes;
  const int b = bt / a.T;
  const uint32_t koff = (uint32_t)(c * row_bytes + g * 16);
  auto unit_base = [&](int ks) -> int64_t { return (((int64_t)b * a.T + ks) * a.Hkv + h) * (D * 2); };
  u32x4 kreg[MT * KT], vreg[MT * KT];
  auto load_rows = [&](const char* base, int64_t rb, u32x4 (&r)[MT * KT]) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const __amdgpu_buffer_rsrc_t rs = group_rsrc(base, rb + (int64_t)mt * 16 * row_bytes, kv_bytes);
#pragma unroll
      for (int kk = 0; kk < KT; kk++)
        r[mt * KT + kk] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(koff + kk * 64), 0, 0);
    }
  };
  NSA_LDS char* kl = (NSA_LDS char*)&kslot[wave][0];

  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl = a.scale_log2;

  auto step = [&]<bool kMore>(int i) __attribute__((always_inline)) {
    const int ks = __builtin_amdgcn_readlane(my_ks, i);
    const int64_t rb_n = kMore ? unit_base(__builtin_amdgcn_readlane(my_ks, i + 1)) : 0;
    // K rows into the slot for the transposed reads (lane (c, g): key row
    // 16 mt + c, 16-byte chunk 4 kk + g)
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const int key = mt * 16 + c;
#pragma unroll
      for (int kk = 0; kk < KT; kk++) {
        const int ch = (kk * 4 + g) ^ v_swizzle<D>(key);
        *(NSA_LDS u32x4*)(kl + key * (D * 2) + ch * 16) = kreg[mt * KT + kk];
      }
    }
    f32x4 s[MT], dp[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KT; kk++) {
        s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[mt * KT + kk]), qf[kk],
                                                        s[mt], 0, 0, 0);
        dp[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vreg[mt * KT + kk]), df[kk],
                                                         dp[mt], 0, 0, 0);
      }
    }
    if constexpr (kMore) {
      load_rows(Kc, rb_n, kreg);
      load_rows(Vc, rb_n, vreg);
    }
    // P^T = exp2(S^T sl - lse2) (zero where masked), dS^T = P^T (dP^T - Delta)
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int key = ks + mt * 16 + g * 4 + jj;
        const float p = (key > t) ? 0.f : fast_exp2(__builtin_fmaf(s[mt][jj], sl, -lse2));
        s[mt][jj] = p * (dp[mt][jj] - delta);
      }
    }
    bf16x8 pf[KQ];
#pragma unroll
    for (int kq = 0; kq < KQ; kq++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        pf[kq][jj] = (__bf16)s[2 * kq][jj];
        pf[kq][4 + jj] = (__bf16)s[2 * kq + 1][jj];
      }
    }
    // dQ^T += K^T dS^T, K^T fragments read transposed from the slot
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
#pragma unroll
      for (int kq = 0; kq < KQ; kq++) {
        bf16x8 kf;
#pragma unroll
        for (int half = 0; half < 2; half++) {
          const int key = kq * 32 + half * 16 + g * 4 + (c >> 2);
          const int d0 = dt * 16 + (c & 3) * 4;
          const int pc = (d0 >> 3) ^ v_swizzle<D>(key);
          const s16x4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (NSA_LDS s16x4*)(kl + key * (D * 2) + pc * 16 + (d0 & 7) * 2));
          const bf16x4 tb = __builtin_bit_cast(bf16x4, tv);
#pragma unroll
          for (int e = 0; e < 4; e++) kf[half * 4 + e] = tb[e];
        }
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, pf[kq], o[dt], 0, 0, 0);
      }
    }
  };
  if (my_n > 0) {
    const int64_t rb0 = unit_base(__builtin_amdgcn_readlane(my_ks, 0));
    load_rows(Kc, rb0, kreg);
    load_rows(Vc, rb0, vreg);
    for (int i = 0; i + 1 < my_n; i++) step.template operator()<true>(i);
    step.template operator()<false>(my_n - 1);
  }

  // sum the waves' partial dQ^T through LDS ([d tile][lane group][column]
  // float4s), scale, store fp32
  __syncthreads();
  float* ow = reinterpret_cast<float*>(&kslot[wave][0]);
#pragma unroll
  for (int dt = 0; dt < DT; dt++) *reinterpret_cast<f32x4*>(ow + ((dt * 4 + g) * 16 + c) * 4) = o[dt];
  __syncthreads();
  for (int dt = wave; dt < DT; dt += kBwdWaves) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kBwdWaves; w++)
      acc += *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(&kslot[w][0]) +
                                             ((dt * 4 + g) * 16 + c) * 4);
    if (cvalid) *reinterpret_cast<f32x4*>(a.dq + qrow + dt * 16 + g * 4) = acc * a.scale;
  }
}

// ---------------------------------------------------------------------------
// dk, dv
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64 * kBwdWaves) bwd_dkdv_kernel(BwdArgs a) {
  constexpr int KT = D / 32;   // k-steps of S = Q K^T over d
  constexpr int DT = D / 16;   // 16-column d tiles of dK, dV
  constexpr int kRow = D * 2;  // bytes of one head's row in the slot
  __shared__ __attribute__((aligned(1024))) char slot[kBwdWaves][2][16 * kRow];   // Q_t, dO_t

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int g = lane >> 4;
  const int nchunk = (a.T + 63) / 64;
  const int wg = blockIdx.x;
  const int chunk = wg % nchunk;
  const int bh = wg / nchunk;
  const int h = bh % a.Hkv;
  const int b = bh / a.Hkv;
  const int key0 = chunk * 64 + wave * 16;     // this wave's 16-key tile (position in the sequence)
  if (key0 >= a.T) return;                     // no barrier follows: a wave past the end just leaves
  const int blk = key0 / a.bs;                 // the block holding the tile

  // K and V rows of the tile as B operands (lane (c, g): key row c, d = 32 kk + 8 g)
  const __bf16* __restrict__ Kp = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* __restrict__ Vp = reinterpret_cast<const __bf16*>(a.v);
  const int key = key0 + c;
  const bool kvalid = key < a.T;
  const int64_t krow = (((int64_t)b * a.T + (kvalid ? key : key0)) * a.Hkv + h) * D;
  bf16x8 kf[KT], vf[KT];
#pragma unroll
  for (int kk = 0; kk < KT; kk++) {
    kf[kk] = *reinterpret_cast<const bf16x8*>(Kp + krow + kk * 32 + g * 8);
    vf[kk] = *reinterpret_cast<const bf16x8*>(Vp + krow + kk * 32 + g * 8);
  }
  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) {
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ dO = reinterpret_cast<const __bf16*>(a.dout);
  NSA_LDS char* qs = (NSA_LDS char*)&slot[wave][0][0];
  NSA_LDS char* ds = (NSA_LDS char*)&slot[wave][1][0];
  const float sl = a.scale_log2;

  // the tile's readers: tokens t >= key0 of this sequence whose first
  // clamp(count, 0, S) entries list blk (blk <= t's own block follows)
  for (int t0 = key0; t0 < a.T; t0 += 64) {
    const int tt = t0 + lane;
    bool reads = false;
    if (tt < a.T) {
      const int64_t row = ((int64_t)b * a.T + tt) * a.Hkv + h;
      int n = a.bc[row];
      n = n < 0 ? 0 : (n > a.S ? a.S : n);
      const int32_t* r = a.bi + row * a.S;
      for (int i = 0; i < n; i++) reads = reads || (r[i] == blk);
    }
    uint64_t todo = __ballot(reads);
    while (todo != 0ull) {
      const int bit = __builtin_ctzll(todo);
      todo &= todo - 1ull;
      const int t = t0 + bit;
      const int64_t tok = (int64_t)b * a.T + t;
      for (int grp = 0; grp < a.gpk; grp++) {
        // Q_t, dO_t of the group's heads: A operands (lane (c, g): head c,
        // d = 32 kk + 8 g), also written row-major to the slot for the
        // transposed B reads; lse and Delta of heads 4 g .. 4 g + 3
        const int hq = (h * a.gpk + grp) * a.gv + c;
        const bool cvalid = c < a.gv;
        const int64_t qrow = (tok * a.Hq + (cvalid ? hq : 0)) * D;
        bf16x8 qa[KT], da[KT];
#pragma unroll
        for (int kk = 0; kk < KT; kk++) {
          if (cvalid) {
            qa[kk] = *reinterpret_cast<const bf16x8*>(Q + qrow + kk * 32 + g * 8);
            da[kk] = *reinterpret_cast<const bf16x8*>(dO + qrow + kk * 32 + g * 8);
          } else {
            qa[kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
            da[kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
          }
          *(NSA_LDS bf16x8*)(qs + c * kRow + (kk * 32 + g * 8) * 2) = qa[kk];
          *(NSA_LDS bf16x8*)(ds + c * kRow + (kk * 32 + g * 8) * 2) = da[kk];
        }
        float lse2[4], dl[4];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int hh = g * 4 + jj;
          const bool hv = hh < a.gv;
          const int64_t li = tok * a.Hq + (h * a.gpk + grp) * a.gv + (hv ? hh : 0);
          lse2[jj] = hv ? a.lse[li] * 1.4426950408889634f : INFINITY;
          dl[jj] = hv ? a.delta[li] : 0.f;
        }
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
          const float p = (key > t) ? 0.f : fast_exp2(__builtin_fmaf(sacc[jj], sl, -lse2[jj]));
          pa[jj] = (__bf16)p;
          sa[jj] = (__bf16)(p * (pacc[jj] - dl[jj]));
        }
        // dV += P^T dO, dK += dS^T Q; B operands (heads 4 g .. + 3 at d =
        // 16 dt + c) read transposed from the slot
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the slot rows are written
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
          const int off = (g * 4 + (c >> 2)) * kRow + (dt * 16 + (c & 3) * 4) * 2;
          const bf16x4 qb = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((NSA_LDS s16x4*)(qs + off)));
          const bf16x4 db = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((NSA_LDS s16x4*)(ds + off)));
          dv[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, db, dv[dt], 0, 0, 0);
          dk[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(sa, qb, dk[dt], 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // the slot reads have returned before it is rewritten
      }
    }
  }
  // dK = scale * sum dS^T Q, dV = sum P^T dO; lane (c, g) holds keys 4 g + jj at d = 16 dt + c
#pragma unroll
  for (int jj = 0; jj < 4; jj++) {
    const int kr = key0 + g * 4 + jj;
    if (kr >= a.T) continue;
    const int64_t o = (((int64_t)b * a.T + kr) * a.Hkv + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      a.dk[o + dt * 16 + c] = dk[dt][jj] * a.scale;
      a.dv[o + dt * 16 + c] = dv[dt][jj];
    }
  }
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
  a.out = out;
  a.lse = lse;
  a.dout = dout;
  a.bi = block_indices;
  a.bc = block_counts;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.B = p.B;
  a.T = p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.S = p.S;
  a.bs = p.bs;
  a.G = p.G;
  a.gv = p.gv;
  a.gpk = p.gpk;
  a.nb = (p.T + p.bs - 1) / p.bs;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int64_t n_dq = (int64_t)p.B * p.T * p.Hkv * p.gpk;
  const int64_t n_kv = (int64_t)p.B * p.Hkv * ((p.T + 63) / 64);
  if (p.D == 64) {
    hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)n_dq), dim3(64 * kBwdWaves), 0, stream, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)n_kv), dim3(64 * kBwdWaves), 0, stream, a);
  } else if (p.D == 128) {
    hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)n_dq), dim3(64 * kBwdWaves), 0, stream, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3((unsigned)n_kv), dim3(64 * kBwdWaves), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nsa
