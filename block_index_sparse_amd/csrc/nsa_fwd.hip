// Native sparse attention forward kernels for gfx950 (CDNA4).
//
// Operation (ejKernel native_sparse_attention API page, module description
// and "Parameters"): for each query token, the G query heads of kv head h
// attend to the keys of the blocks listed for (token, h), causal inside the
// token's own block; softmax(scale * q.k) weighted sum of v, plus the
// log-sum-exp of the scores.
//
// Mapping onto the matrix cores.  One wave owns one work item (a tile of
// consecutive tokens of one sequence and one kv head) and walks the item's
// merged block list in ascending block order.  The MFMA "N" dimension (16
// columns) holds query heads -- the G heads of one token, or 16/G tokens x G
// heads when G < 16 -- so one gathered K/V block feeds every head of the GQA
// group.  The products are computed transposed:
//
//   S^T (keys x cols) = K (keys x D) . Q^T (D x cols)       A = K rows, B = Q
//   O^T (D x cols)   += V^T (D x keys) . P^T (keys x cols)  A = V^T, B = P^T
//
// With this orientation the fp32 accumulator layout of S^T (lane = column,
// four consecutive keys per lane group) is exactly the B-operand layout P^T
// needs, so P never leaves its registers: it is exponentiated, rounded to
// bf16 and fed back to the PV product in place.  V^T fragments come from a
// per-wave LDS copy of the block through ds_read_b64_tr_b16, the gfx950
// transposing LDS read (lanes 4r..4r+3 of each 16-lane group supply row r of
// a 4x16 tile and lane i receives column i).  K fragments are 16-byte global
// loads straight into the A-operand registers.
//
// Softmax: fp32 online softmax in the log2 domain (scores pre-multiplied by
// scale*log2(e), v_exp_f32 for 2^x), running max and normaliser per column,
// cross-lane reductions over the four lane groups, causal mask evaluated only
// on blocks that reach past the item's first token.  The running state is
// the (output, max, normaliser) carry of a flash-attention block step (the
// `flash_attention_block` carry on the ejKernel ragged-decode page).
#include "nsa_internal.h"

namespace nsa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

#define NSA_LDS __attribute__((address_space(3)))

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const ItemHeader* hdr;
  const BlockEntry* lists;
  const int32_t* worklist;
  int32_t Ttot;     // packed token rows
  int32_t Hq, Hkv, G, tpt, n_tiles, n_items, umax, bs;
  float scale_log2;  // scale * log2(e)
};

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs
// on XCD i % 8).  Remap so that each XCD walks consecutive runs of
// kXcdRun workgroups of the longest-first list: neighbouring items (same kv
// head, adjacent tokens, shared sink/local blocks) then share one L2.
constexpr int kXcds = 8;
constexpr int kXcdRun = 8;

__device__ __forceinline__ int xcd_remap(int wg, int nwg) {
  const int group = kXcds * kXcdRun;
  const int full = (nwg / group) * group;
  if (wg >= full) return wg;
  const int x = wg % kXcds, k = wg / kXcds;
  return (k / kXcdRun) * group + x * kXcdRun + (k % kXcdRun);
}

__device__ __forceinline__ float wave_max_groups(float v) {
  // reduce over the four 16-lane groups (lanes c, c+16, c+32, c+48)
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ __forceinline__ float wave_sum_groups(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Column c of column tile n -> (token offset in item, head in group, valid).
__device__ __forceinline__ void column_of(int n, int c, int G, int tpt, int ntok, int& tau,
                                          int& head, bool& valid) {
  if (G <= 16) {
    tau = n * tpt + c / G;
    head = c - (c / G) * G;
    valid = (c < tpt * G) && (tau < ntok);
  } else {
    tau = 0;
    head = n * 16 + c;
    valid = true;
  }
}

// A scheduled header is used only if it stays inside the tensors; a
// workspace that does not hold a matching schedule then cannot make the
// kernel touch memory outside its arguments.
__device__ __forceinline__ bool header_ok(ItemHeader& hd, const FwdArgs& a) {
  if (hd.ntok <= 0 || hd.ntok > 32 || hd.pos0 < 0 || hd.tok0 < hd.pos0) return false;
  if (hd.tok0 + hd.ntok > a.Ttot) return false;
  hd.nunion = min(max(hd.nunion, 0), a.umax);
  return true;
}

__device__ __forceinline__ uint32_t tile_token_mask(int n, int G, int tpt) {
  return G <= 16 ? (((1u << tpt) - 1u) << (n * tpt)) : 1u;
}

// XOR swizzle of 16-byte chunks in the LDS copy of V: rows that one
// transposing read touches together land on distinct bank groups.
template <int D>
__device__ __forceinline__ int v_swizzle(int row) {
  constexpr int kRowsPer256 = 256 / (D * 2) > 0 ? 256 / (D * 2) : 1;
  constexpr int kPairs = D / 16;  // 16-byte chunk pairs per row
  return ((row / kRowsPer256) & (kPairs - 1)) << 1;
}

// ---------------------------------------------------------------------------
// bf16: D in {64, 128}, KB keys per step in {32, 64}, NT column tiles per item
// ---------------------------------------------------------------------------
template <int D, int KB, int NT>
__global__ void __launch_bounds__(256, 2) fwd_bf16_kernel(FwdArgs a) {
  constexpr int KT = D / 32;   // k-steps of S^T = K Q^T
  constexpr int MT = KB / 16;  // 16-key row tiles of S^T
  constexpr int KQ = KB / 32;  // 32-key k-steps of O^T += V^T P^T
  constexpr int DT = D / 16;   // 16-row tiles of O^T
  constexpr int CH = D / 8;    // 16-byte chunks per K/V row
  __shared__ __attribute__((aligned(16))) __bf16 vlds[kWaves][KB * D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int pos = xcd_remap(blockIdx.x, gridDim.x) * kWaves + wave;
  if (pos >= a.n_items) return;
  const int item = a.worklist[pos];
  if (item < 0 || item >= a.n_items) return;
  ItemHeader hd = a.hdr[item];
  if (!header_ok(hd, a)) return;
  const int h = item / a.n_tiles;
  const int bos = hd.tok0 - hd.pos0;
  const int tmin = hd.pos0;
  const int tmax = hd.pos0 + hd.ntok - 1;
  const __bf16* __restrict__ Q = reinterpret_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ K = reinterpret_cast<const __bf16*>(a.k);
  const __bf16* __restrict__ V = reinterpret_cast<const __bf16*>(a.v);
  NSA_LDS __bf16* vl = (NSA_LDS __bf16*)(&vlds[wave][0]);

  int tau[NT], hq[NT], tcol[NT];
  bool cvalid[NT];
  bf16x8 qf[NT][KT];
  f32x4 o[NT][DT];
  float mrun[NT], lrun[NT];
#pragma unroll
  for (int n = 0; n < NT; n++) {
    int head;
    column_of(n, c, a.G, a.tpt, hd.ntok, tau[n], head, cvalid[n]);
    hq[n] = h * a.G + head;
    tcol[n] = hd.pos0 + tau[n];
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
  }

  const BlockEntry* list = a.lists + (int64_t)item * a.umax;
  const int nsteps_per_block = a.bs / KB;
  for (int u = 0; u < hd.nunion; u++) {
    const BlockEntry be = list[u];
    if (be.block < 0 || be.block > tmax / a.bs) continue;
    bool act[NT];
    bool sel[NT];
#pragma unroll
    for (int n = 0; n < NT; n++) {
      act[n] = (be.tokmask & tile_token_mask(n, a.G, a.tpt)) != 0u;
      sel[n] = cvalid[n] && ((be.tokmask >> tau[n]) & 1u);
    }
    for (int sb = 0; sb < nsteps_per_block; sb++) {
      const int kstart = be.block * a.bs + sb * KB;  // first key (sequence-relative)
      if (kstart > tmax) break;
      const bool diag = (kstart + KB - 1) > tmin;
      const int row0 = bos + kstart;

      // ---- stage V[row0 .. row0+KB) into this wave's LDS (swizzled rows)
#pragma unroll
      for (int it = 0; it < KB * CH / 64; it++) {
        const int qd = it * 64 + lane;
        const int r = qd / CH;
        const int ch = qd - r * CH;
        const int grow = min(row0 + r, a.Ttot - 1);
        const i32x4 val = *reinterpret_cast<const i32x4*>(V + ((int64_t)grow * a.Hkv + h) * D + ch * 8);
        *reinterpret_cast<NSA_LDS i32x4*>(vl + r * D + ((ch ^ v_swizzle<D>(r)) * 8)) = val;
      }

      // ---- K fragments: A operand rows = keys 16*mt + c, k = 32*kk + 8*g .. +7
      bf16x8 kf[MT][KT];
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        const int grow = min(row0 + mt * 16 + c, a.Ttot - 1);
        const __bf16* kp = K + ((int64_t)grow * a.Hkv + h) * D + g * 8;
#pragma unroll
        for (int kk = 0; kk < KT; kk++) kf[mt][kk] = *reinterpret_cast<const bf16x8*>(kp + kk * 32);
      }

      bf16x8 pf[NT][KQ];
#pragma unroll
      for (int n = 0; n < NT; n++) {
        if (!act[n]) continue;
        f32x4 s[MT];
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
          s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KT; kk++)
            s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mt][kk], qf[n][kk], s[mt], 0, 0, 0);
        }
        // scale + masks; lane (c, g) holds keys 16*mt + 4*g + jj of column c
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            float x = s[mt][jj] * a.scale_log2;
            const int kp = kstart + mt * 16 + g * 4 + jj;
            if (!sel[n] || (diag && kp > tcol[n])) x = -INFINITY;
            s[mt][jj] = x;
            mx = fmaxf(mx, x);
          }
        }
        mx = wave_max_groups(mx);
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
        rs = wave_sum_groups(rs);
        lrun[n] = lrun[n] * alpha + rs;
        mrun[n] = mnew;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) o[n][dt] *= alpha;
#pragma unroll
        for (int kq = 0; kq < KQ; kq++) {
          bf16x8 pk;
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            pk[jj] = (__bf16)s[2 * kq][jj];
            pk[4 + jj] = (__bf16)s[2 * kq + 1][jj];
          }
          pf[n][kq] = pk;
        }
      }

      // ---- O^T += V^T P^T ; V^T fragments through the transposing LDS read
#pragma unroll
      for (int dt = 0; dt < DT; dt++) {
#pragma unroll
        for (int kq = 0; kq < KQ; kq++) {
          bf16x8 vf;
#pragma unroll
          for (int half = 0; half < 2; half++) {
            const int key = kq * 32 + half * 16 + g * 4 + (c >> 2);
            const int d0 = dt * 16 + (c & 3) * 4;
            const int chk = d0 >> 3;
            const int addr = key * D + ((chk ^ v_swizzle<D>(key)) << 3) + (d0 & 7);
            const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                reinterpret_cast<NSA_LDS s16x4*>(vl + addr));
            const bf16x4 tb = __builtin_bit_cast(bf16x4, t);
#pragma unroll
            for (int e = 0; e < 4; e++) vf[half * 4 + e] = tb[e];
          }
#pragma unroll
          for (int n = 0; n < NT; n++) {
            if (!act[n]) continue;
            o[n][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[n][kq], o[n][dt], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- epilogue: out = O / l (bf16, round to nearest even), lse = ln 2 * (m + log2 l)
  __bf16* __restrict__ Out = reinterpret_cast<__bf16*>(a.out);
#pragma unroll
  for (int n = 0; n < NT; n++) {
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
}

// ---------------------------------------------------------------------------
// fp32: same walk, v_mfma_f32_16x16x4_f32 (fp32 products, fp32 accumulation),
// P stays fp32; V^T fragments are single fp32 elements read from global.
// ---------------------------------------------------------------------------
template <int D, int KB, int NT>
__global__ void __launch_bounds__(256, 2) fwd_f32_kernel(FwdArgs a) {
  constexpr int KT = D / 4;
  constexpr int MT = KB / 16;
  constexpr int DT = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int pos = xcd_remap(blockIdx.x, gridDim.x) * kWaves + wave;
  if (pos >= a.n_items) return;
  const int item = a.worklist[pos];
  if (item < 0 || item >= a.n_items) return;
  ItemHeader hd = a.hdr[item];
  if (!header_ok(hd, a)) return;
  const int h = item / a.n_tiles;
  const int bos = hd.tok0 - hd.pos0;
  const int tmin = hd.pos0;
  const int tmax = hd.pos0 + hd.ntok - 1;
  const float* __restrict__ Q = reinterpret_cast<const float*>(a.q);
  const float* __restrict__ K = reinterpret_cast<const float*>(a.k);
  const float* __restrict__ V = reinterpret_cast<const float*>(a.v);

  int tau[NT], hq[NT], tcol[NT];
  bool cvalid[NT];
  float qf[NT][KT];
  f32x4 o[NT][DT];
  float mrun[NT], lrun[NT];
#pragma unroll
  for (int n = 0; n < NT; n++) {
    int head;
    column_of(n, c, a.G, a.tpt, hd.ntok, tau[n], head, cvalid[n]);
    hq[n] = h * a.G + head;
    tcol[n] = hd.pos0 + tau[n];
    const int64_t qrow = ((int64_t)(hd.tok0 + (cvalid[n] ? tau[n] : 0)) * a.Hq + hq[n]) * D;
#pragma unroll
    for (int kk = 0; kk < KT; kk++) qf[n][kk] = cvalid[n] ? Q[qrow + kk * 4 + g] : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) o[n][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mrun[n] = -INFINITY;
    lrun[n] = 0.f;
  }

  const BlockEntry* list = a.lists + (int64_t)item * a.umax;
  const int nsteps_per_block = a.bs / KB;
  for (int u = 0; u < hd.nunion; u++) {
    const BlockEntry be = list[u];
    if (be.block < 0 || be.block > tmax / a.bs) continue;
    bool act[NT], sel[NT];
#pragma unroll
    for (int n = 0; n < NT; n++) {
      act[n] = (be.tokmask & tile_token_mask(n, a.G, a.tpt)) != 0u;
      sel[n] = cvalid[n] && ((be.tokmask >> tau[n]) & 1u);
    }
    for (int sb = 0; sb < nsteps_per_block; sb++) {
      const int kstart = be.block * a.bs + sb * KB;
      if (kstart > tmax) break;
      const bool diag = (kstart + KB - 1) > tmin;
      const int row0 = bos + kstart;
#pragma unroll
      for (int n = 0; n < NT; n++) {
        if (!act[n]) continue;
        f32x4 s[MT];
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
          const int grow = min(row0 + mt * 16 + c, a.Ttot - 1);
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
            if (!sel[n] || (diag && kp > tcol[n])) x = -INFINITY;
            s[mt][jj] = x;
            mx = fmaxf(mx, x);
          }
        }
        mx = wave_max_groups(mx);
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
        rs = wave_sum_groups(rs);
        lrun[n] = lrun[n] * alpha + rs;
        mrun[n] = mnew;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
          f32x4 acc = o[n][dt] * alpha;
#pragma unroll
          for (int mt = 0; mt < MT; mt++) {
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
              const int grow = min(row0 + mt * 16 + g * 4 + jj, a.Ttot - 1);
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
  for (int n = 0; n < NT; n++) {
    if (!cvalid[n]) continue;
    const float l = lrun[n];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t orow = ((int64_t)(hd.tok0 + tau[n]) * a.Hq + hq[n]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
      f32x4 ov = o[n][dt] * inv;
      *reinterpret_cast<f32x4*>(Out + orow + dt * 16 + g * 4) = ov;
    }
    if (a.lse && g == 0) {
      const float lv = l > 0.f ? (mrun[n] + __log2f(l)) * 0.69314718055994530942f : -INFINITY;
      a.lse[(int64_t)(hd.tok0 + tau[n]) * a.Hq + hq[n]] = lv;
    }
  }
}

typedef void (*KernelFn)(FwdArgs);

template <int D, int KB>
KernelFn pick_nt(bool bf16, int nt) {
  if (bf16) {
    switch (nt) {
      case 1: return fwd_bf16_kernel<D, KB, 1>;
      case 2: return fwd_bf16_kernel<D, KB, 2>;
      case 4: return fwd_bf16_kernel<D, KB, 4>;
    }
  } else {
    switch (nt) {
      case 1: return fwd_f32_kernel<D, KB, 1>;
      case 2: return fwd_f32_kernel<D, KB, 2>;
      case 4: return fwd_f32_kernel<D, KB, 4>;
    }
  }
  return nullptr;
}

KernelFn pick(bool bf16, int D, int KB, int nt) {
  if (D == 64) return KB == 32 ? pick_nt<64, 32>(bf16, nt) : pick_nt<64, 64>(bf16, nt);
  if (D == 128) return KB == 32 ? pick_nt<128, 32>(bf16, nt) : pick_nt<128, 64>(bf16, nt);
  return nullptr;
}

}  // namespace

hipError_t launch_fwd(const Plan& p, const void* q, const void* k, const void* v, float scale,
                      void* out, float* lse, char* ws, hipStream_t stream) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.hdr = reinterpret_cast<const ItemHeader*>(ws + p.off_hdr);
  a.lists = reinterpret_cast<const BlockEntry*>(ws + p.off_lists);
  a.worklist = reinterpret_cast<const int32_t*>(ws + p.off_worklist);
  a.Ttot = p.B * p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.tpt = p.tpt;
  a.n_tiles = p.n_tiles;
  a.n_items = p.n_items;
  a.umax = p.umax;
  a.bs = p.bs;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int KB = p.bs < 64 ? p.bs : 64;
  KernelFn fn = pick(p.bf16, p.D, KB, p.nt);
  if (!fn) return hipErrorInvalidValue;
  const int nwg = (p.n_items + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(fn, dim3(nwg), dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nsa
