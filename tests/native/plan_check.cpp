// Sanitizer driver for the host-side plan arithmetic of the library
// (block_index_sparse_amd/csrc/nsa_plan.h, nsa_bwd_plan.h), built with the host compiler
// alone under -fsanitize=address,undefined and run by
// tests/test_sanitizers.py.  It sweeps hostile dims (sizes at and past the
// int32 range, S = 1024 and beyond, G = 1024, huge batches and sequence
// counts) through the forward and backward plans and checks that every
// call returns a defined status and that every accepted plan is consistent:
// workspace sections 256-byte aligned, in order and inside the total, sizes
// equal to a recomputation in 128-bit integers, and backward grids inside
// 2^32 work-items.  Exit status 0 = all checks passed.
#include <cstdio>
#include <vector>

#include "nsa_bwd_plan.h"
#include "nsa_plan.h"

namespace {

int fails = 0;
long fwd_ok = 0, bwd_ok = 0;   // accepted plans

void expect(bool ok, const char* what, const nsa_dims& d, int bs, int ns) {
  if (ok) return;
  fails++;
  if (fails < 20)
    std::printf("FAIL %s: B=%d T=%d Hq=%d Hkv=%d D=%d S=%d dtype=%d bs=%d num_seqs=%d\n", what, d.batch, d.seqlen,
                d.num_q_heads, d.num_kv_heads, d.head_dim, d.num_selected, (int)d.dtype, bs, ns);
}

bool valid_status(nsa_status s) { return s >= NSA_SUCCESS && s <= NSA_ERROR_LAUNCH_FAILED; }

void check_fwd(const nsa_dims& d, int bs, int ns, bool qblock, bool small_units = false) {
  const bool varlen = ns > 0;
  nsa::Plan p;
  const nsa_status st = nsa::make_plan(&d, bs, ns, varlen, &p, qblock, 256, small_units);
  expect(valid_status(st), "fwd status", d, bs, ns);
  if (st != NSA_SUCCESS) return;
  fwd_ok++;
  const size_t offs[] = {p.off_tile_start, p.off_hdr, p.off_bucket, p.off_blocks, p.off_masks, p.off_units,
                         p.off_off, p.off_total, p.off_worklist, p.off_err, p.bytes};
  for (size_t i = 0; i < sizeof(offs) / sizeof(offs[0]); i++) {
    expect(offs[i] % 256 == 0, "fwd section alignment", d, bs, ns);
    if (i) expect(offs[i] > offs[i - 1] || (i + 1 == sizeof(offs) / sizeof(offs[0]) && offs[i] >= offs[i - 1]),
                  "fwd section order", d, bs, ns);
  }
  using u128 = unsigned __int128;
  const u128 items = (u128)p.n_items;
  const u128 need = items * 16 + items * 4 + items * (u128)p.umax * 4 + items * (u128)p.umax * p.mw * 4 +
                    items * (u128)p.umax_units * 4 + items * 4;
  expect((u128)p.bytes >= need, "fwd workspace holds its sections", d, bs, ns);
  expect(p.tq >= 1 && p.tq <= nsa::kMaxTileTokens && p.mw * 32 >= p.tq, "fwd item width", d, bs, ns);
  expect(p.umax >= 1 && p.umax <= nsa::kMaxUnion, "fwd merged-list bound", d, bs, ns);
  expect(p.n_items >= 1 && (int64_t)p.n_tiles * p.hv == p.n_items, "fwd item count", d, bs, ns);
  expect(p.nwg >= 1 && p.nwg % nsa::kXcds == 0, "fwd workgroups", d, bs, ns);
}

void check_bwd(const nsa_dims& d, int bs) {
  nsa::BwdPlan p;
  const nsa_status st = nsa::make_bwd_plan(&d, bs, &p);
  expect(valid_status(st), "bwd status", d, bs, 0);
  if (st != NSA_SUCCESS) return;
  bwd_ok++;
  const nsa::BwdGrids g = nsa::bwd_grids(p);
  const int64_t lim = INT64_C(1) << 32;
  expect(g.dkdv * nsa::kBwdKvThreads < lim && g.reduce * 256 < lim,
         "bwd grids", d, bs, 0);
  // a dk/dv unit's readers fill at most the 16 MFMA rows, and the kernel's
  // division-free row split is exact
  const int tpt = nsa::bwd_unit_readers(p);
  expect(tpt >= 1 && tpt * p.gv <= 16 && (tpt == 1 || p.gpk == 1), "bwd unit readers", d, bs, 0);
  for (int r = 0; r < 16; r++) expect(((r * nsa::bwd_gv_magic(p)) >> 16) == r / p.gv, "bwd row split", d, bs, 0);
  using u128 = unsigned __int128;
  // segment: the base length for T times the unit's readers, at most 4096 and T
  const int64_t base = p.T > 16384 ? 4096 : (p.T > 8192 ? 2048 : (p.T > 4096 ? 1024 : 512));
  const int64_t segl = std::min<int64_t>(std::min<int64_t>(base * tpt, 4096), p.T);
  expect(nsa::bwd_seg_tokens(p) == segl && segl >= 1, "bwd segment length", d, bs, 0);
  const u128 seg = (u128)segl, T = (u128)p.T, ns = (T + seg - 1) / seg;
  const u128 want = ((u128)p.B * T * p.Hq * 4 + 255) / 256 * 256 +
                    ((u128)p.B * p.Hkv * ((T + p.bs - 1) / p.bs) * ((T + 31) / 32) * 4 + 255) / 256 * 256 +
                    (ns > 1 ? (ns * 2 * (u128)p.B * T * p.Hkv * p.D * 4 + 255) / 256 * 256 : 0) + (u128)p.fp.bytes;
  expect((u128)nsa::bwd_workspace_bytes(p) == want, "bwd workspace size", d, bs, 0);
  // the dq ring runs the forward's plan of the same call: one bf16 column
  // tile per attention wave
  {
    expect(p.fp.bf16 && p.fp.ntpw == 1 && p.fp.tpw * p.fp.gv <= 16 && p.fp.B == p.B && p.fp.T == p.T,
           "bwd ring plan", d, bs, 0);
    check_fwd(d, bs, 0, false, true);
    expect(p.fp.kb * p.fp.nsb == p.fp.bs && (p.fp.nsb == 1 || p.fp.nsb == 2), "bwd ring units", d, bs, 0);
  }
}

}  // namespace

int main() {
  const int32_t Bs[] = {1, 2, 7, 1000, 1 << 20, INT32_MAX};
  const int32_t Ts[] = {1, 31, 64, 65, 4097, 32768, 65536, 1 << 20, INT32_MAX / 2, INT32_MAX};
  const int32_t HqHkv[][2] = {{1, 1}, {16, 1}, {64, 4}, {1024, 1}, {1025, 1}, {48, 3}, {24, 1}, {16, 16}, {3, 2}};
  const int32_t Ds[] = {64, 128, 96, 0};
  const int32_t Ss[] = {1, 16, 64, 65, 1024, 4096, INT32_MAX};
  const int32_t bss[] = {32, 64, 128, 0, -1, 48};
  const int32_t nss[] = {0, 1, 8, 1 << 16, INT32_MAX};
  const int32_t dts[] = {NSA_DTYPE_BF16, NSA_DTYPE_F32, 7, -1};
  long n = 0;
  for (int32_t B : Bs)
    for (int32_t T : Ts)
      for (auto& h : HqHkv)
        for (int32_t D : Ds)
          for (int32_t S : Ss)
            for (int32_t dt : dts) {
              const nsa_dims d{B, T, h[0], h[1], D, S, dt};
              for (int32_t bs : bss) {
                check_bwd(d, bs);
                for (int32_t ns : nss) {
                  if (ns > 0 && B != 1) continue;
                  check_fwd(d, bs, ns, false);
                  if (ns == 0) check_fwd(d, bs, 0, true);
                  n++;
                }
              }
            }
  check_fwd(nsa_dims{1, 32768, 64, 4, 128, 16, NSA_DTYPE_BF16}, 64, 0, false);
  std::printf("plan sanitizer check: %ld dims, %ld forward and %ld backward plans accepted, %s\n", n, fwd_ok,
              bwd_ok, fails ? "FAILED" : "ok");
  return fails ? 1 : 0;
}
