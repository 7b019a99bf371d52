// C ABI of the native sparse attention forward: argument checks, work
// tiling, workspace layout and launches.  See include/nsa.h for the contract.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "nsa.h"
#include "nsa_internal.h"

namespace {

using nsa::Plan;

// The plan of a forward call on the current device (its CU count sets the
// number of persistent workgroups).
nsa_status make_plan(const nsa_dims* d, int32_t block_size, int32_t num_seqs, bool varlen, Plan* p,
                     bool qblock = false) {
  return nsa::make_plan(d, block_size, num_seqs, varlen, p, qblock, nsa::device_cu_count());
}

using nsa::make_bwd_plan;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

nsa_status check_tensors(const Plan& p, const void* q, const void* k, const void* v, const void* out,
                         const void* workspace, size_t workspace_bytes, float scale) {
  if (!q || !k || !v || !out || !workspace) return NSA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return NSA_ERROR_INVALID_VALUE;
  if (!std::isfinite(scale)) return NSA_ERROR_INVALID_VALUE;
  if (workspace_bytes < p.bytes) return NSA_ERROR_WORKSPACE_TOO_SMALL;
  return NSA_SUCCESS;
}

bool log_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("NSA_LOG");
    v = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return v == 1;
}

nsa_status run(const nsa_dims* d, const void* q, const void* k, const void* v,
               const int32_t* block_indices, const int32_t* block_counts, const int32_t* cu_seqlens,
               int32_t num_seqs, bool varlen, int32_t block_size, float scale, void* out, float* lse,
               void* workspace, size_t workspace_bytes, void* stream, bool qblock = false) {
  Plan p;
  nsa_status st = make_plan(d, block_size, num_seqs, varlen, &p, qblock);
  if (st != NSA_SUCCESS) return st;
  if (!block_indices || !block_counts) return NSA_ERROR_INVALID_VALUE;
  if (varlen && !cu_seqlens) return NSA_ERROR_INVALID_VALUE;
  st = check_tensors(p, q, k, v, out, workspace, workspace_bytes, scale);
  if (st != NSA_SUCCESS) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (log_enabled())
    fprintf(stderr, "[nsa] %s%s D=%d bs=%d G=%d gv=%d tpt=%d ntpw=%d tq=%d items=%d umax=%d nwg=%d ws=%zu\n",
            p.bf16 ? "bf16" : "f32", p.qblock ? " qblock" : "", p.D, p.bs, p.G, p.gv, p.tpt, p.ntpw, p.tq,
            p.n_items, p.umax, p.nwg, p.bytes);
  if (nsa::launch_schedule(p, block_indices, block_counts, cu_seqlens, ws, s) != hipSuccess)
    return NSA_ERROR_LAUNCH_FAILED;
  if (nsa::launch_fwd(p, q, k, v, scale, out, lse, ws, s) != hipSuccess)
    return NSA_ERROR_LAUNCH_FAILED;
  return NSA_SUCCESS;
}

// ---------------------------------------------------------------------------
// Scratch of nsa_fwd_noalloc: the schedule workspace of a fixed-length call,
// a static device array every GPU the library runs on holds until the
// process ends.  Host code never uses the array's name as an address: the
// device address of each GPU's copy is looked up once, with that GPU
// current, and kept per device.
constexpr size_t kScratchBytes = NSA_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

nsa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NSA_ERROR_LAUNCH_FAILED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NSA_ERROR_LAUNCH_FAILED;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return NSA_SUCCESS;
}

// The run's device status word, copied where the caller asked for it.
__global__ void copy_status_kernel(const int32_t* __restrict__ err, int32_t* __restrict__ out) {
  if (threadIdx.x == 0) *out = *err;
}

}  // namespace

extern "C" {

size_t nsa_fwd_workspace_size(const nsa_dims* dims, int32_t block_size, int32_t num_seqs) {
  Plan p;
  if (make_plan(dims, block_size, num_seqs, num_seqs > 0, &p) != NSA_SUCCESS) return 0;
  return p.bytes;
}

nsa_status nsa_fwd(const nsa_dims* dims, const void* q, const void* k, const void* v,
                   const int32_t* block_indices, const int32_t* block_counts, int32_t block_size,
                   float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return run(dims, q, k, v, block_indices, block_counts, nullptr, 0, false, block_size, scale, out,
             lse, workspace, workspace_bytes, stream);
}

nsa_status nsa_fwd_noalloc(const nsa_dims* dims, const void* q, const void* k, const void* v,
                           const int32_t* block_indices, const int32_t* block_counts,
                           int32_t block_size, float scale, void* out, float* lse,
                           int32_t* device_status, void* stream) {
  Plan p;
  nsa_status st = make_plan(dims, block_size, 0, false, &p);
  if (st != NSA_SUCCESS) return st;
  // argument errors first: they need no device
  if (!block_indices || !block_counts || !q || !k || !v || !out) return NSA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return NSA_ERROR_INVALID_VALUE;
  if (!std::isfinite(scale)) return NSA_ERROR_INVALID_VALUE;
  if (p.bytes > kScratchBytes) return NSA_ERROR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != NSA_SUCCESS) return st;
  st = run(dims, q, k, v, block_indices, block_counts, nullptr, 0, false, block_size, scale, out, lse, ws,
           kScratchBytes, stream);
  if (st != NSA_SUCCESS || !device_status) return st;
  hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(ws) + p.off_err), device_status);
  return hipGetLastError() == hipSuccess ? NSA_SUCCESS : NSA_ERROR_LAUNCH_FAILED;
}

nsa_status nsa_fwd_varlen(const nsa_dims* dims, const void* q, const void* k, const void* v,
                          const int32_t* block_indices, const int32_t* block_counts,
                          const int32_t* cu_seqlens, int32_t num_seqs, int32_t block_size,
                          float scale, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return run(dims, q, k, v, block_indices, block_counts, cu_seqlens, num_seqs, true, block_size,
             scale, out, lse, workspace, workspace_bytes, stream);
}

nsa_status nsa_fwd_qblock(const nsa_dims* dims, const void* q, const void* k, const void* v,
                          const int32_t* block_indices, const int32_t* block_counts,
                          int32_t block_size, float scale, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return run(dims, q, k, v, block_indices, block_counts, nullptr, 0, false, block_size, scale, out,
             lse, workspace, workspace_bytes, stream, true);
}

nsa_status nsa_fwd_schedule_qblock(const nsa_dims* dims, const int32_t* block_indices,
                                   const int32_t* block_counts, int32_t block_size,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   size_t* list_offset, int32_t* list_len) {
  Plan p;
  nsa_status st = make_plan(dims, block_size, 0, false, &p, true);
  if (st != NSA_SUCCESS) return st;
  if (!block_indices || !block_counts || !workspace) return NSA_ERROR_INVALID_VALUE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return NSA_ERROR_INVALID_VALUE;
  if (workspace_bytes < p.bytes) return NSA_ERROR_WORKSPACE_TOO_SMALL;
  if (nsa::launch_schedule(p, block_indices, block_counts, nullptr, reinterpret_cast<char*>(workspace),
                           reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return NSA_ERROR_LAUNCH_FAILED;
  if (list_offset) *list_offset = p.off_worklist;
  if (list_len) *list_len = p.n_items;
  return NSA_SUCCESS;
}

nsa_status nsa_fwd_schedule(const nsa_dims* dims, const int32_t* block_indices,
                            const int32_t* block_counts, const int32_t* cu_seqlens,
                            int32_t num_seqs, int32_t block_size, void* workspace,
                            size_t workspace_bytes, void* stream, size_t* list_offset,
                            int32_t* list_len) {
  const bool varlen = cu_seqlens != nullptr;
  Plan p;
  nsa_status st = make_plan(dims, block_size, varlen ? num_seqs : 0, varlen, &p);
  if (st != NSA_SUCCESS) return st;
  if (!block_indices || !block_counts || !workspace) return NSA_ERROR_INVALID_VALUE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return NSA_ERROR_INVALID_VALUE;
  if (workspace_bytes < p.bytes) return NSA_ERROR_WORKSPACE_TOO_SMALL;
  if (nsa::launch_schedule(p, block_indices, block_counts, cu_seqlens,
                           reinterpret_cast<char*>(workspace),
                           reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return NSA_ERROR_LAUNCH_FAILED;
  if (list_offset) *list_offset = p.off_worklist;
  if (list_len) *list_len = p.n_items;
  return NSA_SUCCESS;
}

nsa_status nsa_fwd_execute(const nsa_dims* dims, const void* q, const void* k, const void* v,
                           int32_t num_seqs, int32_t block_size, float scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  nsa_status st = make_plan(dims, block_size, num_seqs, num_seqs > 0, &p);
  if (st != NSA_SUCCESS) return st;
  st = check_tensors(p, q, k, v, out, workspace, workspace_bytes, scale);
  if (st != NSA_SUCCESS) return st;
  if (nsa::launch_fwd(p, q, k, v, scale, out, lse, reinterpret_cast<char*>(workspace),
                      reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return NSA_ERROR_LAUNCH_FAILED;
  return NSA_SUCCESS;
}

nsa_status nsa_fwd_device_status(const nsa_dims* dims, int32_t block_size, int32_t num_seqs,
                                 const void* workspace, size_t workspace_bytes, void* stream,
                                 int32_t* status) {
  Plan p;
  nsa_status st = make_plan(dims, block_size, num_seqs, num_seqs > 0, &p);
  if (st != NSA_SUCCESS) return st;
  if (!workspace || !status) return NSA_ERROR_INVALID_VALUE;
  if (workspace_bytes < p.bytes) return NSA_ERROR_WORKSPACE_TOO_SMALL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t word = 0;
  if (hipMemcpyAsync(&word, reinterpret_cast<const char*>(workspace) + p.off_err, sizeof(word),
                     hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return NSA_ERROR_LAUNCH_FAILED;
  *status = word;
  return NSA_SUCCESS;
}

nsa_status nsa_decode(const nsa_dims* d, const void* q, const void* k, const void* v,
                      const int32_t* seq_lens, const int32_t* block_indices,
                      const int32_t* block_counts, int32_t block_size, float scale, void* out,
                      float* lse, void* stream) {
  if (!d) return NSA_ERROR_INVALID_VALUE;
  if (d->batch <= 0 || d->seqlen <= 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 ||
      d->head_dim <= 0 || d->num_selected <= 0 || block_size <= 0)
    return NSA_ERROR_INVALID_VALUE;
  if (d->num_q_heads % d->num_kv_heads) return NSA_ERROR_INVALID_VALUE;
  if (d->dtype != NSA_DTYPE_BF16) return NSA_ERROR_NOT_SUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return NSA_ERROR_NOT_SUPPORTED;
  if (block_size != 32 && block_size != 64 && block_size != 128) return NSA_ERROR_NOT_SUPPORTED;
  if (d->num_selected > 64) return NSA_ERROR_NOT_SUPPORTED;
  nsa::DecodePlan p;
  p.B = d->batch;
  p.Smax = d->seqlen;
  p.Hq = d->num_q_heads;
  p.Hkv = d->num_kv_heads;
  p.D = d->head_dim;
  p.S = d->num_selected;
  p.bs = block_size;
  p.G = p.Hq / p.Hkv;
  if (p.G <= 16) {
    p.gv = p.G;
    p.gpk = 1;
  } else if (p.G % 16 == 0 && p.G <= 1024) {
    p.gv = 16;
    p.gpk = p.G / 16;
  } else {
    return NSA_ERROR_NOT_SUPPORTED;
  }
  const int64_t rows = (int64_t)p.B * p.Smax;
  if (rows > INT32_MAX / 2 || !nsa::product_le(rows, p.Hkv, p.D, INT64_C(1) << 40) ||
      !nsa::product_le(p.B, p.Hkv, p.gpk, INT32_MAX / 2))
    return NSA_ERROR_NOT_SUPPORTED;
  if (!q || !k || !v || !out || !seq_lens || !block_indices || !block_counts) return NSA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return NSA_ERROR_INVALID_VALUE;
  if (!std::isfinite(scale)) return NSA_ERROR_INVALID_VALUE;
  if (nsa::launch_decode(p, q, k, v, seq_lens, block_indices, block_counts, scale, out, lse,
                         reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return NSA_ERROR_LAUNCH_FAILED;
  return NSA_SUCCESS;
}

size_t nsa_bwd_workspace_size(const nsa_dims* dims, int32_t block_size) {
  nsa::BwdPlan p;
  if (make_bwd_plan(dims, block_size, &p) != NSA_SUCCESS) return 0;
  return nsa::bwd_workspace_bytes(p);
}

nsa_status nsa_bwd(const nsa_dims* d, const void* q, const void* k, const void* v, const void* out,
                   const float* lse, const void* dout, const int32_t* block_indices,
                   const int32_t* block_counts, int32_t block_size, float scale, float* dq, float* dk,
                   float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  nsa::BwdPlan p;
  nsa_status st = make_bwd_plan(d, block_size, &p, nsa::device_cu_count());
  if (st != NSA_SUCCESS) return st;
  if (!q || !k || !v || !out || !lse || !dout || !block_indices || !block_counts || !dq || !dk || !dv ||
      !workspace)
    return NSA_ERROR_INVALID_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return NSA_ERROR_INVALID_VALUE;
  if (!std::isfinite(scale)) return NSA_ERROR_INVALID_VALUE;
  if (workspace_bytes < nsa::bwd_workspace_bytes(p)) return NSA_ERROR_WORKSPACE_TOO_SMALL;
  if (nsa::launch_bwd(p, q, k, v, out, lse, dout, block_indices, block_counts, scale, dq, dk, dv,
                      reinterpret_cast<float*>(workspace), reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return NSA_ERROR_LAUNCH_FAILED;
  return NSA_SUCCESS;
}

nsa_status nsa_bwd_device_status(const nsa_dims* dims, int32_t block_size, const void* workspace,
                                 size_t workspace_bytes, void* stream, int32_t* status) {
  nsa::BwdPlan p;
  nsa_status st = make_bwd_plan(dims, block_size, &p);
  if (st != NSA_SUCCESS) return st;
  if (!workspace || !status) return NSA_ERROR_INVALID_VALUE;
  if (workspace_bytes < nsa::bwd_workspace_bytes(p)) return NSA_ERROR_WORKSPACE_TOO_SMALL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t word = 0;
  const char* at = reinterpret_cast<const char*>(workspace) + nsa::bwd_schedule_offset(p) + p.fp.off_err;
  if (hipMemcpyAsync(&word, at, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return NSA_ERROR_LAUNCH_FAILED;
  *status = word;
  return NSA_SUCCESS;
}

const char* nsa_status_string(nsa_status status) {
  switch (status) {
    case NSA_SUCCESS: return "NSA_SUCCESS";
    case NSA_ERROR_INVALID_VALUE: return "NSA_ERROR_INVALID_VALUE";
    case NSA_ERROR_NOT_SUPPORTED: return "NSA_ERROR_NOT_SUPPORTED";
    case NSA_ERROR_WORKSPACE_TOO_SMALL: return "NSA_ERROR_WORKSPACE_TOO_SMALL";
    case NSA_ERROR_LAUNCH_FAILED: return "NSA_ERROR_LAUNCH_FAILED";
  }
  return "NSA_UNKNOWN_STATUS";
}

int32_t nsa_abi_version(void) { return NSA_ABI_VERSION; }

}  // extern "C"
