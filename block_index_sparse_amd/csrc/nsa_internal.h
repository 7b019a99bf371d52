// Internal declarations shared by the host API and the gfx950 kernels of the
// native sparse attention forward.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nsa_bwd_plan.h"
#include "nsa_plan.h"

namespace nsa {

// Unit-table word: one per streamed unit (list entry x key sub-block).
//   bit 31     unit is live (block in range, first key not past the item's last token)
//   bits 24-27 attention waves that read the unit
//   bits 0-23  block id
__host__ __device__ constexpr uint32_t unit_word(int32_t block, int32_t npart) {
  return 0x80000000u | ((uint32_t)npart << 24) | (uint32_t)block;
}

// Launchers (defined in the .hip files).
hipError_t launch_schedule(const Plan& p, const int32_t* block_indices, const int32_t* block_counts,
                           const int32_t* cu_seqlens, char* ws, hipStream_t stream);
hipError_t launch_fwd(const Plan& p, const void* q, const void* k, const void* v, float scale,
                      void* out, float* lse, char* ws, hipStream_t stream);
hipError_t launch_dq_ring(const Plan& p, const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const void* dout, float scale, float* dq, float* delta,
                          uint32_t* readers, int32_t rd_nb, int32_t rd_nw, char* ws, hipStream_t stream);
hipError_t launch_decode(const DecodePlan& p, const void* q, const void* k, const void* v,
                         const int32_t* seq_lens, const int32_t* block_indices,
                         const int32_t* block_counts, float scale, void* out, float* lse,
                         hipStream_t stream);
hipError_t launch_bwd(const BwdPlan& p, const void* q, const void* k, const void* v, const void* out,
                      const float* lse, const void* dout, const int32_t* block_indices,
                      const int32_t* block_counts, float scale, float* dq, float* dk, float* dv,
                      float* delta, hipStream_t stream);
int device_cu_count();

}  // namespace nsa
