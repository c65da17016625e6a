// Internal launcher declarations shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/abg.h"

namespace abg {

// Launch parameters of the attention forward after host-side validation.
struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* bias;          // compact bias, or NULL when pair is given
  const void* pair;           // bf16 pair representation [., P, P, 128] whose
                              // projection replaces bias (bf16 with the cap)
  const void* weight;         // bf16 [128, 8] projection weight with pair
  void* out;
  float* ws;                  // fp32 partials when kv_splits > 1, else unused
  int64_t B;
  int64_t Sq;                 // query positions in q / out
  int64_t Sk;                 // key positions (the sequence length)
  int64_t q_offset;           // position of q's first row in the sequence
  int64_t Dv;                 // 128, or 192 (bf16 with the cap)
  int64_t bias_batch_stride;  // elements (of pair when pair is given)
  int64_t bias_group;
  int64_t kv_splits;          // key ranges computed by separate workgroups
  float scale;
  float softcap;
  abg_dtype dtype;
};

hipError_t launch_biased_mqa_fwd(const AttnLaunch& a, hipStream_t stream);

// Bytes of the library-owned scratch array that abg_biased_mqa_fwd_ex_noalloc
// uses in place of a caller's workspace (one copy per GPU).
constexpr int64_t kScratchBytes = ABG_NOALLOC_SCRATCH_BYTES;

// Device address of that array on the current device (looked up once per
// device with hipGetSymbolAddress, then cached).
hipError_t scratch_address(void** ptr);

hipError_t launch_pair_bias_project(const void* pair, const void* weight, float* bias,
                                    int64_t Bp, int64_t P, int64_t C, abg_dtype dtype,
                                    hipStream_t stream);

}  // namespace abg
