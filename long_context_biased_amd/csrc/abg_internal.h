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
  const float* bias;
  void* out;
  int64_t B;
  int64_t S;
  int64_t Dv;                 // 128, or 192 (bf16 with the cap)
  int64_t bias_batch_stride;  // elements
  int64_t bias_group;
  float scale;
  float softcap;
  abg_dtype dtype;
};

hipError_t launch_biased_mqa_fwd(const AttnLaunch& a, hipStream_t stream);

hipError_t launch_pair_bias_project(const void* pair, const void* weight, float* bias,
                                    int64_t Bp, int64_t P, int64_t C, abg_dtype dtype,
                                    hipStream_t stream);

}  // namespace abg
