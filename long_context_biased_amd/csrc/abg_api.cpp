// C ABI of libabg: argument validation and dispatch to the HIP launchers.
//
// Every check runs on the host before any HIP call, so a rejected call
// enqueues nothing and touches no device state (and can be exercised on a
// machine without a GPU).  Contract: include/abg.h.

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "abg_internal.h"

namespace {

thread_local std::string g_last_error;

abg_status fail(abg_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
abg_status fail(abg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

int64_t elem_bytes(abg_dtype d) { return d == ABG_BF16 ? 2 : 4; }

abg_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ABG_OK;
  return fail(ABG_ERR_DEVICE, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// Validation and launch shared by the attention entry points: the bias
// comes either compact (bias, float32 [., Hq, P, P]) or as the pair
// representation and projection weight it is projected from (pair, bf16
// [., P, P, C], and weight [C, Hq]); bias_batch_stride and bias_group then
// describe pair.
// With use_scratch the partials of key ranges go to the library's own
// scratch array instead of a caller's workspace (workspace is ignored): the
// request is rejected if it needs more than that array holds, and the
// array's device address is looked up only after every argument passed.
abg_status attention(const void* q, const void* k, const void* v, const float* bias,
                     const void* pair, const void* weight, int64_t C, void* out,
                     void* workspace, int64_t workspace_bytes, int64_t B, int64_t Sq,
                     int64_t Sk, int64_t q_offset, int64_t Hq, int64_t Dk, int64_t Dv,
                     int64_t bias_batch_stride, int64_t bias_group, int64_t kv_splits,
                     float scale, float softcap, abg_dtype dtype, void* stream,
                     bool use_scratch = false) {
  if (dtype != ABG_F32 && dtype != ABG_BF16)
    return fail(ABG_ERR_VALUE, "dtype %d is not ABG_F32 or ABG_BF16", (int)dtype);
  if (!q) return fail(ABG_ERR_NULL, "q is NULL");
  if (!k) return fail(ABG_ERR_NULL, "k is NULL");
  if (!v) return fail(ABG_ERR_NULL, "v is NULL");
  if (!out) return fail(ABG_ERR_NULL, "out is NULL");
  if (B < 1 || B > 65535) return fail(ABG_ERR_SHAPE, "B = %lld must be in [1, 65535]", (long long)B);
  if (!std::isfinite(softcap) || softcap < 0.f)
    return fail(ABG_ERR_VALUE, "softcap must be finite and >= 0");
  // the bf16 path with the cap (the fast kernel) also takes value width 192
  // and the pair form; every path takes any length and key ranges
  const bool fast = dtype == ABG_BF16 && softcap > 0.f;
  if (Sk < 1 || Sk > 262144)
    return fail(ABG_ERR_SHAPE, "S = %lld must be in [1, 262144]", (long long)Sk);
  if (Sq < 1 || Sq > Sk)
    return fail(ABG_ERR_SHAPE, "Sq = %lld must be in [1, Sk = %lld]", (long long)Sq, (long long)Sk);
  if (q_offset < 0 || q_offset > Sk - Sq)
    return fail(ABG_ERR_SHAPE, "q_offset = %lld must be in [0, Sk - Sq = %lld]", (long long)q_offset,
                (long long)(Sk - Sq));
  if (q_offset % 16 != 0)
    return fail(ABG_ERR_UNSUPPORTED, "q_offset = %lld must be a multiple of 16", (long long)q_offset);
  if (Hq != 8) return fail(ABG_ERR_UNSUPPORTED, "Hq = %lld: only 8 query heads are supported", (long long)Hq);
  if (Dk != 128) return fail(ABG_ERR_UNSUPPORTED, "Dk = %lld: only 128 is supported", (long long)Dk);
  if (Dv != 128 && Dv != 192)
    return fail(ABG_ERR_UNSUPPORTED, "Dv = %lld: only 128 and 192 are supported", (long long)Dv);
  if (!std::isfinite(scale)) return fail(ABG_ERR_VALUE, "scale is not finite");
  if (Dv == 192 && !fast)
    return fail(ABG_ERR_UNSUPPORTED, "Dv = 192 is implemented for bf16 inputs with softcap > 0 only");
  if (kv_splits < 1 || kv_splits > 64)
    return fail(ABG_ERR_SHAPE, "kv_splits = %lld must be in [1, 64]", (long long)kv_splits);
  const int64_t tiles = (Sk + 63) / 64;
  if (tiles % kv_splits != 0)
    return fail(ABG_ERR_SHAPE, "kv_splits = %lld must divide the %lld key tiles", (long long)kv_splits,
                (long long)tiles);
  const int64_t ws_need = abg_biased_mqa_fwd_workspace_bytes(B, Sq, Hq, Dv, kv_splits);
  if (use_scratch) {
    if (kv_splits > 1 && (ws_need < 0 || ws_need > abg::kScratchBytes))
      return fail(ABG_ERR_SHAPE,
                  "kv_splits = %lld needs %lld bytes of partials; the no-allocation entry point "
                  "holds at most %lld (use fewer key ranges or fewer query positions per call, "
                  "or abg_biased_mqa_fwd_ex with a workspace)",
                  (long long)kv_splits, (long long)ws_need, (long long)abg::kScratchBytes);
  } else {
    if (kv_splits > 1 && !workspace) return fail(ABG_ERR_NULL, "workspace is NULL (kv_splits > 1)");
    if (kv_splits > 1 && workspace_bytes < ws_need)
      return fail(ABG_ERR_SHAPE, "workspace_bytes = %lld, need %lld", (long long)workspace_bytes,
                  (long long)ws_need);
  }
  // the merge of the partials runs one thread per 4 output values in a
  // one-dimensional grid of 256-thread workgroups
  if (kv_splits > 1 && B * Sq * Hq * (Dv / 4) > (int64_t)INT32_MAX * 256)
    return fail(ABG_ERR_SHAPE, "B * Sq = %lld query positions are too many for kv_splits > 1",
                (long long)(B * Sq));
  if (bias_group < 1 || bias_group > B)
    return fail(ABG_ERR_SHAPE, "%s_group = %lld must be in [1, B]", pair ? "pair" : "bias",
                (long long)bias_group);
  const int64_t P = (Sk + 15) / 16;  // compact bias cells per side
  if (pair) {
    // the projection inside the attention kernel: its fast path only
    if (!fast)
      return fail(ABG_ERR_UNSUPPORTED, "the pair form is implemented for ABG_BF16 with softcap > 0 only");
    if (C != 128) return fail(ABG_ERR_UNSUPPORTED, "C = %lld: only 128 pair channels are supported", (long long)C);
  }
  // per-item block of the bias (elements) or of the pair representation
  const int64_t bias_elems = pair ? P * P * C : Hq * P * P;
  if (bias_batch_stride < 0 || bias_batch_stride > (int64_t(1) << 40))
    return fail(ABG_ERR_SHAPE, "%s_batch_stride = %lld must be in [0, 2^40]", pair ? "pair" : "bias",
                (long long)bias_batch_stride);
  if (bias_batch_stride != 0 && bias_batch_stride < bias_elems)
    return fail(ABG_ERR_SHAPE, "%s_batch_stride = %lld must be 0 or >= %lld", pair ? "pair" : "bias",
                (long long)bias_batch_stride, (long long)bias_elems);
  if (bias_batch_stride % (pair ? 8 : 4) != 0)
    return fail(ABG_ERR_ALIGN, "%s_batch_stride must be a multiple of %d elements", pair ? "pair" : "bias",
                pair ? 8 : 4);
  const void* bsrc = pair ? pair : static_cast<const void*>(bias);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(bsrc) || !aligned16(out))
    return fail(ABG_ERR_ALIGN, "q, k, v, %s and out must be 16-byte aligned", pair ? "pair" : "bias");
  if (pair && !aligned16(weight)) return fail(ABG_ERR_ALIGN, "weight must be 16-byte aligned");
  if (kv_splits > 1 && !use_scratch && !aligned16(workspace))
    return fail(ABG_ERR_ALIGN, "workspace must be 16-byte aligned");
  const int64_t E = elem_bytes(dtype);
  const int64_t q_bytes = B * Sq * Hq * Dk * E;
  const int64_t kv_bytes = B * Sk * Dk * E;
  const int64_t n_bias = (B - 1) / bias_group + 1;
  const int64_t bias_bytes = ((n_bias - 1) * bias_batch_stride + bias_elems) * (pair ? 2 : 4);
  const int64_t w_bytes = pair ? C * Hq * 2 : 0;
  const int64_t out_bytes = B * Sq * Hq * Dv * E;
  if (overlaps(out, out_bytes, q, q_bytes)) return fail(ABG_ERR_ALIAS, "out overlaps q");
  if (overlaps(out, out_bytes, k, kv_bytes)) return fail(ABG_ERR_ALIAS, "out overlaps k");
  if (overlaps(out, out_bytes, v, B * Sk * Dv * E)) return fail(ABG_ERR_ALIAS, "out overlaps v");
  if (overlaps(out, out_bytes, bsrc, bias_bytes))
    return fail(ABG_ERR_ALIAS, "out overlaps %s", pair ? "pair" : "bias");
  if (pair && overlaps(out, out_bytes, weight, w_bytes)) return fail(ABG_ERR_ALIAS, "out overlaps weight");
  if (kv_splits > 1 && !use_scratch) {
    const void* ins[6] = {q, k, v, bsrc, out, weight};
    const int64_t sz[6] = {q_bytes, kv_bytes, B * Sk * Dv * E, bias_bytes, out_bytes, w_bytes};
    for (int i = 0; i < (pair ? 6 : 5); ++i)
      if (overlaps(workspace, ws_need, ins[i], sz[i]))
        return fail(ABG_ERR_ALIAS, "workspace overlaps an input or the output");
  }

  if (kv_splits > 1 && use_scratch) {
    // the scratch array's device address (never its host-side name)
    const abg_status st = device_status(abg::scratch_address(&workspace), "scratch address lookup");
    if (st != ABG_OK) return st;
  }
  abg::AttnLaunch a{q, k, v, bias, pair, weight, out, static_cast<float*>(workspace), B, Sq, Sk,
                    q_offset, Dv, bias_batch_stride, bias_group, kv_splits, scale, softcap, dtype};
  hipError_t e = abg::launch_biased_mqa_fwd(a, static_cast<hipStream_t>(stream));
  return device_status(e, "biased_mqa_fwd launch");
}

}  // namespace

extern "C" {

int abg_abi_version(void) { return ABG_ABI_VERSION; }

const char* abg_status_string(int status) {
  switch (status) {
    case ABG_OK: return "ABG_OK";
    case ABG_ERR_NULL: return "ABG_ERR_NULL";
    case ABG_ERR_SHAPE: return "ABG_ERR_SHAPE";
    case ABG_ERR_UNSUPPORTED: return "ABG_ERR_UNSUPPORTED";
    case ABG_ERR_ALIGN: return "ABG_ERR_ALIGN";
    case ABG_ERR_VALUE: return "ABG_ERR_VALUE";
    case ABG_ERR_ALIAS: return "ABG_ERR_ALIAS";
    case ABG_ERR_DEVICE: return "ABG_ERR_DEVICE";
    default: return "ABG_UNKNOWN_STATUS";
  }
}

const char* abg_last_error(void) { return g_last_error.c_str(); }

abg_status abg_pair_bias_project(const void* pair, const void* weight, float* bias,
                                 int64_t Bp, int64_t P, int64_t C, int64_t H,
                                 abg_dtype dtype, void* stream) {
  g_last_error.clear();
  if (dtype != ABG_F32 && dtype != ABG_BF16)
    return fail(ABG_ERR_VALUE, "dtype %d is not ABG_F32 or ABG_BF16", (int)dtype);
  if (!pair) return fail(ABG_ERR_NULL, "pair is NULL");
  if (!weight) return fail(ABG_ERR_NULL, "weight is NULL");
  if (!bias) return fail(ABG_ERR_NULL, "bias is NULL");
  if (Bp < 1) return fail(ABG_ERR_SHAPE, "Bp = %lld must be >= 1", (long long)Bp);
  if (P < 1 || P > 65536) return fail(ABG_ERR_SHAPE, "P = %lld must be in [1, 65536]", (long long)P);
  if (C < 8 || C > 512 || C % 8 != 0)
    return fail(ABG_ERR_UNSUPPORTED, "C = %lld must be a multiple of 8 in [8, 512]", (long long)C);
  if (H != 8) return fail(ABG_ERR_UNSUPPORTED, "H = %lld: only 8 heads are supported", (long long)H);
  if (Bp > (int64_t(1) << 40) / (P * P))
    return fail(ABG_ERR_SHAPE, "Bp * P * P is too large");
  if (!aligned16(pair)) return fail(ABG_ERR_ALIGN, "pair is not 16-byte aligned");
  if (!aligned16(weight)) return fail(ABG_ERR_ALIGN, "weight is not 16-byte aligned");
  if (!aligned16(bias)) return fail(ABG_ERR_ALIGN, "bias is not 16-byte aligned");
  const int64_t E = elem_bytes(dtype);
  const int64_t out_bytes = Bp * H * P * P * 4;
  if (overlaps(bias, out_bytes, pair, Bp * P * P * C * E))
    return fail(ABG_ERR_ALIAS, "bias overlaps pair");
  if (overlaps(bias, out_bytes, weight, C * H * E))
    return fail(ABG_ERR_ALIAS, "bias overlaps weight");
  hipError_t e = abg::launch_pair_bias_project(pair, weight, bias, Bp, P, C, dtype,
                                               static_cast<hipStream_t>(stream));
  return device_status(e, "pair_bias_project launch");
}

abg_status abg_biased_mqa_fwd(const void* q, const void* k, const void* v,
                              const float* bias, void* out,
                              int64_t B, int64_t S, int64_t Hq, int64_t Dk, int64_t Dv,
                              int64_t bias_batch_stride, int64_t bias_group,
                              float scale, float softcap,
                              abg_dtype dtype, void* stream) {
  return abg_biased_mqa_fwd_ex(q, k, v, bias, out, nullptr, 0, B, S, S, 0, Hq, Dk, Dv,
                               bias_batch_stride, bias_group, 1, scale, softcap, dtype, stream);
}

int64_t abg_biased_mqa_fwd_workspace_bytes(int64_t B, int64_t Sq, int64_t Hq, int64_t Dv,
                                           int64_t kv_splits) {
  if (B < 1 || Sq < 1 || Hq < 1 || Dv < 1 || kv_splits < 1 || kv_splits > 64) return -1;
  if (kv_splits == 1) return 0;
  // a product past int64 is out of range as well
  int64_t n = kv_splits;
  const int64_t f[5] = {B, Sq, Hq, Dv + 1, 4};
  for (int64_t x : f)
    if (__builtin_mul_overflow(n, x, &n)) return -1;
  return n;
}

abg_status abg_biased_mqa_fwd_ex(const void* q, const void* k, const void* v,
                                 const float* bias, void* out,
                                 void* workspace, int64_t workspace_bytes,
                                 int64_t B, int64_t Sq, int64_t Sk, int64_t q_offset,
                                 int64_t Hq, int64_t Dk, int64_t Dv,
                                 int64_t bias_batch_stride, int64_t bias_group,
                                 int64_t kv_splits, float scale, float softcap,
                                 abg_dtype dtype, void* stream) {
  g_last_error.clear();
  if (!bias) return fail(ABG_ERR_NULL, "bias is NULL");
  return attention(q, k, v, bias, nullptr, nullptr, 0, out, workspace, workspace_bytes, B, Sq, Sk,
                   q_offset, Hq, Dk, Dv, bias_batch_stride, bias_group, kv_splits, scale, softcap,
                   dtype, stream);
}

abg_status abg_biased_mqa_fwd_ex_noalloc(const void* q, const void* k, const void* v,
                                         const float* bias, void* out,
                                         int64_t B, int64_t Sq, int64_t Sk, int64_t q_offset,
                                         int64_t Hq, int64_t Dk, int64_t Dv,
                                         int64_t bias_batch_stride, int64_t bias_group,
                                         int64_t kv_splits, float scale, float softcap,
                                         abg_dtype dtype, void* stream) {
  g_last_error.clear();
  if (!bias) return fail(ABG_ERR_NULL, "bias is NULL");
  return attention(q, k, v, bias, nullptr, nullptr, 0, out, nullptr, 0, B, Sq, Sk, q_offset, Hq,
                   Dk, Dv, bias_batch_stride, bias_group, kv_splits, scale, softcap, dtype, stream,
                   true);
}

abg_status abg_pair_biased_mqa_fwd(const void* q, const void* k, const void* v,
                                   const void* pair, const void* weight, void* out,
                                   void* workspace, int64_t workspace_bytes,
                                   int64_t B, int64_t Sq, int64_t Sk, int64_t q_offset,
                                   int64_t Hq, int64_t Dk, int64_t Dv, int64_t C,
                                   int64_t pair_batch_stride, int64_t pair_group,
                                   int64_t kv_splits, float scale, float softcap,
                                   abg_dtype dtype, void* stream) {
  g_last_error.clear();
  if (!pair) return fail(ABG_ERR_NULL, "pair is NULL");
  if (!weight) return fail(ABG_ERR_NULL, "weight is NULL");
  return attention(q, k, v, nullptr, pair, weight, C, out, workspace, workspace_bytes, B, Sq, Sk,
                   q_offset, Hq, Dk, Dv, pair_batch_stride, pair_group, kv_splits, scale, softcap,
                   dtype, stream);
}

}  // extern "C"
