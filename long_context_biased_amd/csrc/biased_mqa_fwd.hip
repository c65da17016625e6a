// Fused biased, soft-capped multi-query attention forward for gfx950 (MI355X).
//
// Computes, for every batch item b, position i and query head h,
//   x_ij = scale * q_i.k_j + bias[h, i>>4, j>>4]
//   L_ij = cap * tanh(x_ij / cap)                 (cap > 0; cap == 0: L = x)
//   out_i = sum_j softmax_j(L_i.) v_j
// as described on the web page "Making Full-Context AlphaGenome Fit on an RTX
// 3090", section "Why stock FlashAttention was not a drop-in replacement"
// (logit equation, 8 query heads sharing one K/V head, bias cell per 16
// positions, BF16 products with FP32 accumulation), evaluated tile by tile as
// in section "Online softmax, one block at a time", so that neither the dense
// logits nor the dense repeated bias ever exist.
//
// Work decomposition (differs from the page's one-program-per-head kernel):
//   * one workgroup owns 32 query positions x all 8 heads = 256 query rows;
//     because K and V are shared by the heads, every K/V tile staged in LDS
//     serves all 8 heads at once;
//   * each wave owns HPW heads x 32 positions; lane (r = lane & 31,
//     g = lane >> 5) owns query row r of each of its heads;
//   * the score tile is computed transposed, S^T = K . Q^T, with the 32x32
//     MFMA: A = 32 keys x 16 dk from LDS, B = 16 dk x 32 query rows held in
//     registers for the whole kernel.  In the 32x32 accumulator layout lane
//     (r, g) then holds 16 scores of its own query row, so row sums need no
//     cross-lane traffic until the end, and the probabilities feed the PV
//     MFMA (O^T = V^T . P^T) as its B operand straight from registers.  The
//     keys loaded into A are permuted (bits 2 and 3 of the row swapped) so
//     that each lane's 8-value B fragment covers 8 consecutive keys;
//   * V is transposed into LDS (V^T, keys contiguous) while it is staged, so
//     the PV A operand is one 16-byte LDS read per lane;
//   * the compact bias cells of a tile (8 heads x 2 position cells x 4 key
//     cells) are staged with the tile, pre-multiplied by the exponent-domain
//     constant; the index (i>>4, j>>4) is fixed per lane and register;
//   * K/V/bias tiles are double-buffered in LDS with one barrier per tile; the
//     next tile's global loads are in flight while the current one computes.
//
// Soft-capped softmax (cap > 0): since |L| < cap, exp(L - cap) lies in
// (e^-2cap, 1] and can be used directly: the running maximum of the online
// recurrence is replaced by its upper bound cap, which is exact by the shift
// invariance of softmax and needs no rescaling.  With y = exp(2x/cap),
//   exp(L - cap) = exp(-2 cap / (1 + y))
// which costs exp2, fma, rcp, exp2 per logit with every constant folded.
// Without the cap the kernel keeps the running maximum and rescales (m, d, n)
// per tile exactly as in the update equations of the page.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "abg_internal.h"

namespace abg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kHeads = 8;      // query heads (one shared K/V head)
constexpr int kD = 128;        // head dim of Q/K and of V
constexpr int kTileKeys = 64;  // keys per LDS tile
constexpr int kBlockPos = 32;  // query positions per workgroup
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Element-type traits: a "fragment" is the 8 consecutive k-values one lane
// contributes to a 32x32 MFMA.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<__bf16> { using type = bf16x8; };
template <> struct Frag<float> { using type = f32x8; };

__device__ __forceinline__ void mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int m = 0; m < 8; ++m) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m], b[m], acc, 0, 0, 0);
}

// 16-byte loads/stores (the ABI guarantees 16-byte alignment only).
template <typename F>
__device__ __forceinline__ F load_frag(const char* p) {
  if constexpr (sizeof(F) == 16) {
    return *reinterpret_cast<const F*>(p);
  } else {
    uint4 lo = *reinterpret_cast<const uint4*>(p);
    uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
    F f;
    __builtin_memcpy(&f, &lo, 16);
    __builtin_memcpy(reinterpret_cast<char*>(&f) + 16, &hi, 16);
    return f;
  }
}

// Row permutation of the K operand: swap bits 2 and 3.
__device__ __forceinline__ int key_perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <typename T, int HPW, bool CAPPED>
struct Cfg {
  static constexpr int E = sizeof(T);
  static constexpr int NW = kHeads / HPW;        // waves per workgroup
  static constexpr int NT = 64 * NW;             // threads per workgroup
  static constexpr int K_ROW = kD * E;           // bytes per K row in LDS
  static constexpr int K_CHUNKS = K_ROW / 16;    // 16-B chunks per K row
  static constexpr int VT_ROW = kTileKeys * E;   // bytes per V^T row in LDS
  static constexpr int VT_CHUNKS = VT_ROW / 16;
  static constexpr int K_BYTES = kTileKeys * K_ROW;
  static constexpr int VT_BYTES = kD * VT_ROW;
  static constexpr int BIAS_OFF = K_BYTES + VT_BYTES;
  static constexpr int STAGE = BIAS_OFF + 256;   // 64 bias floats
  static constexpr int OUT_BYTES = kBlockPos * kHeads * kD * E;
  static constexpr int SMEM = (2 * STAGE > OUT_BYTES) ? 2 * STAGE : OUT_BYTES;
  static constexpr int K_PT = (kTileKeys * K_CHUNKS) / NT;  // K chunks per thread
  static constexpr int V_PT = 512 / NT;                     // 4x4 V units per thread
  using VRow = typename std::conditional<E == 2, uint2, uint4>::type;  // 4 elements
  static_assert(K_PT * NT == kTileKeys * K_CHUNKS, "K tile split");
  static_assert(V_PT * NT == 512, "V tile split");
};

template <typename T, int HPW, bool CAPPED>
__global__ __launch_bounds__(64 * (kHeads / HPW), 1)
void biased_mqa_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k,
                           const T* __restrict__ v, const float* __restrict__ bias,
                           T* __restrict__ out, int S, int64_t bias_batch_stride,
                           int bias_group, float alpha, float beta_mul, float den_a) {
  using C = Cfg<T, HPW, CAPPED>;
  using F = typename Frag<T>::type;
  constexpr int E = C::E;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 31;
  const int g = lane >> 5;
  const int b = blockIdx.y;
  const int pos0 = blockIdx.x * kBlockPos;
  const int P = S >> 4;
  const int n_tiles = S / kTileKeys;

  const char* kb_ptr = reinterpret_cast<const char*>(k + (int64_t)b * S * kD);
  const char* vb_ptr = reinterpret_cast<const char*>(v + (int64_t)b * S * kD);
  const float* bias_b = bias + (int64_t)(b / bias_group) * bias_batch_stride;

  // ---- Q fragments (B operand), held for the whole kernel -----------------
  F qf[HPW][kD / 16];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = wave * HPW + hh;
    const char* qrow = reinterpret_cast<const char*>(
        q + (((int64_t)b * S + pos0 + r) * kHeads + h) * kD);
#pragma unroll
    for (int kc = 0; kc < kD / 16; ++kc) qf[hh][kc] = load_frag<F>(qrow + (kc * 16 + 8 * g) * E);
  }

  // ---- tile staging: global -> registers -> LDS ---------------------------
  uint4 kreg[C::K_PT];
  typename C::VRow vreg[C::V_PT][4];
  float breg = 0.f;

  auto load_tile = [&](int t) {
    const char* kt = kb_ptr + (int64_t)t * kTileKeys * C::K_ROW;
#pragma unroll
    for (int i = 0; i < C::K_PT; ++i)
      kreg[i] = *reinterpret_cast<const uint4*>(kt + (tid + C::NT * i) * 16);
    const char* vt = vb_ptr + (int64_t)t * kTileKeys * kD * E;
#pragma unroll
    for (int i = 0; i < C::V_PT; ++i) {
      const int u = tid + C::NT * i;
      const int dvg = u & 31, kg = u >> 5;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vreg[i][e] = *reinterpret_cast<const typename C::VRow*>(
            vt + (int64_t)(kg * 4 + e) * kD * E + dvg * 4 * E);
    }
    if (tid < 64) {
      const int h = tid >> 3, pb = (tid >> 2) & 1, cell = tid & 3;
      breg = bias_b[((int64_t)h * P + (pos0 >> 4) + pb) * P + t * 4 + cell] * beta_mul;
    }
  };

  auto store_tile = [&](int stage) {
    char* st = smem + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::K_PT; ++i) {
      const int id = tid + C::NT * i;
      const int row = id / C::K_CHUNKS, c = id % C::K_CHUNKS;
      *reinterpret_cast<uint4*>(st + row * C::K_ROW + ((c ^ (row & (C::K_CHUNKS - 1))) * 16)) = kreg[i];
    }
    char* vtl = st + C::K_BYTES;
#pragma unroll
    for (int i = 0; i < C::V_PT; ++i) {
      const int u = tid + C::NT * i;
      const int dvg = u & 31, kg = u >> 5;
      const int byte = kg * 4 * E;             // key offset of this group in a V^T row
      const int chunk = byte >> 4, inb = byte & 15;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = dvg * 4 + e;
        char* dst = vtl + d * C::VT_ROW + ((chunk ^ (d & (C::VT_CHUNKS - 1))) * 16) + inb;
        if constexpr (E == 2) {
          // column e of the 4x4 block of bf16 (rows = keys)
          const uint32_t s0 = (e < 2) ? vreg[i][0].x : vreg[i][0].y;
          const uint32_t s1 = (e < 2) ? vreg[i][1].x : vreg[i][1].y;
          const uint32_t s2 = (e < 2) ? vreg[i][2].x : vreg[i][2].y;
          const uint32_t s3 = (e < 2) ? vreg[i][3].x : vreg[i][3].y;
          uint2 o;
          if ((e & 1) == 0) {
            o.x = (s0 & 0xffffu) | (s1 << 16);
            o.y = (s2 & 0xffffu) | (s3 << 16);
          } else {
            o.x = (s0 >> 16) | (s1 & 0xffff0000u);
            o.y = (s2 >> 16) | (s3 & 0xffff0000u);
          }
          *reinterpret_cast<uint2*>(dst) = o;
        } else {
          uint4 o;
          o.x = reinterpret_cast<const uint32_t*>(&vreg[i][0])[e];
          o.y = reinterpret_cast<const uint32_t*>(&vreg[i][1])[e];
          o.z = reinterpret_cast<const uint32_t*>(&vreg[i][2])[e];
          o.w = reinterpret_cast<const uint32_t*>(&vreg[i][3])[e];
          *reinterpret_cast<uint4*>(dst) = o;
        }
      }
    }
    if (tid < 64) reinterpret_cast<float*>(st + C::BIAS_OFF)[tid] = breg;
  };

  // ---- accumulators ----------------------------------------------------------
  f32x16 O[HPW][4];
  float rowsum[HPW];
  float mrun[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    rowsum[hh] = 0.f;
    mrun[hh] = -__builtin_inff();
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int x = 0; x < 16; ++x) O[hh][db][x] = 0.f;
  }

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const int kperm = key_perm(r);
  const int pb = r >> 4;  // position cell of this lane's query row within the block

  for (int t = 0; t < n_tiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const char* st = smem + cur * C::STAGE;
    const float* bl = reinterpret_cast<const float*>(st + C::BIAS_OFF);

    // ---- S^T = K . Q^T for two 32-key blocks -------------------------------
    f32x16 Sacc[HPW][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
        for (int x = 0; x < 16; ++x) Sacc[hh][kb][x] = 0.f;
      const int row = kb * 32 + kperm;
      const char* krow = st + row * C::K_ROW;
#pragma unroll
      for (int kc = 0; kc < kD / 16; ++kc) {
        F a;
        if constexpr (E == 2) {
          const int c = 2 * kc + g;
          a = *reinterpret_cast<const F*>(krow + ((c ^ (row & (C::K_CHUNKS - 1))) * 16));
        } else {
          const int c = 4 * kc + 2 * g;
          uint4 lo = *reinterpret_cast<const uint4*>(krow + ((c ^ (row & (C::K_CHUNKS - 1))) * 16));
          uint4 hi = *reinterpret_cast<const uint4*>(krow + (((c + 1) ^ (row & (C::K_CHUNKS - 1))) * 16));
          __builtin_memcpy(&a, &lo, 16);
          __builtin_memcpy(reinterpret_cast<char*>(&a) + 16, &hi, 16);
        }
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) mfma(Sacc[hh][kb], a, qf[hh][kc]);
      }
    }

    // ---- bias, soft-cap, softmax weights --------------------------------------
    F pf[HPW][4];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = wave * HPW + hh;
      const float* brow = bl + h * 8 + pb * 4;
      float pv[2][16];
      if constexpr (CAPPED) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const float beta = brow[kb * 2 + (x >> 3)];
            const float t2 = __builtin_fmaf(Sacc[hh][kb][x], alpha, beta);
            const float y = __builtin_amdgcn_exp2f(t2);
            const float dd = __builtin_fmaf(y, den_a, den_a);
            pv[kb][x] = __builtin_amdgcn_exp2f(__builtin_amdgcn_rcpf(dd));
          }
      } else {
        float u[2][16];
        float mt = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            u[kb][x] = __builtin_fmaf(Sacc[hh][kb][x], alpha, brow[kb * 2 + (x >> 3)]);
            mt = __builtin_fmaxf(mt, u[kb][x]);
          }
        mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
        const float mnew = __builtin_fmaxf(mrun[hh], mt);
        const float sc = __builtin_amdgcn_exp2f(mrun[hh] - mnew);
        mrun[hh] = mnew;
        rowsum[hh] *= sc;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int x = 0; x < 16; ++x) O[hh][db][x] *= sc;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int x = 0; x < 16; ++x) pv[kb][x] = __builtin_amdgcn_exp2f(u[kb][x] - mnew);
      }
      // pack to the PV B operand; the row sum uses the values that PV uses
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          F f;
#pragma unroll
          for (int m = 0; m < 8; ++m) f[m] = static_cast<T>(pv[kb][8 * half + m]);
          pf[hh][2 * kb + half] = f;
          if constexpr (E == 2) {
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int m = 0; m < 8; m += 2) {
              bf16x2 pr = {f[m], f[m + 1]};
              rowsum[hh] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rowsum[hh], false);
            }
          } else {
#pragma unroll
            for (int m = 0; m < 8; ++m) rowsum[hh] += f[m];
          }
        }
    }

    // ---- O^T += V^T . P^T ---------------------------------------------------------
    const char* vtl = st + C::K_BYTES;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + r;
      const char* vrow = vtl + d * C::VT_ROW;
#pragma unroll
      for (int kc2 = 0; kc2 < 4; ++kc2) {
        F a;
        if constexpr (E == 2) {
          const int c = 2 * kc2 + g;
          a = *reinterpret_cast<const F*>(vrow + ((c ^ (d & (C::VT_CHUNKS - 1))) * 16));
        } else {
          const int c = 4 * kc2 + 2 * g;
          uint4 lo = *reinterpret_cast<const uint4*>(vrow + ((c ^ (d & (C::VT_CHUNKS - 1))) * 16));
          uint4 hi = *reinterpret_cast<const uint4*>(vrow + (((c + 1) ^ (d & (C::VT_CHUNKS - 1))) * 16));
          __builtin_memcpy(&a, &lo, 16);
          __builtin_memcpy(reinterpret_cast<char*>(&a) + 16, &hi, 16);
        }
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) mfma(O[hh][db], a, pf[hh][kc2]);
      }
    }

    if (t + 1 < n_tiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / rowsum, stage in LDS, coalesced store -------------------------
  constexpr int OUT_ROW = kHeads * kD * E;  // bytes per query position
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = wave * HPW + hh;
    const float tot = rowsum[hh] + __shfl_xor(rowsum[hh], 32);
    const float inv = 1.0f / tot;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dv = db * 32 + 8 * j + 4 * g;
        const int byte = (h * kD + dv) * E;
        const int chunk = byte >> 4, inb = byte & 15;
        char* dst = smem + r * OUT_ROW + ((chunk ^ r) * 16) + inb;
        if constexpr (E == 2) {
          bf16x2 lo = {(__bf16)(O[hh][db][4 * j + 0] * inv), (__bf16)(O[hh][db][4 * j + 1] * inv)};
          bf16x2 hi = {(__bf16)(O[hh][db][4 * j + 2] * inv), (__bf16)(O[hh][db][4 * j + 3] * inv)};
          uint2 w;
          __builtin_memcpy(&w.x, &lo, 4);
          __builtin_memcpy(&w.y, &hi, 4);
          *reinterpret_cast<uint2*>(dst) = w;
        } else {
          float4 w = make_float4(O[hh][db][4 * j + 0] * inv, O[hh][db][4 * j + 1] * inv,
                                 O[hh][db][4 * j + 2] * inv, O[hh][db][4 * j + 3] * inv);
          *reinterpret_cast<float4*>(dst) = w;
        }
      }
  }
  __syncthreads();
  char* ob = reinterpret_cast<char*>(out + ((int64_t)b * S + pos0) * kHeads * kD);
  constexpr int CHUNKS_PER_POS = OUT_ROW / 16;
  constexpr int TOTAL = kBlockPos * CHUNKS_PER_POS;
#pragma unroll
  for (int i = 0; i < TOTAL / C::NT; ++i) {
    const int id = tid + C::NT * i;
    const int rr = id / CHUNKS_PER_POS, c = id % CHUNKS_PER_POS;
    *reinterpret_cast<uint4*>(ob + (int64_t)id * 16) =
        *reinterpret_cast<const uint4*>(smem + rr * OUT_ROW + ((c ^ rr) * 16));
  }
}

template <typename T, int HPW, bool CAPPED>
hipError_t launch_typed(const AttnLaunch& a, hipStream_t stream) {
  using C = Cfg<T, HPW, CAPPED>;
  float alpha, beta_mul, den_a;
  if (CAPPED) {
    // exponent of y = exp(2x/cap) in base 2: (2 log2 e / cap) * x
    beta_mul = 2.0f * kLog2e / a.softcap;
    alpha = a.scale * beta_mul;
    den_a = -1.0f / (2.0f * a.softcap * kLog2e);
  } else {
    beta_mul = kLog2e;
    alpha = a.scale * kLog2e;
    den_a = 0.f;
  }
  dim3 grid((unsigned)(a.S / kBlockPos), (unsigned)a.B);
  hipLaunchKernelGGL((biased_mqa_fwd_kernel<T, HPW, CAPPED>), grid, dim3(C::NT), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), a.bias, static_cast<T*>(a.out), (int)a.S,
                     a.bias_batch_stride, (int)a.bias_group, alpha, beta_mul, den_a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_biased_mqa_fwd(const AttnLaunch& a, hipStream_t stream) {
  const bool capped = a.softcap > 0.f;
  if (a.dtype == ABG_BF16) {
    return capped ? launch_typed<__bf16, 2, true>(a, stream)
                  : launch_typed<__bf16, 2, false>(a, stream);
  }
  return capped ? launch_typed<float, 1, true>(a, stream)
                : launch_typed<float, 1, false>(a, stream);
}

}  // namespace abg
