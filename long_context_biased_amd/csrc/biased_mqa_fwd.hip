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
//   * one workgroup owns 32 query positions x all 8 heads = 256 query rows,
//     one wave per head (8 waves, 2 per SIMD).  K and V are shared by the
//     heads, so every K/V tile staged in LDS serves all 8 heads at once;
//   * lane (r = lane & 31, g = lane >> 5) of a wave owns query row r;
//   * scores are computed transposed, S^T = K . Q^T, with the 32x32x16 MFMA:
//     A = 32 keys x 16 dk from LDS, B = 16 dk x 32 query rows held in
//     registers for the whole kernel.  In the 32x32 accumulator layout lane
//     (r, g) then holds 16 scores of its own query row, so row sums need no
//     cross-lane traffic until the end, and the probabilities feed the PV
//     MFMA (O^T = V^T . P^T) as its B operand straight from registers.  The
//     keys loaded into A are permuted (bits 2 and 3 of the row swapped) so
//     that each lane's 8-value B fragment covers 8 consecutive keys;
//   * V is transposed into LDS (V^T, keys contiguous) while it is staged, so
//     a PV A operand is one 16-byte LDS read per lane;
//   * the compact bias cells of a tile (8 heads x 2 position cells x 4 key
//     cells) are staged with the tile, pre-multiplied by the exponent-domain
//     constant; the index (i>>4, j>>4) is fixed per lane and register;
//   * software pipeline: a 64-key tile is two 32-key halves.  Each stage
//     issues 16 MFMAs (PV of one half + QK^T of the next tile's half) and, in
//     between, the soft-cap/softmax VALU chain of another half, so the matrix
//     cores and the VALU work at the same time inside one wave; the second
//     wave on the SIMD fills the remaining gaps;
//   * LDS tiles are triple-buffered for bf16 (one barrier per tile) and
//     double-buffered for float32 (two barriers per tile, LDS budget); the
//     global loads of tile t+3 are in flight while tile t computes.
//
// Soft-capped softmax (cap > 0): since |L| < cap, exp(L - cap) lies in
// (e^-2cap, 1] and can be used directly: the running maximum of the online
// recurrence is replaced by its upper bound cap, which is exact by the shift
// invariance of softmax and needs no rescaling.  With y = exp(2x/cap),
//   exp(L - cap) = exp(-2 cap / (1 + y))
// which costs exp2, fma, rcp, exp2 per logit with every constant folded.
// Without the cap the kernel keeps the running maximum and rescales (m, d, n)
// per 32-key half exactly as in the update equations of the page.
// The row sum adds the probabilities as rounded for the PV product.

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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeads = 8;      // query heads (one shared K/V head)
constexpr int kD = 128;        // head dim of Q/K and of V
constexpr int kTileKeys = 64;  // keys per LDS tile
constexpr int kBlockPos = 32;  // query positions per workgroup
constexpr int kThreads = 64 * kHeads;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Traits;
template <> struct Traits<__bf16> {
  using F = bf16x8;   // 8 consecutive k-values of one lane for a 32x32 MFMA
  using VRow = u32x2; // 4 V elements
  static constexpr int NBUF = 3;
};
template <> struct Traits<float> {
  using F = f32x8;
  using VRow = u32x4;
  static constexpr int NBUF = 2;
};

template <typename T>
struct Lay {
  static constexpr int E = sizeof(T);
  static constexpr int K_ROW = kD * E;           // bytes per K row in LDS
  static constexpr int K_CHUNKS = K_ROW / 16;    // 16-B chunks per K row
  static constexpr int VT_ROW = kTileKeys * E;   // bytes per V^T row in LDS
  static constexpr int VT_CHUNKS = VT_ROW / 16;
  static constexpr int K_BYTES = kTileKeys * K_ROW;
  static constexpr int VT_BYTES = kD * VT_ROW;
  static constexpr int BIAS_OFF = K_BYTES + VT_BYTES;
  static constexpr int STAGE = BIAS_OFF + 256;   // + 64 bias floats
  static constexpr int NBUF = Traits<T>::NBUF;
  static constexpr int OUT_ROW = kHeads * kD * E;  // output bytes per position
  static constexpr int OUT_BYTES = kBlockPos * OUT_ROW;
  static constexpr int SMEM = (NBUF * STAGE > OUT_BYTES) ? NBUF * STAGE : OUT_BYTES;
  static constexpr int K_PT = (kTileKeys * K_CHUNKS) / kThreads;  // K chunks per thread
  static_assert(K_PT * kThreads == kTileKeys * K_CHUNKS, "K tile split");
  static_assert(kThreads == 512, "one 4x4 V block per thread");
};

__device__ __forceinline__ void mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int m = 0; m < 8; ++m) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m], b[m], acc, 0, 0, 0);
}

// A fragment of 8 consecutive elements at byte offset `off` of LDS; float32
// fragments are two 16-byte chunks (c, c ^ 1 after the swizzle).
template <typename T>
__device__ __forceinline__ typename Traits<T>::F lds_frag(const char* base, int off0, int off1) {
  using F = typename Traits<T>::F;
  if constexpr (sizeof(T) == 2) {
    (void)off1;
    return *reinterpret_cast<const F*>(base + off0);
  } else {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + off0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + off1);
    F f;
    __builtin_memcpy(&f, &lo, 16);
    __builtin_memcpy(reinterpret_cast<char*>(&f) + 16, &hi, 16);
    return f;
  }
}

// Row permutation of the K operand: swap bits 2 and 3.
__device__ __forceinline__ int key_perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// One tile's global data held in registers between its load and its LDS store.
template <typename T>
struct Staged {
  u32x4 k[Lay<T>::K_PT];
  typename Traits<T>::VRow v[4];
  float bias;
};

// Per-thread addresses of the staging copy (loop invariant).
template <typename T>
struct StageAddr {
  int k_lds[Lay<T>::K_PT];
  int v_glb;       // bytes from the tile base to this thread's first V row
  int v_lds[4];    // V^T destinations of the 4 columns of the 4x4 block
  int64_t b_glb;   // element offset of this thread's bias cell (tile 0)
};

template <typename T>
__device__ __forceinline__ void load_tile(Staged<T>& st, const StageAddr<T>& ad, const char* kb,
                                          const char* vb, const float* bias_b, int t, int tid,
                                          float beta_mul) {
  using L = Lay<T>;
  const char* kt = kb + (int64_t)t * kTileKeys * L::K_ROW;
#pragma unroll
  for (int i = 0; i < L::K_PT; ++i)
    st.k[i] = *reinterpret_cast<const u32x4*>(kt + (tid + kThreads * i) * 16);
  const char* vt = vb + (int64_t)t * kTileKeys * kD * L::E + ad.v_glb;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    st.v[e] = *reinterpret_cast<const typename Traits<T>::VRow*>(vt + e * kD * L::E);
  if (tid < 64) st.bias = bias_b[ad.b_glb + t * 4] * beta_mul;
}

template <typename T>
__device__ __forceinline__ void store_tile(const Staged<T>& st, const StageAddr<T>& ad, char* buf,
                                           int tid) {
  using L = Lay<T>;
#pragma unroll
  for (int i = 0; i < L::K_PT; ++i) *reinterpret_cast<u32x4*>(buf + ad.k_lds[i]) = st.k[i];
  // 4x4 block (rows = 4 keys, columns = 4 value channels) -> 4 rows of V^T
  if constexpr (L::E == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t s0 = (e < 2) ? st.v[0].x : st.v[0].y;
      const uint32_t s1 = (e < 2) ? st.v[1].x : st.v[1].y;
      const uint32_t s2 = (e < 2) ? st.v[2].x : st.v[2].y;
      const uint32_t s3 = (e < 2) ? st.v[3].x : st.v[3].y;
      u32x2 o;
      if ((e & 1) == 0) {
        o.x = __builtin_amdgcn_perm(s1, s0, 0x05040100u);  // lo halves
        o.y = __builtin_amdgcn_perm(s3, s2, 0x05040100u);
      } else {
        o.x = __builtin_amdgcn_perm(s1, s0, 0x07060302u);  // hi halves
        o.y = __builtin_amdgcn_perm(s3, s2, 0x07060302u);
      }
      *reinterpret_cast<u32x2*>(buf + ad.v_lds[e]) = o;
    }
  } else {
    *reinterpret_cast<u32x4*>(buf + ad.v_lds[0]) = u32x4{st.v[0].x, st.v[1].x, st.v[2].x, st.v[3].x};
    *reinterpret_cast<u32x4*>(buf + ad.v_lds[1]) = u32x4{st.v[0].y, st.v[1].y, st.v[2].y, st.v[3].y};
    *reinterpret_cast<u32x4*>(buf + ad.v_lds[2]) = u32x4{st.v[0].z, st.v[1].z, st.v[2].z, st.v[3].z};
    *reinterpret_cast<u32x4*>(buf + ad.v_lds[3]) = u32x4{st.v[0].w, st.v[1].w, st.v[2].w, st.v[3].w};
  }
  if (tid < 64) reinterpret_cast<float*>(buf + L::BIAS_OFF)[tid] = st.bias;
}

// S^T (32 keys of half kb) x (32 query rows) = K . Q^T
template <typename T>
__device__ __forceinline__ f32x16 qk_half(const char* buf, const int (&k_off)[2][8][2],
                                          const typename Traits<T>::F (&qf)[kD / 16], int kb) {
  f32x16 s = {};
#pragma unroll
  for (int kc = 0; kc < kD / 16; ++kc) {
    const auto a = lds_frag<T>(buf, k_off[kb][kc][0], k_off[kb][kc][1]);
    mfma(s, a, qf[kc]);
  }
  return s;
}

// O^T += V^T (keys of half kb) . P^T
template <typename T>
__device__ __forceinline__ void pv_half(const char* buf, const int (&v_off)[4][4][2],
                                        const typename Traits<T>::F (&p)[2], f32x16 (&O)[4],
                                        int kb) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kc2 = 2 * kb + half;
      const auto a = lds_frag<T>(buf, v_off[db][kc2][0], v_off[db][kc2][1]);
      mfma(O[db], a, p[half]);
    }
}

// Soft-capped weights exp(L - cap) of 16 scores (key cells beta.x for x < 8,
// beta.y for x >= 8), packed as the PV operand; the row sum adds the packed
// values.
template <typename T>
__device__ __forceinline__ void softmax_capped(const f32x16& s, f32x2 beta, float alpha,
                                               float den_a, float& rowsum,
                                               typename Traits<T>::F (&p)[2]) {
  float w[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const float t2 = __builtin_fmaf(s[x], alpha, x < 8 ? beta.x : beta.y);
    const float y = __builtin_amdgcn_exp2f(t2);
    const float d = __builtin_fmaf(y, den_a, den_a);
    w[x] = __builtin_amdgcn_exp2f(__builtin_amdgcn_rcpf(d));
  }
  if constexpr (sizeof(T) == 2) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x2 pr[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x2 two = {w[8 * half + 2 * m], w[8 * half + 2 * m + 1]};
        pr[m] = __builtin_convertvector(two, bf16x2);
        rowsum = __builtin_amdgcn_fdot2_f32_bf16(pr[m], ones, rowsum, false);
      }
      bf16x8 f;
      __builtin_memcpy(&f, pr, 16);
      p[half] = f;
    }
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x8 f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        f[m] = w[8 * half + m];
        rowsum += w[8 * half + m];
      }
      p[half] = f;
    }
  }
}

// Uncapped online softmax of one 32-key half: returns the factor by which the
// running numerator must be rescaled.
template <typename T>
__device__ __forceinline__ float softmax_online(const f32x16& s, f32x2 beta, float alpha,
                                                float& mrun, float& rowsum,
                                                typename Traits<T>::F (&p)[2]) {
  float u[16];
  float mt = -__builtin_inff();
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    u[x] = __builtin_fmaf(s[x], alpha, x < 8 ? beta.x : beta.y);
    mt = __builtin_fmaxf(mt, u[x]);
  }
  mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
  const float mnew = __builtin_fmaxf(mrun, mt);
  const float sc = __builtin_amdgcn_exp2f(mrun - mnew);
  mrun = mnew;
  rowsum *= sc;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    typename Traits<T>::F f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const T pv = static_cast<T>(__builtin_amdgcn_exp2f(u[8 * half + m] - mnew));
      f[m] = pv;
      rowsum += static_cast<float>(pv);
    }
    p[half] = f;
  }
  return sc;
}

template <typename T, bool CAPPED>
__device__ __forceinline__ void softmax_half(const f32x16& s, f32x2 beta, float alpha, float den_a,
                                             float& mrun, float& rowsum, f32x16 (&O)[4],
                                             typename Traits<T>::F (&p)[2]) {
  if constexpr (CAPPED) {
    (void)mrun;
    (void)O;
    softmax_capped<T>(s, beta, alpha, den_a, rowsum, p);
  } else {
    (void)den_a;
    const float sc = softmax_online<T>(s, beta, alpha, mrun, rowsum, p);
#pragma unroll
    for (int db = 0; db < 4; ++db) O[db] *= sc;
  }
}

template <typename T, bool CAPPED>
__global__ __launch_bounds__(kThreads, 1)
void biased_mqa_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k,
                           const T* __restrict__ v, const float* __restrict__ bias,
                           T* __restrict__ out, int S, int64_t bias_batch_stride,
                           int bias_group, float alpha, float beta_mul, float den_a) {
  using L = Lay<T>;
  using F = typename Traits<T>::F;
  constexpr int E = L::E;
  constexpr int NBUF = L::NBUF;
  __shared__ __attribute__((aligned(16))) char smem[L::SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int h = tid >> 6;  // wave = head
  const int r = lane & 31;
  const int g = lane >> 5;
  const int b = blockIdx.y;
  const int pos0 = blockIdx.x * kBlockPos;
  const int P = S >> 4;
  const int n = S / kTileKeys;

  const char* kb_ptr = reinterpret_cast<const char*>(k + (int64_t)b * S * kD);
  const char* vb_ptr = reinterpret_cast<const char*>(v + (int64_t)b * S * kD);
  const float* bias_b = bias + (int64_t)(b / bias_group) * bias_batch_stride;

  // ---- Q fragments (B operand), held for the whole kernel -----------------
  F qf[kD / 16];
  {
    const char* qrow = reinterpret_cast<const char*>(q + (((int64_t)b * S + pos0 + r) * kHeads + h) * kD);
#pragma unroll
    for (int kc = 0; kc < kD / 16; ++kc) {
      const char* p = qrow + (kc * 16 + 8 * g) * E;
      if constexpr (E == 2) {
        qf[kc] = *reinterpret_cast<const F*>(p);
      } else {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
        __builtin_memcpy(&qf[kc], &lo, 16);
        __builtin_memcpy(reinterpret_cast<char*>(&qf[kc]) + 16, &hi, 16);
      }
    }
  }

  // ---- loop-invariant addresses -----------------------------------------------
  StageAddr<T> ad;
#pragma unroll
  for (int i = 0; i < L::K_PT; ++i) {
    const int id = tid + kThreads * i;
    const int row = id / L::K_CHUNKS, c = id % L::K_CHUNKS;
    ad.k_lds[i] = row * L::K_ROW + ((c ^ (row & (L::K_CHUNKS - 1))) * 16);
  }
  {
    const int dvg = tid & 31, kg = tid >> 5;  // 4x4 block: keys 4kg.., channels 4dvg..
    ad.v_glb = (kg * 4) * kD * E + dvg * 4 * E;
    const int byte = kg * 4 * E;
    const int chunk = byte >> 4, inb = byte & 15;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = dvg * 4 + e;
      ad.v_lds[e] = L::K_BYTES + d * L::VT_ROW + ((chunk ^ (d & (L::VT_CHUNKS - 1))) * 16) + inb;
    }
    const int bh = tid >> 3, pb = (tid >> 2) & 1, cell = tid & 3;
    ad.b_glb = ((int64_t)bh * P + (pos0 >> 4) + pb) * P + cell;
  }
  int k_off[2][8][2];
  {
    const int kp = key_perm(r);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = kb * 32 + kp;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const int c = (E == 2) ? (2 * kc + g) : (4 * kc + 2 * g);
        k_off[kb][kc][0] = row * L::K_ROW + ((c ^ (row & (L::K_CHUNKS - 1))) * 16);
        k_off[kb][kc][1] = row * L::K_ROW + (((c + 1) ^ (row & (L::K_CHUNKS - 1))) * 16);
      }
    }
  }
  int v_off[4][4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = db * 32 + r;
#pragma unroll
    for (int kc2 = 0; kc2 < 4; ++kc2) {
      const int c = (E == 2) ? (2 * kc2 + g) : (4 * kc2 + 2 * g);
      v_off[db][kc2][0] = L::K_BYTES + d * L::VT_ROW + ((c ^ (d & (L::VT_CHUNKS - 1))) * 16);
      v_off[db][kc2][1] = L::K_BYTES + d * L::VT_ROW + (((c + 1) ^ (d & (L::VT_CHUNKS - 1))) * 16);
    }
  }
  // bias cells of this lane's row: [h][pb][4 key cells] inside a staged tile
  const int bias_lds = L::BIAS_OFF + (h * 8 + (r >> 4) * 4) * 4;

  // ---- accumulators ----------------------------------------------------------
  f32x16 O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x16{};
  float rowsum = 0.f;
  float mrun = -__builtin_inff();

  // ---- prologue -----------------------------------------------------------------
  Staged<T> st;
  load_tile<T>(st, ad, kb_ptr, vb_ptr, bias_b, 0, tid, beta_mul);
  store_tile<T>(st, ad, smem, tid);
  if (n > 1) {
    load_tile<T>(st, ad, kb_ptr, vb_ptr, bias_b, 1, tid, beta_mul);
    store_tile<T>(st, ad, smem + L::STAGE, tid);
  }
  if (n > 2) load_tile<T>(st, ad, kb_ptr, vb_ptr, bias_b, 2, tid, beta_mul);
  __syncthreads();

  f32x16 S0 = qk_half<T>(smem, k_off, qf, 0);
  f32x16 S1 = qk_half<T>(smem, k_off, qf, 1);
  F P0[2], P1[2];
  {
    const f32x2 beta = *reinterpret_cast<const f32x2*>(smem + bias_lds);
    softmax_half<T, CAPPED>(S0, beta, alpha, den_a, mrun, rowsum, O, P0);
  }

  int cur = 0;  // buffer of tile t
  for (int t = 0; t < n; ++t) {
    const int nxt = (cur + 1 == NBUF) ? 0 : cur + 1;
    const bool has_next = t + 1 < n;
    const char* bcur = smem + cur * L::STAGE;
    const char* bnxt = smem + nxt * L::STAGE;
    if constexpr (NBUF == 3) {
      if (t + 2 < n) {
        const int b2 = (nxt + 1 == NBUF) ? 0 : nxt + 1;
        store_tile<T>(st, ad, smem + b2 * L::STAGE, tid);
        if (t + 3 < n) load_tile<T>(st, ad, kb_ptr, vb_ptr, bias_b, t + 3, tid, beta_mul);
      }
    }
    // Stage X: PV(t, half 0) + QK(t+1, half 0) || softmax(t, half 1)
    pv_half<T>(bcur, v_off, P0, O, 0);
    if (has_next) S0 = qk_half<T>(bnxt, k_off, qf, 0);
    {
      const f32x2 beta = *reinterpret_cast<const f32x2*>(bcur + bias_lds + 8);
      softmax_half<T, CAPPED>(S1, beta, alpha, den_a, mrun, rowsum, O, P1);
    }
    // Stage Y: PV(t, half 1) + QK(t+1, half 1) || softmax(t+1, half 0)
    pv_half<T>(bcur, v_off, P1, O, 1);
    if (has_next) {
      S1 = qk_half<T>(bnxt, k_off, qf, 1);
      const f32x2 beta = *reinterpret_cast<const f32x2*>(bnxt + bias_lds);
      softmax_half<T, CAPPED>(S0, beta, alpha, den_a, mrun, rowsum, O, P0);
    }
    if constexpr (NBUF == 2) {
      __syncthreads();  // every wave is done with tile t
      if (t + 2 < n) {
        store_tile<T>(st, ad, smem + cur * L::STAGE, tid);
        if (t + 3 < n) load_tile<T>(st, ad, kb_ptr, vb_ptr, bias_b, t + 3, tid, beta_mul);
      }
    }
    __syncthreads();
    cur = nxt;
  }

  // ---- epilogue: O / rowsum, stage in LDS, coalesced store -------------------------
  const float tot = rowsum + __shfl_xor(rowsum, 32);
  const float inv = 1.0f / tot;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dv = db * 32 + 8 * j + 4 * g;
      const int byte = (h * kD + dv) * E;
      const int chunk = byte >> 4, inb = byte & 15;
      char* dst = smem + r * L::OUT_ROW + ((chunk ^ r) * 16) + inb;
      if constexpr (E == 2) {
        const f32x2 a = {O[db][4 * j + 0] * inv, O[db][4 * j + 1] * inv};
        const f32x2 c = {O[db][4 * j + 2] * inv, O[db][4 * j + 3] * inv};
        bf16x2 lo = __builtin_convertvector(a, bf16x2);
        bf16x2 hi = __builtin_convertvector(c, bf16x2);
        u32x2 w;
        w.x = __builtin_bit_cast(unsigned int, lo);
        w.y = __builtin_bit_cast(unsigned int, hi);
        *reinterpret_cast<u32x2*>(dst) = w;
      } else {
        const f32x4 w = {O[db][4 * j + 0] * inv, O[db][4 * j + 1] * inv,
                         O[db][4 * j + 2] * inv, O[db][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(dst) = w;
      }
    }
  __syncthreads();
  char* ob = reinterpret_cast<char*>(out + ((int64_t)b * S + pos0) * kHeads * kD);
  constexpr int CHUNKS_PER_POS = L::OUT_ROW / 16;
  constexpr int TOTAL = kBlockPos * CHUNKS_PER_POS;
#pragma unroll
  for (int i = 0; i < TOTAL / kThreads; ++i) {
    const int id = tid + kThreads * i;
    const int rr = id / CHUNKS_PER_POS, c = id % CHUNKS_PER_POS;
    *reinterpret_cast<u32x4*>(ob + (int64_t)id * 16) =
        *reinterpret_cast<const u32x4*>(smem + rr * L::OUT_ROW + ((c ^ rr) * 16));
  }
}

template <typename T, bool CAPPED>
hipError_t launch_typed(const AttnLaunch& a, hipStream_t stream) {
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
  hipLaunchKernelGGL((biased_mqa_fwd_kernel<T, CAPPED>), grid, dim3(kThreads), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), a.bias, static_cast<T*>(a.out), (int)a.S,
                     a.bias_batch_stride, (int)a.bias_group, alpha, beta_mul, den_a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_biased_mqa_fwd(const AttnLaunch& a, hipStream_t stream) {
  const bool capped = a.softcap > 0.f;
  if (a.dtype == ABG_BF16)
    return capped ? launch_typed<__bf16, true>(a, stream) : launch_typed<__bf16, false>(a, stream);
  return capped ? launch_typed<float, true>(a, stream) : launch_typed<float, false>(a, stream);
}

}  // namespace abg
