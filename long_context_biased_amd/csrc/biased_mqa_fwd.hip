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
//     keys loaded into A are permuted (bits 2 and 3 of the row swapped; the
//     permutation is applied when K is staged in LDS) so that each lane's
//     8-value B fragment covers 8 consecutive keys;
//   * tiles are staged in LDS in one of two ways.  The generic kernel
//     (float32) stages through registers: V is transposed into
//     LDS (V^T, keys contiguous) so a PV A operand is one 16-byte LDS read
//     per lane; LDS rows are padded by 16 bytes (K: 272 B, V^T: 144 B for
//     bf16) so the 32 rows read by a half-wave fall in distinct banks; the
//     compact bias cells of a tile (8 heads x 2 position cells x 4 key
//     cells) are staged with it, pre-multiplied by the exponent-domain
//     constant, and the index (i>>4, j>>4) is fixed per lane and register.
//     The bf16 kernel (with or without the cap) copies HBM straight to LDS, keeps V
//     row-major and reads it transposed, and brings the bias in either as
//     the soft-cap's fma multiplier (compact bias with the cap) or as the
//     start of each QK^T accumulator (the pair form, and without the cap;
//     see the block comment of that path);
//   * software pipeline: a 64-key tile is two 32-key halves.  Each stage
//     issues 16 MFMAs (PV of one half + QK^T of the next tile's half) and,
//     woven between them, the soft-cap/softmax chain of another half, so the
//     matrix cores and the VALU work at the same time inside one wave; the
//     second wave on the SIMD fills the remaining gaps.  For bf16 the
//     order is fixed by hand: 16 slots of {LDS read three MFMAs ahead, one
//     MFMA, five softmax micro-ops (three without the cap)}, the softmax written as a
//     skewed pipeline over its 16 values so dependent operations are far
//     apart;
//   * LDS tiles are triple-buffered for bf16 (one barrier per tile) and
//     double-buffered for float32 (two barriers per tile, LDS budget); the
//     global loads of later tiles are in flight while tile t computes.
//
// Soft-capped softmax (cap > 0): since |L| < cap, exp(L - cap) lies in
// (e^-2cap, 1] and can be used directly: the running maximum of the online
// recurrence is replaced by its upper bound cap, which is exact by the shift
// invariance of softmax and needs no rescaling.  With y = exp(2x/cap),
//   exp(L - cap) = exp(-2 cap / (1 + y))
// which costs exp2, fma, rcp, exp2 per logit with every constant folded.
// Without the cap the kernels keep the running maximum of the update
// equations of the page: the generic kernel rescales (m, d, n) per 32-key
// half; the bf16 kernel moves its reference maximum only when a row
// outgrows it by 2^8 (update_ref).
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeads = 8;      // query heads (one shared K/V head)
constexpr int kD = 128;        // head dim of Q/K and of V
constexpr int kTileKeys = 64;  // keys per LDS tile
constexpr int kBlockPos = 32;  // query positions per workgroup
constexpr int kThreads = 64 * kHeads;
constexpr float kLog2e = 1.4426950408889634f;
// Heads per wave of the bf16 soft-capped kernel.  1 (built): eight waves, two
// per SIMD.  2: four waves, one per SIMD, each LDS fragment feeding two
// MFMAs; it compiles, spills a few registers and runs about a third slower
// (one wave per SIMD cannot hide the softmax's latencies).
#ifndef ABG_FAST_HPW
#define ABG_FAST_HPW 1
#endif
constexpr int kFastHeadsPerWave = ABG_FAST_HPW;

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
  static constexpr int K_ROW = kD * E;            // payload bytes per K row
  static constexpr int K_STRIDE = K_ROW + 16;     // padded row pitch in LDS
  static constexpr int K_CHUNKS = K_ROW / 16;     // 16-B chunks per K row
  static constexpr int VT_ROW = kTileKeys * E;    // payload bytes per V^T row
  static constexpr int VT_STRIDE = VT_ROW + 16;
  static constexpr int K_BYTES = kTileKeys * K_STRIDE;
  static constexpr int VT_BYTES = kD * VT_STRIDE;
  static constexpr int BIAS_OFF = K_BYTES + VT_BYTES;
  static constexpr int STAGE = BIAS_OFF + 256;    // + 64 bias floats
  static constexpr int NBUF = Traits<T>::NBUF;
  static constexpr int OUT_ROW = kHeads * kD * E; // output bytes per position
  static constexpr int OUT_BYTES = kBlockPos * OUT_ROW;
  static constexpr int SMEM = (NBUF * STAGE > OUT_BYTES) ? NBUF * STAGE : OUT_BYTES;
  static constexpr int K_PT = (kTileKeys * K_CHUNKS) / kThreads;  // K chunks per thread
  static constexpr int K_ROWS_PER_PASS = kThreads / K_CHUNKS;
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

// 8 consecutive elements at byte offset `off` of LDS.
template <typename T>
__device__ __forceinline__ typename Traits<T>::F lds_frag(const char* base, int off) {
  using F = typename Traits<T>::F;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const F*>(base + off);
  } else {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + off);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + off + 16);
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
struct StageAddr {
  int k_lds;       // LDS byte offset of this thread's first K chunk
  int v_glb;       // bytes from the V tile base to this thread's first V row
  int v_lds;       // LDS byte offset of the first V^T row of this thread's block
  int64_t b_glb;   // element offset of this thread's bias cell (tile 0)
  // for sequences that end inside a tile: key rows are clamped to the last
  // one, key cells to the last cell
  int k_row;       // key row (within a tile) of this thread's first K chunk
  int k_cb;        // byte offset of that chunk within its row
  int v_row;       // first of the 4 key rows of this thread's V block
  int v_cb;        // byte offset of its 4 value channels within a row
  int64_t b_row;   // element offset of this thread's bias row (cell 0)
  int b_cell;      // key cell of this thread within a tile
};

// TAIL: the sequence may end inside tile t (S keys, P cells); rows and cells
// past the end read the last ones, so the stage holds finite data there.
template <typename T, bool TAIL>
__device__ __forceinline__ void load_tile(Staged<T>& st, const StageAddr& ad, const char* kb,
                                          const char* vb, const float* bias_b, int t, int tid,
                                          float beta_mul, int S, int P) {
  using L = Lay<T>;
  if constexpr (TAIL) {
    // 32-bit byte offsets from the item's base: S <= 2^18 rows of at most
    // 512 bytes
    const int key0 = t * kTileKeys;
#pragma unroll
    for (int i = 0; i < L::K_PT; ++i) {
      const int key = min(key0 + ad.k_row + i * L::K_ROWS_PER_PASS, S - 1);
      st.k[i] = *reinterpret_cast<const u32x4*>(kb + (uint32_t)(key * L::K_ROW + ad.k_cb));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = min(key0 + ad.v_row + e, S - 1);
      st.v[e] = *reinterpret_cast<const typename Traits<T>::VRow*>(
          vb + (uint32_t)(key * kD * L::E + ad.v_cb));
    }
    st.bias = bias_b[ad.b_row + min(t * 4 + ad.b_cell, P - 1)] * beta_mul;
  } else {
    (void)S;
    (void)P;
    const char* kt = kb + (int64_t)t * kTileKeys * L::K_ROW;
#pragma unroll
    for (int i = 0; i < L::K_PT; ++i)
      st.k[i] = *reinterpret_cast<const u32x4*>(kt + (tid + kThreads * i) * 16);
    const char* vt = vb + (int64_t)t * kTileKeys * kD * L::E + ad.v_glb;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      st.v[e] = *reinterpret_cast<const typename Traits<T>::VRow*>(vt + e * kD * L::E);
    st.bias = bias_b[ad.b_glb + t * 4] * beta_mul;
  }
}

template <typename T>
__device__ __forceinline__ void store_tile(const Staged<T>& st, const StageAddr& ad, char* buf,
                                           int tid) {
  using L = Lay<T>;
#pragma unroll
  for (int i = 0; i < L::K_PT; ++i)
    *reinterpret_cast<u32x4*>(buf + ad.k_lds + i * L::K_ROWS_PER_PASS * L::K_STRIDE) = st.k[i];
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
      *reinterpret_cast<u32x2*>(buf + ad.v_lds + e * L::VT_STRIDE) = o;
    }
  } else {
    *reinterpret_cast<u32x4*>(buf + ad.v_lds + 0 * L::VT_STRIDE) = u32x4{st.v[0].x, st.v[1].x, st.v[2].x, st.v[3].x};
    *reinterpret_cast<u32x4*>(buf + ad.v_lds + 1 * L::VT_STRIDE) = u32x4{st.v[0].y, st.v[1].y, st.v[2].y, st.v[3].y};
    *reinterpret_cast<u32x4*>(buf + ad.v_lds + 2 * L::VT_STRIDE) = u32x4{st.v[0].z, st.v[1].z, st.v[2].z, st.v[3].z};
    *reinterpret_cast<u32x4*>(buf + ad.v_lds + 3 * L::VT_STRIDE) = u32x4{st.v[0].w, st.v[1].w, st.v[2].w, st.v[3].w};
  }
  // every wave writes the same 64 cells (same values): no branch in the loop
  reinterpret_cast<float*>(buf + L::BIAS_OFF)[tid & 63] = st.bias;
}

// S^T (32 keys of half kb) x (32 query rows) = K . Q^T.  `kbase` = this lane's
// K fragment base inside a stage.
template <typename T>
__device__ __forceinline__ f32x16 qk_half(const char* buf, int kbase,
                                          const typename Traits<T>::F (&qf)[kD / 16], int kb) {
  using L = Lay<T>;
  f32x16 s = {};
#pragma unroll
  for (int kc = 0; kc < kD / 16; ++kc)
    mfma(s, lds_frag<T>(buf, kbase + kb * 32 * L::K_STRIDE + kc * 16 * L::E), qf[kc]);
  return s;
}

// O^T += V^T (keys of half kb) . P^T.  `vbase` = this lane's V^T fragment base.
template <typename T>
__device__ __forceinline__ void pv_half(const char* buf, int vbase,
                                        const typename Traits<T>::F (&p)[2], f32x16 (&O)[4],
                                        int kb) {
  using L = Lay<T>;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kc2 = 2 * kb + half;
      mfma(O[db], lds_frag<T>(buf, vbase + db * 32 * L::VT_STRIDE + kc2 * 16 * L::E), p[half]);
    }
}

// Keys past the end of the sequence get p = 0.  A lane (g = lane >> 5)
// holds, for one 32-key half of a tile, 8 packed probability pairs; pair m
// covers keys 16 (m >> 2) + 8 g + 2 (m & 3) and the next one, counted from the
// half's first key.  `k` is that offset without the 8 g term and `lim` the
// number of keys of the sequence from the half's first key on, less 8 g.
// The low 16 bits of a pair hold its first key.
__device__ __forceinline__ int lane_g() { return (int)(threadIdx.x >> 5) & 1; }
__device__ __forceinline__ bf16x2 mask_pair(bf16x2 p, int k, int lim) {
  const uint32_t u = __builtin_bit_cast(uint32_t, p);
  return __builtin_bit_cast(bf16x2, k + 1 < lim ? u : (k < lim ? (u & 0xFFFFu) : 0u));
}

// Soft-capped weights exp(L - cap) of 16 scores (key cells beta.x for x < 8,
// beta.y for x >= 8), packed as the PV operand; the row sum adds the packed
// values.
// Value x of a lane holds key 16 (x >> 3) + 8 g + (x & 7) of the half; with
// MASK, keys at or past `lim` (counted from the half's first key, less 8 g)
// get weight 0.
template <typename T, bool MASK>
__device__ __forceinline__ void softmax_capped(const f32x16& s, f32x2 beta, float alpha,
                                               float den_a, float& rowsum,
                                               typename Traits<T>::F (&p)[2], int lim) {
  float w[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const float t2 = __builtin_fmaf(s[x], alpha, x < 8 ? beta.x : beta.y);
    const float y = __builtin_amdgcn_exp2f(t2);
    const float d = __builtin_fmaf(y, den_a, den_a);
    w[x] = __builtin_amdgcn_exp2f(__builtin_amdgcn_rcpf(d));
    if constexpr (MASK) w[x] = 16 * (x >> 3) + (x & 7) < lim ? w[x] : 0.f;
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
// With MASK, keys past the end (as in softmax_capped) get exponent -inf:
// weight 0, and no part in the maximum.  The row's first half always holds
// key 0, so the running maximum is finite from the first half on.
template <typename T, bool MASK>
__device__ __forceinline__ float softmax_online(const f32x16& s, f32x2 beta, float alpha,
                                                float& mrun, float& rowsum,
                                                typename Traits<T>::F (&p)[2], int lim) {
  float u[16];
  float mt = -__builtin_inff();
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    u[x] = __builtin_fmaf(s[x], alpha, x < 8 ? beta.x : beta.y);
    if constexpr (MASK) u[x] = 16 * (x >> 3) + (x & 7) < lim ? u[x] : -__builtin_inff();
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

template <typename T, bool CAPPED, bool MASK>
__device__ __forceinline__ void softmax_half(const f32x16& s, f32x2 beta, float alpha, float den_a,
                                             float& mrun, float& rowsum, f32x16 (&O)[4],
                                             typename Traits<T>::F (&p)[2], int lim) {
  if constexpr (CAPPED) {
    (void)mrun;
    (void)O;
    softmax_capped<T, MASK>(s, beta, alpha, den_a, rowsum, p, lim);
  } else {
    (void)den_a;
    const float sc = softmax_online<T, MASK>(s, beta, alpha, mrun, rowsum, p, lim);
#pragma unroll
    for (int db = 0; db < 4; ++db) O[db] *= sc;
  }
}

// ---------------------------------------------------------------------------
// Fixed-order stage for bf16 with the cap.
//
// Softmax micro-operations of one 32-key half (16 values per lane).  The
// scores arrive as exponents t (Q pre-scaled by alpha), and A is the fma's
// multiplier: with the compact bias t = alpha s (the accumulator started from
// zero) and the bias cell enters as A = a 2^beta (cap_multiplier); in the
// pair form t = alpha s + beta (the accumulator started from the expanded
// offsets) and A = a:
//   pass 1: y = exp2(t)   2: d = fma(y, A, a)   3: r = rcp(d)   4: w = exp2(r)
//   pass 5: pack pair k to bf16       6: row sum += the packed pair
// issued as a skewed pipeline: at step tau, pass p works on value
// tau - 3 (p - 1), and pair k is packed two steps after its second value is
// done.
// ---------------------------------------------------------------------------
struct SmOp { int pass, idx; };
// NP arithmetic passes per value (with the cap 4: exp2, fma, rcp, exp2;
// without it 2: subtract the reference maximum, exp2), then 8 packs and 8
// sums: 16 NP + 16 micro-ops.
template <int NP>
struct SmTable {
  static constexpr int N = 16 * NP + 16;
  SmOp op[N];
};
template <int NP>
constexpr SmTable<NP> make_sm_table() {
  SmTable<NP> t{};
  int n = 0;
  constexpr int lag = 3, fe = (NP - 1) * lag + 3;
  for (int tau = 0; n < SmTable<NP>::N; ++tau) {
    for (int p = 1; p <= NP; ++p) {
      const int x = tau - (p - 1) * lag;
      if (x >= 0 && x < 16) t.op[n++] = SmOp{p, x};
    }
    if (tau >= fe && (tau - fe) % 2 == 0 && (tau - fe) / 2 < 8) t.op[n++] = SmOp{5, (tau - fe) / 2};
    if (tau >= fe + 1 && (tau - fe - 1) % 2 == 0 && (tau - fe - 1) / 2 < 8)
      t.op[n++] = SmOp{6, (tau - fe - 1) / 2};
  }
  return t;
}
constexpr SmTable<4> kSm = make_sm_table<4>();
constexpr SmTable<2> kSmU = make_sm_table<2>();
constexpr int kSmOps = SmTable<4>::N;   // 80
constexpr int kSmOpsU = SmTable<2>::N;  // 48

struct SmState {
  float v[16];
  bf16x2 pk[8];
};

__device__ __forceinline__ void sm_op(int pass, int x, SmState& st, const f32x16& s, float den_a,
                                      f32x2 am, float& rowsum) {
  switch (pass) {
    case 1: st.v[x] = __builtin_amdgcn_exp2f(s[x]); break;
    case 2: st.v[x] = __builtin_fmaf(st.v[x], x < 8 ? am.x : am.y, den_a); break;
    case 3: st.v[x] = __builtin_amdgcn_rcpf(st.v[x]); break;
    case 4: st.v[x] = __builtin_amdgcn_exp2f(st.v[x]); break;
    case 5: {
      const f32x2 two = {st.v[2 * x], st.v[2 * x + 1]};
      st.pk[x] = __builtin_convertvector(two, bf16x2);
      break;
    }
    default: {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      rowsum = __builtin_amdgcn_fdot2_f32_bf16(st.pk[x], ones, rowsum, false);
      break;
    }
  }
}

// O / rowsum -> output dtype, staged through LDS (XOR-swizzled 16-byte
// chunks) so the 32 positions x 8 heads x DV block, contiguous in HBM, is
// written with coalesced 16-byte stores.  The caller has passed a barrier
// after the last read of the tile buffers, and another between the staging
// and the copy.
template <typename T, int DV = kD>
__device__ __forceinline__ void stage_output(char* smem, const f32x16 (&O)[DV / 32], float rowsum,
                                             int r, int g, int h) {
  constexpr int E = sizeof(T);
  constexpr int OUT_ROW = kHeads * DV * E;
  const float tot = rowsum + __shfl_xor(rowsum, 32);
  const float inv = 1.0f / tot;
#pragma unroll
  for (int db = 0; db < DV / 32; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dv = db * 32 + 8 * j + 4 * g;
      const int byte = (h * DV + dv) * E;
      const int chunk = byte >> 4, inb = byte & 15;
      char* dst = smem + r * OUT_ROW + ((chunk ^ r) * 16) + inb;
      if constexpr (E == 2) {
        const f32x2 a = {O[db][4 * j + 0] * inv, O[db][4 * j + 1] * inv};
        const f32x2 c = {O[db][4 * j + 2] * inv, O[db][4 * j + 3] * inv};
        u32x2 w;
        w.x = __builtin_bit_cast(unsigned int, __builtin_convertvector(a, bf16x2));
        w.y = __builtin_bit_cast(unsigned int, __builtin_convertvector(c, bf16x2));
        *reinterpret_cast<u32x2*>(dst) = w;
      } else {
        const f32x4 w = {O[db][4 * j + 0] * inv, O[db][4 * j + 1] * inv,
                         O[db][4 * j + 2] * inv, O[db][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(dst) = w;
      }
    }
}

template <typename T, int NT, int DV = kD>
__device__ __forceinline__ void copy_output(const char* smem, T* __restrict__ out_block, int tid,
                                            int valid_rows = kBlockPos) {
  constexpr int OUT_ROW = kHeads * DV * sizeof(T);
  char* ob = reinterpret_cast<char*>(out_block);
  constexpr int CHUNKS_PER_POS = OUT_ROW / 16;
  constexpr int TOTAL = kBlockPos * CHUNKS_PER_POS;
#pragma unroll
  for (int i = 0; i < TOTAL / NT; ++i) {
    const int id = tid + NT * i;
    const int rr = id / CHUNKS_PER_POS, c = id % CHUNKS_PER_POS;
    if (rr < valid_rows)
      *reinterpret_cast<u32x4*>(ob + (int64_t)id * 16) =
          *reinterpret_cast<const u32x4*>(smem + rr * OUT_ROW + ((c ^ rr) * 16));
  }
}

// TAIL: S need not be a multiple of the 64-key tile nor Sq of the 32-query
// block.  Key rows and cells past the end are clamped when staged and their
// weights masked to 0; query rows past Sq read row Sq - 1 and are not stored.
// SPLIT: workgroup z of the grid takes key tiles [z n, z n + n) (n =
// tiles_per_split) and writes its partial state to the workspace instead of
// the output, for merge_partials_kernel: with the cap the numerator rows and
// the denominators (the maximum is the fixed cap); without it the normalised
// rows n / d and log2 d + m (m the running maximum, base 2).
template <typename T, bool CAPPED, bool TAIL, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1)
void biased_mqa_fwd_kernel(const T* __restrict__ q, const T* __restrict__ k,
                           const T* __restrict__ v, const float* __restrict__ bias,
                           T* __restrict__ out, float* __restrict__ ws, int Sq, int S,
                           int q_offset, int tiles_per_split, int64_t bias_batch_stride,
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
  const int qpos0 = blockIdx.x * kBlockPos;  // first row of this block in q / out
  const int pos0 = q_offset + qpos0;         // its position in the sequence
  const int P = (S + 15) >> 4;
  // this workgroup's key tiles: t0 .. last (tile indices in the sequence)
  const int t0 = SPLIT ? (int)blockIdx.z * tiles_per_split : 0;
  const int last = SPLIT ? t0 + tiles_per_split - 1 : (S + kTileKeys - 1) / kTileKeys - 1;
  // keys of the sequence from a half's first key on, less 8 g, is
  // lim0 - (that key's index)
  const int lim0 = S - 8 * g;

  const char* kb_ptr = reinterpret_cast<const char*>(k + (int64_t)b * S * kD);
  const char* vb_ptr = reinterpret_cast<const char*>(v + (int64_t)b * S * kD);
  const float* bias_b = bias + (int64_t)(b / bias_group) * bias_batch_stride;

  // ---- Q fragments (B operand), held for the whole kernel -----------------
  F qf[kD / 16];
  {
    const int qi = TAIL ? min(qpos0 + r, Sq - 1) : qpos0 + r;
    const char* qrow = reinterpret_cast<const char*>(q + (((int64_t)b * Sq + qi) * kHeads + h) * kD);
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
  StageAddr ad;
  {
    // K rows are stored permuted (LDS row kb*32 + rho holds key kb*32 +
    // key_perm(rho)), so the 8 lanes of an LDS read phase read 8 consecutive
    // padded rows: distinct banks.
    const int key = tid / L::K_CHUNKS;
    const int row = (key & ~31) | key_perm(key & 31);
    ad.k_lds = row * L::K_STRIDE + (tid % L::K_CHUNKS) * 16;
    ad.k_row = key;
    ad.k_cb = (tid % L::K_CHUNKS) * 16;
  }
  {
    // 4x4 block: keys 4kg.., channels 4dvg..; lanes run over kg first so the
    // transposed stores of a write phase hit distinct banks.
    const int lane6 = tid & 63, w = tid >> 6;
    const int kg = (lane6 & 7) | ((w & 1) << 3);
    const int dvg = ((lane6 >> 3) & 7) | ((w >> 1) << 3);
    ad.v_glb = (kg * 4) * kD * E + dvg * 4 * E;
    ad.v_lds = L::K_BYTES + (dvg * 4) * L::VT_STRIDE + kg * 4 * E;
    ad.v_row = kg * 4;
    ad.v_cb = dvg * 4 * E;
    const int bt = tid & 63;
    const int bh = bt >> 3, pb = (bt >> 2) & 1, cell = bt & 3;
    ad.b_glb = ((int64_t)bh * P + (pos0 >> 4) + pb) * P + cell;
    ad.b_row = ((int64_t)bh * P + min((pos0 >> 4) + pb, P - 1)) * P;
    ad.b_cell = cell;
  }
  // per-lane A fragment bases inside a stage (lane r reads LDS row r, which
  // holds key key_perm(r) of the 32-key half)
  const int kbase = r * L::K_STRIDE + 8 * g * E;
  const int vbase = L::K_BYTES + r * L::VT_STRIDE + 8 * g * E;
  // bias cells of this lane's row: [h][pb][4 key cells] inside a staged tile
  const int bias_lds = L::BIAS_OFF + (h * 8 + (r >> 4) * 4) * 4;

  // ---- accumulators ----------------------------------------------------------
  f32x16 O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x16{};
  float rowsum = 0.f;
  float mrun = -__builtin_inff();

  // ---- prologue -----------------------------------------------------------------
  // Tile indices past the range are clamped to its last tile: the extra
  // loads and stores go to a buffer nobody reads, and the loop body stays one
  // basic block for the instruction scheduler.
  Staged<T> st;
  load_tile<T, TAIL>(st, ad, kb_ptr, vb_ptr, bias_b, t0, tid, beta_mul, S, P);
  store_tile<T>(st, ad, smem, tid);
  load_tile<T, TAIL>(st, ad, kb_ptr, vb_ptr, bias_b, min(t0 + 1, last), tid, beta_mul, S, P);
  store_tile<T>(st, ad, smem + L::STAGE, tid);
  load_tile<T, TAIL>(st, ad, kb_ptr, vb_ptr, bias_b, min(t0 + 2, last), tid, beta_mul, S, P);
  __syncthreads();

  f32x16 S0 = qk_half<T>(smem, kbase, qf, 0);
  f32x16 S1 = qk_half<T>(smem, kbase, qf, 1);
  F P0[2], P1[2];
  {
    const f32x2 beta = *reinterpret_cast<const f32x2*>(smem + bias_lds);
    softmax_half<T, CAPPED, TAIL>(S0, beta, alpha, den_a, mrun, rowsum, O, P0,
                                  lim0 - t0 * kTileKeys);
  }

  int cur = 0;  // buffer of tile t
  {
    for (int t = t0; t < last; ++t) {
      const int nxt = (cur + 1 == NBUF) ? 0 : cur + 1;
      const char* bcur = smem + cur * L::STAGE;
      const char* bnxt = smem + nxt * L::STAGE;
      if constexpr (NBUF == 3) {
        const int nn = (nxt + 1 == NBUF) ? 0 : nxt + 1;
        store_tile<T>(st, ad, smem + nn * L::STAGE, tid);
        load_tile<T, TAIL>(st, ad, kb_ptr, vb_ptr, bias_b, min(t + 3, last), tid, beta_mul, S, P);
      }
      // X: PV(t, half 0) + QK(t+1, half 0) || softmax(t, half 1)
      pv_half<T>(bcur, vbase, P0, O, 0);
      S0 = qk_half<T>(bnxt, kbase, qf, 0);
      {
        const f32x2 beta = *reinterpret_cast<const f32x2*>(bcur + bias_lds + 8);
        softmax_half<T, CAPPED, TAIL>(S1, beta, alpha, den_a, mrun, rowsum, O, P1,
                                      lim0 - t * kTileKeys - 32);
      }
      // Y: PV(t, half 1) + QK(t+1, half 1) || softmax(t+1, half 0)
      pv_half<T>(bcur, vbase, P1, O, 1);
      S1 = qk_half<T>(bnxt, kbase, qf, 1);
      {
        const f32x2 beta = *reinterpret_cast<const f32x2*>(bnxt + bias_lds);
        softmax_half<T, CAPPED, TAIL>(S0, beta, alpha, den_a, mrun, rowsum, O, P0,
                                      lim0 - (t + 1) * kTileKeys);
      }
      if constexpr (NBUF == 2) {
        __syncthreads();  // every wave is done with tile t: its buffer is free
        store_tile<T>(st, ad, smem + cur * L::STAGE, tid);
        load_tile<T, TAIL>(st, ad, kb_ptr, vb_ptr, bias_b, min(t + 3, last), tid, beta_mul, S, P);
      }
      __syncthreads();
      cur = nxt;
    }
  }
  // last tile: PV of both halves and the softmax of its second half
  {
    const char* bcur = smem + cur * L::STAGE;
    pv_half<T>(bcur, vbase, P0, O, 0);
    const f32x2 beta = *reinterpret_cast<const f32x2*>(bcur + bias_lds + 8);
    softmax_half<T, CAPPED, TAIL>(S1, beta, alpha, den_a, mrun, rowsum, O, P1,
                                  lim0 - last * kTileKeys - 32);
    pv_half<T>(bcur, vbase, P1, O, 1);
  }
  if constexpr (SPLIT) {
    // partial rows [split][b][pos][h][128] and per-row values [split][b][pos][h],
    // float32; lane (r, g) holds channels 32 db + 8 j + 4 g .. + 3 of its row
    const int64_t rows = (int64_t)gridDim.y * Sq * kHeads;
    const int64_t row = ((int64_t)blockIdx.z * gridDim.y + b) * Sq * kHeads +
                        (int64_t)(qpos0 + r) * kHeads + h;
    const float tot = rowsum + __shfl_xor(rowsum, 32);
    if (!TAIL || qpos0 + r < Sq) {
      // uncapped: store n / d and the row's log2-sum-exp, so that the merge
      // needs no numerator scaling per range
      const float inv = CAPPED ? 1.0f : 1.0f / tot;
      float* nrow = ws + row * kD + 4 * g;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 x = {O[db][4 * j] * inv, O[db][4 * j + 1] * inv, O[db][4 * j + 2] * inv,
                           O[db][4 * j + 3] * inv};
          *reinterpret_cast<f32x4*>(nrow + 32 * db + 8 * j) = x;
        }
      if (g == 0) ws[(int64_t)gridDim.z * rows * kD + row] = CAPPED ? tot : mrun + __builtin_amdgcn_logf(tot);
    }
  } else {
    (void)ws;
    __syncthreads();  // the output staging below reuses the tile buffers
    stage_output<T>(smem, O, rowsum, r, g, h);
    __syncthreads();
    copy_output<T, kThreads>(smem, out + ((int64_t)b * Sq + qpos0) * kHeads * kD, tid,
                             TAIL ? min(kBlockPos, Sq - qpos0) : kBlockPos);
  }
}

// ===========================================================================
// gfx950 path for bf16 inputs with the cap.
//
// LDS (bytes, value width 128): V tiles at s * 16 KiB (s = 0..2), K tiles at
// 48 KiB + s * 16 KiB, bias cells at 96 KiB + s * 256, pair vectors (when the
// bias is projected in the kernel) at 96.75 KiB + s * 2 KiB, exponent
// offsets expanded to the accumulator layout at 102.75 KiB + s * 2 KiB.
// The softmax exponent comes out of the MFMA: Q is scaled by the exponent
// factor when it is loaded.  With the compact bias and the cap each lane
// reads its own cell of the tile and scales the soft-cap's fma by it
// (cap_multiplier), the accumulator starting from zero; in the pair form and
// without the cap each QK^T accumulator starts from the tile's expanded
// offsets (bias x exponent factor), written one iteration ahead by the wave
// that reads them.  Tiles arrive straight from HBM with
// global_load_lds_dwordx4 (16 bytes per lane, no register staging); each lane
// fetches the chunk that belongs at its LDS slot, which applies the layouts:
//   * K: LDS row kb*32 + rho holds key kb*32 + key_perm(rho); its 16-byte
//     chunk c sits at c ^ (row & 15), so the 16 lanes of an LDS read phase
//     (16 consecutive rows, same chunk) hit distinct banks;
//   * V: row-major as in HBM, 32-byte slot u of key row j at
//     u ^ (j & 3) ^ ((u & 1) << 2).
//     The PV A operand (8 consecutive keys of one value channel) comes from
//     two ds_read_b64_tr_b16: in each 16-lane group, lane a + 4k returns
//     element b of its 8 bytes to lane 4a + b as element k, so lane s reading
//     key row s/4, channels 4(s%4).. delivers 4 keys of one channel per lane;
//     the 4 rows x 32 bytes of a group land in distinct banks, and the two
//     groups of a half-wave (odd and even slots) in different bank halves.
// The main loop is unrolled three times so every LDS address is a
// loop-invariant register plus an immediate offset.
// ===========================================================================
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// LDS layout for value width DV (128 or 192).
template <int DV>
struct FP {
  static constexpr int NBUF = 3;
  static constexpr int NPV = DV / 32;               // 32-channel blocks of V
  static constexpr int KROW = kD * 2;               // bytes per K row
  static constexpr int KTILE = kTileKeys * KROW;    // 16 KiB
  static constexpr int VROW = DV * 2;               // bytes per V row
  static constexpr int VTILE = kTileKeys * VROW;    // 16 or 24 KiB
  static constexpr int V0 = 0;
  static constexpr int K0 = NBUF * VTILE;
  static constexpr int B0 = K0 + NBUF * KTILE;
  // pair vectors of one tile when the bias is projected in the kernel: 2
  // query cells x 4 key cells x 128 channels, bf16
  static constexpr int PTILE = 2 * 4 * 128 * 2;
  static constexpr int PR0 = B0 + NBUF * 256;
  // exponent offsets of one tile expanded to the accumulator layout: per head,
  // half and query cell the 16 values a lane adds to its QK^T accumulator
  // (8 x key cell 2 half, 8 x key cell 2 half + 1), float
  static constexpr int XBS = kHeads * 2 * 2 * 16 * 4;
  static constexpr int XB0 = PR0 + NBUF * PTILE;
  static constexpr int SMEM = XB0 + NBUF * XBS;
  static_assert(SMEM >= kBlockPos * kHeads * DV * 2, "output staging fits in the tile buffers");
};

// MFMA order inside a stage (NPV = DV / 32 blocks of value channels):
// The same without the cap: pass 1 subtracts the row's reference maximum
// (base-2 exponents), pass 2 takes exp2; packs and sums as above.
__device__ __forceinline__ void sm_op_u(int pass, int x, SmState& st, const f32x16& s, float mref,
                                        float& rowsum) {
  switch (pass) {
    case 1: st.v[x] = s[x] - mref; break;
    case 2: st.v[x] = __builtin_amdgcn_exp2f(st.v[x]); break;
    case 5: {
      const f32x2 two = {st.v[2 * x], st.v[2 * x + 1]};
      st.pk[x] = __builtin_convertvector(two, bf16x2);
      break;
    }
    default: {
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      rowsum = __builtin_amdgcn_fdot2_f32_bf16(st.pk[x], ones, rowsum, false);
      break;
    }
  }
}

// The values of lanes l and l ^ 32 of x, in every lane l (in either order).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; given two copies of x they come out as
// (x[0..31], x[0..31]) and (x[32..63], x[32..63]).  Written out here: through
// the compiler's builtin, this toolchain hands back the first result in place
// of the second (both results came out equal on gfx950), which would drop
// the other half's value.  The nops keep the instruction's distance from the
// VALU writes of its operands.
__device__ __forceinline__ f32x2 swap_halves(float x) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
#pragma clang diagnostic pop
  return f32x2{__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)};
}

// Running maximum without the cap (the page's online update, base 2): the
// maximum of a row over the 32 keys of a half (16 exponents in this lane,
// 16 in lane l ^ 32).  The reference moves only when some row of the wave
// exceeds it by more than 8, so weights stay below 2^8 (exact enough in
// bf16, far from overflow) and the accumulators are rescaled rarely; f is
// the factor for what was accumulated against the old reference (1 when it
// stays).  Returns whether the wave moved its reference (uniform).
__device__ __forceinline__ bool update_ref(const f32x16& s, float& mref, float& f) {
  const float a0 = fmaxf(fmaxf(s[0], s[1]), s[2]), a1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
  const float a2 = fmaxf(fmaxf(s[6], s[7]), s[8]), a3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
  const float a4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
  const float m = fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), s[15]));
  const f32x2 sw = swap_halves(m);
  const float mh = fmaxf(sw.x, sw.y);
  const bool any = __builtin_amdgcn_ballot_w64(mh > mref + 8.f) != 0;
  const float mn = any ? fmaxf(mref, mh) : mref;
  f = __builtin_amdgcn_exp2f(mref - mn);
  mref = mn;
  return any;
}

// PV(db 0..2, half 0), QK(kc 0..7), PV(db 3..NPV-1, half 0), PV(db 0..NPV-1,
// half 1) -- 8 + 2 NPV slots.  The QK^T chain ends mid-stage, long before the
// next stage's softmax reads it, and the first three MFMAs read V only.
__device__ __forceinline__ constexpr bool slot_is_qk(int j) { return j >= 3 && j <= 10; }
__device__ __forceinline__ constexpr int slot_kc(int j) { return j - 3; }
template <int NPV>
__device__ __forceinline__ constexpr int slot_db(int j) {
  return j < 3 ? j : (j < 8 + NPV ? j - 8 : j - 8 - NPV);
}
template <int NPV>
__device__ __forceinline__ constexpr int slot_half(int j) { return j < 8 + NPV ? 0 : 1; }
// The softmax micro-ops of a stage spread over its slots: as evenly as
// possible, the first slots taking one more.
template <int NSLOT, int NOPS = kSmOps>
__device__ __forceinline__ constexpr int sm_count(int j) {
  return NOPS / NSLOT + (j < NOPS % NSLOT ? 1 : 0);
}
template <int NSLOT, int NOPS = kSmOps>
__device__ __forceinline__ constexpr int sm_begin(int j) {
  return j * (NOPS / NSLOT) + (j < NOPS % NSLOT ? j : NOPS % NSLOT);
}

// V rows in LDS are row-major as in HBM, in 32-byte slots (16 channels)
// permuted per row.  DV = 128 (8 slots): slot u of row j sits at
// u ^ (j & 3) ^ ((u & 1) << 2).  DV = 192 (12 slots, rows 384 bytes so row j
// starts in bank half j & 1): slot u sits at u ^ (j & 2), which stays inside
// each aligned group of 4 slots.  Either way the 8 (row, slot) pairs a
// half-wave touches in one transposing read fall in distinct banks.
template <int DV>
__device__ __forceinline__ constexpr int v_physical_slot(int u, int j) {
  return DV == 128 ? (u ^ (j & 3) ^ ((u & 1) << 2)) : (u ^ (j & 2));
}
template <int DV>
__device__ __forceinline__ constexpr int v_logical_slot(int p, int j) {
  if (DV == 128) {
    const int ps = p ^ (j & 3);
    return ps ^ ((ps & 1) << 2);
  }
  return p ^ (j & 2);
}

// A operand of K^T tiles: 8 dk values of key row kb*32 + r.
template <int DV, int S>
__device__ __forceinline__ bf16x8 kfrag(const char* smem, const int (&kro)[8], int kb, int kc) {
  using L = FP<DV>;
  return *reinterpret_cast<const bf16x8*>(smem + kro[kc] + S * L::KTILE + kb * 32 * L::KROW);
}
// A operand of V^T tiles: 8 keys (16-key chunk kc2) of one value channel.
template <int DV, int S>
__device__ __forceinline__ bf16x8 vfrag(const char* smem, const int (&vro)[DV / 32], int db, int kc2) {
  using L = FP<DV>;
  const char* p = smem + vro[db] + S * L::VTILE + kc2 * 16 * L::VROW;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * L::VROW));
  bf16x8 f;
  __builtin_memcpy(&f, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&f) + 8, &hi, 8);
  return f;
}

// The expanded offsets of the tile in slot S, half KB, for this lane's query
// cell: the start of a QK^T accumulator.  xbl[hh] = XB0 + head * 256 +
// qc * 64 (bytes).
template <int HPW, int S, int KB, int DV>
__device__ __forceinline__ f32x16 beta_acc(const char* smem, const int (&xbl)[HPW], int hh) {
  return *reinterpret_cast<const f32x16*>(smem + xbl[hh] + S * FP<DV>::XBS + KB * 128);
}

// The soft-capped weight with the bias cell as a multiplier.  With
// y = 2^(alpha s) from the MFMA and beta = bias x beta_mul,
//   exp(L - cap) = exp2(rcp(a (1 + 2^(alpha s + beta)))) = exp2(rcp(fma(y, A, a))),
//   A = a 2^beta,
// so the bias needs no work per logit: it scales the fma that the cap needs
// anyway, and the QK^T accumulator starts from zero.  beta is clamped to
// [-100, 100]: beyond it the weight is saturated (2^beta's factor moves
// 1 + 2^(alpha s + beta) by less than 2^-70 relative) unless |alpha s| > 100
// as well, which needs |scale q.k| above 34.7 cap -- a logit no attention
// input reaches; inside the range the product is the exact exponent sum up to
// rounding.
__device__ __forceinline__ float cap_multiplier(float cell, float beta_mul, float den_a) {
  return den_a * __builtin_amdgcn_exp2f(__builtin_amdgcn_fmed3f(cell * beta_mul, -100.f, 100.f));
}
// The value v holds in lane (l & ~3) + K of each quad.
template <int K>
__device__ __forceinline__ float quad_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), K * 0x55, 0xF, 0xF, false));
}
// Lane l's compact-bias cell of slot S ([head][query cell][key cell] as
// copied) for head `head`: query cell (l & 31) >> 4 (its row's), key cell
// l & 3 of the tile.  AGAIN (the tails): the address is worked out afresh,
// not kept in a register from the prologue through the whole key loop.
template <int DV, int S, bool AGAIN = false>
__device__ __forceinline__ float cell_read(const char* smem, int head) {
  int lane = (int)threadIdx.x & 63;
  if constexpr (AGAIN) asm volatile("" : "+v"(lane));
  const int v = ((lane & 31) >> 4) * 4 + (lane & 3);
  return reinterpret_cast<const float*>(smem + FP<DV>::B0 + S * 256)[head * 8 + v];
}
// The two multipliers of half KB (key cells 2 KB and 2 KB + 1) from the
// lane values of a tile.
template <int KB>
__device__ __forceinline__ f32x2 half_multipliers(float am) {
  return f32x2{quad_bcast<2 * KB>(am), quad_bcast<2 * KB + 1>(am)};
}

// x plus the value x holds in the lane that the DPP control CTRL names
// (within each row of 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                  0xF, 0xF, false));
}
// Sum over each group of 8 lanes (every lane of the group gets the same sum:
// each step adds the same two values in either order): quad_perm 1,0,3,2,
// quad_perm 2,3,0,1, row_half_mirror.
__device__ __forceinline__ float sum8(float x) { return dpp_add<0x141>(dpp_add<0x4E>(dpp_add<0xB1>(x))); }

// Expanded-offset entry (float index within a head's 64) that lane l writes
// for the cell of pair vector l >> 3 = 4 qc + kc: copy l & 7 of the 8 copies
// of key cell kc in the half kc >> 1, query cell qc.
__device__ __forceinline__ int pair_entry(int lane) {
  const int v = lane >> 3, qc = v >> 2, kc = v & 3;
  return (kc >> 1) * 32 + qc * 16 + (kc & 1) * 8 + (lane & 7);
}

// The projection of the next tile's bias cells (pair form), woven into a
// stage as one VALU micro-op per slot: slots 0..7 the dot products (two
// chains), 8 their sum, 9..11 the sum over the 8 lanes of a vector, 12 the
// scale and the store of the expanded entry.  Same operations, in the same
// order, as pair_store, whose dependent chain would otherwise stall the wave
// between two stages.
template <int HPW>
struct ProjIn {
  const bf16x8* pv;           // [2] this lane's pair channels
  const uint32_t (*wreg)[8];  // [HPW][8] projection weights
  float beta_mul;
  float* dst[HPW];            // this lane's expanded entry, per head
};
struct ProjState {
  float s0, s1, t;
};
template <int HPW>
__device__ __forceinline__ void proj_op(int j, const ProjIn<HPW>& in, ProjState& st, int hh) {
  if (j < 8) {
    const bf16x2 w = __builtin_bit_cast(bf16x2, in.wreg[hh][j]);
    const bf16x2 x = {in.pv[j >> 2][2 * (j & 3)], in.pv[j >> 2][2 * (j & 3) + 1]};
    if (j & 1) st.s1 = __builtin_amdgcn_fdot2_f32_bf16(x, w, st.s1, false);
    else st.s0 = __builtin_amdgcn_fdot2_f32_bf16(x, w, st.s0, false);
  } else if (j == 8) {
    st.t = st.s0 + st.s1;
  } else if (j == 9) {
    st.t = dpp_add<0xB1>(st.t);
  } else if (j == 10) {
    st.t = dpp_add<0x4E>(st.t);
  } else if (j == 11) {
    st.t = dpp_add<0x141>(st.t);
  } else if (j == 12) {
    *in.dst[hh] = st.t * in.beta_mul;
  }
}
// A scheduling group of n VALU instructions (the builtin takes its count as
// a constant; n is a constant once the slot loop is unrolled).
template <int N>
__device__ __forceinline__ void valu_group() { __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, N, 0); }
__device__ __forceinline__ void valu_group_n(int n) {
  if (n == 3) valu_group<3>(); else if (n == 4) valu_group<4>(); else if (n == 5) valu_group<5>(); else if (n == 6) valu_group<6>();
  else if (n == 7) valu_group<7>(); else if (n == 8) valu_group<8>(); else if (n == 10) valu_group<10>();
  else if (n == 12) valu_group<12>(); else valu_group<14>();
}

// One stage: for each of the HPW heads of the wave, 8 + 2 DV/32 MFMAs (PV of
// half KB of the tile in V stage SV, QK^T of half KB of the tile in K stage
// SK, its accumulator started from zero when the bias is the softmax's
// multiplier (MUL), else from that half's exponent offsets) woven with
// the softmax of the exponents `ssm` into `pout`.  Each A fragment read from
// LDS feeds the MFMAs of all HPW heads.  ring[] holds A fragments three
// slots ahead; the last three slots fetch the first three fragments of the
// following stage (PV on half NKB of V stage NSV).
template <int HPW, int DV, int SV, int SK, int KB, int NSV, int NKB, bool CAP, bool MUL, bool PROJ = false>
__device__ __forceinline__ void fstage(const char* smem, const int (&kro)[8],
                                       const int (&vro)[DV / 32], const int (&xbl)[HPW],
                                       const bf16x8 (&qf)[HPW][8], f32x16 (&O)[HPW][DV / 32],
                                       f32x16 (&sout)[HPW], const bf16x8 (&pin)[HPW][2],
                                       const f32x16 (&ssm)[HPW], float den_a, float (&rowsum)[HPW],
                                       float (&mref)[HPW], bf16x8 (&pout)[HPW][2], bf16x8 (&ring)[4],
                                       const f32x2 (&amx)[HPW], const ProjIn<HPW>* proj = nullptr) {
  constexpr int NPV = DV / 32;
  constexpr int NSLOT = 8 + 2 * NPV;
  constexpr int NOPS = CAP ? kSmOps : kSmOpsU;
  SmState sm[HPW];
  // without the cap: the half's maximum first; the row sums take the
  // factor now, the value accumulators after this stage's PV products
  // (which still add weights taken against the old reference)
  bool moved[HPW];
  float fac[HPW];
  if constexpr (!CAP) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      moved[hh] = update_ref(ssm[hh], mref[hh], fac[hh]);
      rowsum[hh] *= fac[hh];
    }
  }
  ProjState pst[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) pst[hh] = ProjState{0.f, 0.f, 0.f};
  // QK^T of the next half: from zero when the bias is the softmax's
  // multiplier (MUL), from its exponent offsets otherwise
  f32x16 acc[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) acc[hh] = MUL ? f32x16{} : beta_acc<HPW, SK, KB, DV>(smem, xbl, hh);
#pragma unroll
  for (int j = 0; j < NSLOT; ++j) {
    const int jn = j + 3;
    if (jn < NSLOT) {
      ring[jn & 3] = slot_is_qk(jn) ? kfrag<DV, SK>(smem, kro, KB, slot_kc(jn))
                                    : vfrag<DV, SV>(smem, vro, slot_db<NPV>(jn), 2 * KB + slot_half<NPV>(jn));
    } else {
      ring[jn & 3] = vfrag<DV, NSV>(smem, vro, slot_db<NPV>(jn - NSLOT), 2 * NKB);
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      if (slot_is_qk(j)) {
        mfma(acc[hh], ring[j & 3], qf[hh][slot_kc(j)]);
      } else {
        mfma(O[hh][slot_db<NPV>(j)], ring[j & 3], pin[hh][slot_half<NPV>(j)]);
      }
#pragma unroll
      for (int u = 0; u < sm_count<NSLOT, NOPS>(j); ++u) {
        if constexpr (CAP)
          sm_op(kSm.op[sm_begin<NSLOT>(j) + u].pass, kSm.op[sm_begin<NSLOT>(j) + u].idx, sm[hh],
                ssm[hh], den_a, amx[hh], rowsum[hh]);
        else
          sm_op_u(kSmU.op[sm_begin<NSLOT, NOPS>(j) + u].pass, kSmU.op[sm_begin<NSLOT, NOPS>(j) + u].idx,
                  sm[hh], ssm[hh], mref[hh], rowsum[hh]);
      }
      if constexpr (PROJ) proj_op<HPW>(j, *proj, pst[hh], hh);
    }
    // inside the slot: the MFMA first, then the LDS reads, then the VALU work
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    valu_group_n((sm_count<NSLOT, NOPS>(j) + (PROJ && j <= 12 ? 1 : 0)) * HPW);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!CAP) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
      if (moved[hh]) {
#pragma unroll
        for (int db = 0; db < NPV; ++db) O[hh][db] *= fac[hh];
      }
  }
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    sout[hh] = acc[hh];
    bf16x8 f0, f1;
    __builtin_memcpy(&f0, &sm[hh].pk[0], 16);
    __builtin_memcpy(&f1, &sm[hh].pk[4], 16);
    pout[hh][0] = f0;
    pout[hh][1] = f1;
  }
}

// Direct HBM -> LDS copy of 16 bytes per lane: lane l's bytes at base + voff
// land at LDS address lds + 16 l (base and lds uniform across the wave).  The
// copy is written out here rather than through the compiler's builtin: the
// compiler cannot tell which LDS bytes such a copy writes, so after the
// builtin it makes every later LDS access wait for the copy to finish, which
// would turn the prefetch of the next tiles into a stall.  The kernel orders
// the copies itself: each one is waited for (vmcnt 0) and followed by a
// workgroup barrier before any lane reads its LDS stage.  M0 is read when the
// copy issues; nothing else in these kernels uses M0.
__device__ __forceinline__ void lds_copy16(const char* base, int voff, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// Direct HBM -> LDS copy of 4 bytes per lane: lane l's float at addr lands at
// LDS address lds + 4 l.  Same ordering rules as lds_copy16.
__device__ __forceinline__ void lds_copy4(const float* addr, uint32_t lds) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(addr), "s"(lds)
               : "memory", "m0");
#pragma clang diagnostic pop
}

template <int HPW, int DV, bool FUSED>
struct FastCtx {
  static constexpr int NW = kHeads / HPW;   // waves per workgroup
  // direct 16-byte loads per lane per tile: K, V
  static constexpr int LPW_K = FP<DV>::KTILE / (1024 * NW);
  static constexpr int LPW_V = FP<DV>::VTILE / (1024 * NW);
  static_assert(LPW_K * 1024 * NW == FP<DV>::KTILE && LPW_V * 1024 * NW == FP<DV>::VTILE,
                "tiles split evenly over the waves");
  const char* kb_ptr;   // K of this batch item
  const char* vb_ptr;   // V of this batch item
  const float* bias_lane;  // compact-bias cell that this lane copies for tile 0
  int goff_k[LPW_K], goff_v[LPW_V];  // per-lane source offsets of the direct loads
  // A tile that ends the sequence early: its relative index in this
  // workgroup's range (or -1) and its number of keys.  Its copies are clamped
  // to its last row (rows past the end get finite data of that row, and p = 0
  // from the mask), and the bias cells to the last cell: bias_cap is the
  // largest cell offset from bias_lane that stays in the bias row.
  int tile_end, kv_end;
  int bias_cap;
  // FUSED: waves 0 and 1 copy the pair vectors of query cell `wave` (row
  // pr_base): lane l the 16 bytes (l & 15) of key cell pr_cell + 4 t (its
  // vector l >> 4 of the tile), clamped to the last cell pm1.  wreg holds
  // the projection weights this lane multiplies: W[16 (l & 7) + i][head]
  // for i = 0..15, as bf16 pairs.
  const char* pr_base;
  int pr_cell, pm1;
  uint32_t wreg[HPW][8];
  int wave;             // wave index (uniform)
  float beta_mul;       // factor of the bias in the exp2 argument
};

// Direct HBM -> LDS copy of K and V of tile t into stage S (LPW_K + LPW_V
// loads per lane, 1 KiB per wave each).
template <int HPW, int DV, bool TAIL, bool FUSED, int S>
__device__ __forceinline__ void issue_kv(char* smem, const FastCtx<HPW, DV, FUSED>& c, int t) {
  using L = FP<DV>;
  using Ctx = FastCtx<HPW, DV, FUSED>;
  const char* kt = c.kb_ptr + (int64_t)t * L::KTILE;
  const char* vt = c.vb_ptr + (int64_t)t * L::VTILE;
  const uint32_t lds = (uint32_t)(size_t)(lds_void*)smem;
  // rows of the tile that exist (uniform); the offsets of rows past them are
  // clamped to the last 16 bytes of the last one
  const int rows = (TAIL && t == c.tile_end) ? c.kv_end : kTileKeys;
  const int kcap = rows * L::KROW - 16, vcap = rows * L::VROW - 16;
#pragma unroll
  for (int j = 0; j < Ctx::LPW_K; ++j)
    lds_copy16(kt, TAIL ? min(c.goff_k[j], kcap) : c.goff_k[j],
               lds + L::K0 + S * L::KTILE + (uint32_t)((Ctx::LPW_K * c.wave + j) * 1024));
#pragma unroll
  for (int j = 0; j < Ctx::LPW_V; ++j)
    lds_copy16(vt, TAIL ? min(c.goff_v[j], vcap) : c.goff_v[j],
               lds + L::V0 + S * L::VTILE + (uint32_t)((Ctx::LPW_V * c.wave + j) * 1024));
}

// Direct copy of what tile t's exponent offsets are made from into slot S:
// its 64 compact-bias cells (8 heads x 2 query cells x 4 key cells, one per
// lane of wave 0), or with FUSED its 8 pair vectors (2 query cells x 4 key
// cells, 1 KiB per query cell, waves 0 and 1).  Cells past the last one are
// clamped to it.
template <int HPW, int DV, bool TAIL, bool FUSED, int S>
__device__ __forceinline__ void issue_cells(char* smem, const FastCtx<HPW, DV, FUSED>& c, int t) {
  using L = FP<DV>;
  const uint32_t lds = (uint32_t)(size_t)(lds_void*)smem;
  if constexpr (FUSED) {
    if (c.wave < 2)
      lds_copy16(c.pr_base, min(c.pr_cell + 4 * t, c.pm1) * 256 + (int)(threadIdx.x & 15) * 16,
                 lds + L::PR0 + S * L::PTILE + c.wave * 1024);
  } else {
    if (c.wave == 0)
      lds_copy4(c.bias_lane + (TAIL ? min(4 * t, c.bias_cap) : 4 * t), lds + L::B0 + S * 256);
  }
}


// Wait for this wave's direct loads (and the bias load), then the workgroup
// barrier that publishes them.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
}


// Exponent offsets of the tile in slot S for the wave's heads: beta = bias
// cell x the exponent factor, written expanded to the accumulator layout of
// the QK^T product (XB0: per head, half hf and query cell qc, 8 copies of key
// cell 2 hf and 8 of key cell 2 hf + 1), so that a QK^T accumulator starts
// from them with four broadcast LDS reads and the softmax needs no add.  A
// wave writes, and later reads, only its own heads' offsets, so the in-order
// LDS accesses of the wave suffice: no barrier.
//
// From copied compact-bias cells: lane l writes entry l of the head's 64
// (hf = l >> 5, qc = (l >> 4) & 1, key cell 2 hf + ((l >> 3) & 1)).
// The read and the write are separate calls so that the loop can issue the
// read before a stage and the write after it: read right before its use, the
// cell would make the wave wait for every LDS read in flight, the ring's
// prefetches included.
template <int HPW, int DV, int S>
__device__ __forceinline__ void bias_cells_load(const char* smem, int wave, float (&b)[HPW]) {
  using L = FP<DV>;
  const int lane = (int)threadIdx.x & 63;
  const int cell = ((lane >> 4) & 1) * 4 + 2 * (lane >> 5) + ((lane >> 3) & 1);
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
    b[hh] = reinterpret_cast<const float*>(smem + L::B0 + S * 256)[(wave * HPW + hh) * 8 + cell];
}
template <int HPW, int DV, int S>
__device__ __forceinline__ void expand_bias_store(char* smem, int wave, float beta_mul,
                                                  const float (&b)[HPW]) {
  using L = FP<DV>;
  const int lane = (int)threadIdx.x & 63;
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
    reinterpret_cast<float*>(smem + L::XB0 + S * L::XBS)[(wave * HPW + hh) * 64 + lane] =
        b[hh] * beta_mul;
}
template <int HPW, int DV, int S>
__device__ __forceinline__ void expand_bias(char* smem, int wave, float beta_mul) {
  float b[HPW];
  bias_cells_load<HPW, DV, S>(smem, wave, b);
  expand_bias_store<HPW, DV, S>(smem, wave, beta_mul, b);
}

// Projected from the pair vectors (FUSED).  Cell (qc, kc) of head h is
// sum_c pair[qc, kc, c] W[c, h] (bf16 products, float32 sums).  Lane l holds
// channels 16 (l & 7) .. + 15 of pair vector l >> 3 = 4 qc + kc (pair_load);
// the 8 lanes of a vector sum it, and lane l & 7 writes copy l & 7 of the
// cell's 8 (pair_store between two stages, or proj_op woven into one).
template <int DV, int S>
__device__ __forceinline__ void pair_load(const char* smem, bf16x8 (&a)[2]) {
  using L = FP<DV>;
  const int lane = (int)threadIdx.x & 63;
  const char* pt = smem + L::PR0 + S * L::PTILE + (lane >> 3) * 256 + (lane & 7) * 32;
  a[0] = *reinterpret_cast<const bf16x8*>(pt);
  a[1] = *reinterpret_cast<const bf16x8*>(pt + 16);
}
template <int HPW, int DV, int S>
__device__ __forceinline__ void pair_store(char* smem, const bf16x8 (&a)[2], const uint32_t (&wreg)[HPW][8],
                                           int wave, float beta_mul) {
  using L = FP<DV>;
  const int entry = pair_entry((int)threadIdx.x & 63);
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    float s[2] = {0.f, 0.f};  // two chains, added at the end
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x2 w = __builtin_bit_cast(bf16x2, wreg[hh][i]);
      const bf16x2 x = {a[i >> 2][2 * (i & 3)], a[i >> 2][2 * (i & 3) + 1]};
      s[i & 1] = __builtin_amdgcn_fdot2_f32_bf16(x, w, s[i & 1], false);
    }
    const float t = sum8(s[0] + s[1]) * beta_mul;
    reinterpret_cast<float*>(smem + L::XB0 + S * L::XBS)[(wave * HPW + hh) * 64 + entry] = t;
  }
}

// One pipelined iteration for tile t in stage C.
template <int HPW, int DV, bool TAIL, bool FUSED, bool CAP, int C>
__device__ __forceinline__ void fast_iter(char* smem, const FastCtx<HPW, DV, FUSED>& c, int t, int last,
                                          const int (&kro)[8], const int (&vro)[DV / 32],
                                          const int (&xbl)[HPW], const bf16x8 (&qf)[HPW][8],
                                          f32x16 (&O)[HPW][DV / 32], f32x16 (&S0)[HPW],
                                          f32x16 (&S1)[HPW], bf16x8 (&P0)[HPW][2],
                                          bf16x8 (&P1)[HPW][2],
                                          float den_a, float (&rowsum)[HPW], float (&mref)[HPW],
                                          bf16x8 (&ring)[4], float (&amA)[HPW], float (&amB)[HPW]) {
  constexpr int NXT = (C + 1) % 3, NN = (C + 2) % 3;
  constexpr bool MUL = CAP && !FUSED;  // the bias cell as the softmax's multiplier
  // K and V of tile t+2 into the stage that held tile t-1, and the cells of
  // tile t+3 into the slot that held tile t's (read two iterations ago);
  // past the end the copies are clamped and land where nobody reads again
  issue_kv<HPW, DV, TAIL, FUSED, NN>(smem, c, min(t + 2, last));
  issue_cells<HPW, DV, TAIL, FUSED, C>(smem, c, min(t + 3, last));
  // pair vectors of tile t+2: read during X (value width 128), or after it
  // (192, whose stage leaves no registers for them); its compact-bias cells
  // are read during X as well (value width 128)
  bf16x8 pv[2];
  float bc[HPW], amC[HPW];
  if constexpr (FUSED && DV == 128) pair_load<DV, NN>(smem, pv);
  if constexpr (!FUSED && !CAP) bias_cells_load<HPW, DV, NN>(smem, c.wave, bc);
  if constexpr (MUL && DV == 128) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) bc[hh] = cell_read<DV, NN>(smem, c.wave * HPW + hh);
  }
  // the multipliers of the halves each stage weighs: tile t's second half
  // (X), tile t+1's first (Y); a alone in the pair form
  f32x2 amx[HPW], amy[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    amx[hh] = MUL ? half_multipliers<1>(amA[hh]) : f32x2{den_a, den_a};
    amy[hh] = MUL ? half_multipliers<0>(amB[hh]) : f32x2{den_a, den_a};
  }
  // X: PV(t, half 0) + QK(t+1, half 0) || softmax(t, half 1) -> P1
  fstage<HPW, DV, C, NXT, 0, C, 1, CAP, MUL>(smem, kro, vro, xbl, qf, O, S0, P0, S1, den_a, rowsum, mref, P1, ring,
                                             amx);
  // tile t+2: its cell multiplier (compact bias with the cap) or expanded
  // exponent offsets (otherwise), worked out within this iteration so that
  // no LDS count is carried across the loop's back edge
  if constexpr (MUL && DV == 128) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) amC[hh] = cap_multiplier(bc[hh], c.beta_mul, den_a);
  }
  if constexpr (MUL && DV != 128) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) bc[hh] = cell_read<DV, NN>(smem, c.wave * HPW + hh);
  }
  if constexpr (FUSED && DV != 128) {
    pair_load<DV, NN>(smem, pv);
    pair_store<HPW, DV, NN>(smem, pv, c.wreg, c.wave, c.beta_mul);
  }
  if constexpr (!FUSED && !CAP) expand_bias_store<HPW, DV, NN>(smem, c.wave, c.beta_mul, bc);
  // Y: PV(t, half 1) + QK(t+1, half 1) || softmax(t+1, half 0) -> P0
  if constexpr (FUSED && DV == 128) {
    // value width 128: the projection of tile t+2 woven into stage Y
    ProjIn<HPW> pj;
    pj.pv = pv;
    pj.wreg = c.wreg;
    pj.beta_mul = c.beta_mul;
    const int entry = pair_entry((int)threadIdx.x & 63);
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
      pj.dst[hh] = reinterpret_cast<float*>(smem + FP<DV>::XB0 + NN * FP<DV>::XBS) +
                   (c.wave * HPW + hh) * 64 + entry;
    fstage<HPW, DV, C, NXT, 1, NXT, 0, CAP, MUL, true>(smem, kro, vro, xbl, qf, O, S1, P1, S0, den_a, rowsum, mref,
                                                       P0, ring, amy, &pj);
  } else {
    fstage<HPW, DV, C, NXT, 1, NXT, 0, CAP, MUL>(smem, kro, vro, xbl, qf, O, S1, P1, S0, den_a, rowsum, mref, P0,
                                                 ring, amy);
  }
  if constexpr (MUL && DV != 128) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) amC[hh] = cap_multiplier(bc[hh], c.beta_mul, den_a);
  }
  tile_barrier();
  if constexpr (MUL) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      amA[hh] = amB[hh];
      amB[hh] = amC[hh];
    }
  }
}

// Soft-capped weights exp(L - cap) of 16 exponents t from the accumulator,
// with the half's two fma multipliers am (the cells' cap_multiplier when t =
// alpha s, den_a when t already holds the offset), packed as the PV operand;
// the row sum adds the packed values.  MASK: keys past the end of the
// sequence get p = 0.
template <bool MASK>
__device__ __forceinline__ void softmax_exp(const f32x16& t, float den_a, f32x2 am, float& rowsum,
                                            bf16x8 (&p)[2], int lim) {
  float w[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const float y = __builtin_amdgcn_exp2f(t[x]);
    const float d = __builtin_fmaf(y, x < 8 ? am.x : am.y, den_a);
    w[x] = __builtin_amdgcn_exp2f(__builtin_amdgcn_rcpf(d));
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    bf16x2 pr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x2 two = {w[8 * half + 2 * m], w[8 * half + 2 * m + 1]};
      pr[m] = __builtin_convertvector(two, bf16x2);
      if constexpr (MASK) pr[m] = mask_pair(pr[m], 16 * half + 2 * m, lim);
      rowsum = __builtin_amdgcn_fdot2_f32_bf16(pr[m], ones, rowsum, false);
    }
    bf16x8 f;
    __builtin_memcpy(&f, pr, 16);
    p[half] = f;
  }
}

// The weights without the cap, 2^(u - reference) for 16 base-2 exponents u,
// after moving the reference (update_ref) and rescaling what O and the row
// sum hold; packed and summed as softmax_exp.  MASK as there; a masked key
// takes exponent -inf before the maximum is formed, so that the finite but
// meaningless score of a clamped padding row can neither move the reference
// nor take weight (the maximum runs over keys that exist).
template <bool MASK, int NPV>
__device__ __forceinline__ void softmax_exp_u(const f32x16& u_in, float& mref, float& rowsum,
                                              f32x16 (&O)[NPV], bf16x8 (&p)[2], int lim) {
  f32x16 u = u_in;
  if constexpr (MASK) {
#pragma unroll
    for (int x = 0; x < 16; ++x)
      if (16 * (x >> 3) + (x & 7) >= lim) u[x] = -__builtin_inff();
  }
  float f;
  if (update_ref(u, mref, f)) {
#pragma unroll
    for (int db = 0; db < NPV; ++db) O[db] *= f;
  }
  rowsum *= f;
  float w[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) w[x] = __builtin_amdgcn_exp2f(u[x] - mref);
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    bf16x2 pr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x2 two = {w[8 * half + 2 * m], w[8 * half + 2 * m + 1]};
      pr[m] = __builtin_convertvector(two, bf16x2);
      if constexpr (MASK) pr[m] = mask_pair(pr[m], 16 * half + 2 * m, lim);
      rowsum = __builtin_amdgcn_fdot2_f32_bf16(pr[m], ones, rowsum, false);
    }
    bf16x8 f8;
    __builtin_memcpy(&f8, pr, 16);
    p[half] = f8;
  }
}
// The weights of one half, with or without the cap.
template <bool CAP, bool MASK, int NPV>
__device__ __forceinline__ void softmax_any(const f32x16& t, float den_a, f32x2 am, float& rowsum, float& mref,
                                            f32x16 (&O)[NPV], bf16x8 (&p)[2], int lim) {
  if constexpr (CAP) softmax_exp<MASK>(t, den_a, am, rowsum, p, lim);
  else softmax_exp_u<MASK, NPV>(t, mref, rowsum, O, p, lim);
}

// Last tile (stage C): PV of both halves and the softmax of its second half.
template <int HPW, int DV, bool TAIL, bool CAP, int C, bool FUSED>
__device__ __forceinline__ void fast_tail(int klim_half1, const char* smem, const int (&vro)[DV / 32],
                                          f32x16 (&O)[HPW][DV / 32], const f32x16 (&S1)[HPW],
                                          const bf16x8 (&P0)[HPW][2], float den_a,
                                          float (&rowsum)[HPW], float (&mref)[HPW], int head0, float beta_mul) {
  // the tile's cell multipliers (compact bias with the cap), read again from
  // its slot (which still holds them) rather than carried out of the loop in
  // registers
  constexpr bool MUL = CAP && !FUSED;
  float am[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
    am[hh] = MUL ? cap_multiplier(cell_read<DV, C, true>(smem, head0 + hh), beta_mul, den_a) : den_a;
#pragma unroll
  for (int db = 0; db < DV / 32; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 a = vfrag<DV, C>(smem, vro, db, half);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) mfma(O[hh][db], a, P0[hh][half]);
      __builtin_amdgcn_sched_barrier(0);
    }
  // the compiler would otherwise hoist the second half's value reads and
  // products above the softmax and run out of registers at value width 192
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 P1[HPW][2];
  const int lim = klim_half1 - 8 * lane_g();
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
    softmax_any<CAP, TAIL, DV / 32>(S1[hh], den_a, MUL ? half_multipliers<1>(am[hh]) : f32x2{den_a, den_a},
                                    rowsum[hh], mref[hh], O[hh], P1[hh], lim);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int db = 0; db < DV / 32; ++db)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 a = vfrag<DV, C>(smem, vro, db, 2 + half);
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) mfma(O[hh][db], a, P1[hh][half]);
    }
}

// B operand of QK^T, pre-scaled: lane (r, g) holds alpha x dk 16 kc + 8 g ..
// + 7 of its query row (rounded to bf16), for the HPW heads that follow
// `qrow`.  With the accumulator started from beta, the product is then the
// softmax exponent itself.
template <int HPW>
__device__ __forceinline__ void load_q(const __bf16* qrow, int g, float alpha, bf16x8 (&qf)[HPW][kD / 16]) {
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int kc = 0; kc < kD / 16; ++kc) {
      const bf16x8 raw = *reinterpret_cast<const bf16x8*>(qrow + hh * kD + kc * 16 + 8 * g);
      qf[hh][kc] = __builtin_convertvector(__builtin_convertvector(raw, f32x8) * alpha, bf16x8);
    }
}
// LDS offsets of the K^T A operand (key row r, XOR-swizzled 16-byte chunks).
template <int DV>
__device__ __forceinline__ void k_read_offsets(int r, int g, int (&kro)[8]) {
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) kro[kc] = FP<DV>::K0 + r * FP<DV>::KROW + (((2 * kc + g) ^ (r & 15)) * 16);
}

// A tile that ends the sequence early, in stage C, taken on its own after
// the pipelined tiles: QK of both halves, the masked softmax, PV of both
// halves.  `lim0` is the number of keys of the sequence from the tile's
// first key on; `qb` points at the first of the wave's heads in query row
// qpos0 of this workgroup (rows past Sq read row Sq - 1).  Q and the K
// offsets are loaded again here rather than kept from the start: holding
// them past the pipelined loop costs more registers than that loop leaves.
// The tile's cells (or its expanded exponent offsets: the pair form, and
// without the cap) were staged two iterations before.
template <int HPW, int DV, bool CAP, int C, bool FUSED>
__device__ __forceinline__ void fast_partial(int lim0, const __bf16* qb, int qpos0, int Sq, const char* smem,
                                             const int (&vro)[DV / 32], const int (&xbl)[HPW],
                                             f32x16 (&O)[HPW][DV / 32], float alpha, float den_a,
                                             float (&rowsum)[HPW], float (&mref)[HPW], int head0, float beta_mul) {
  // opaque to the compiler, so that it reloads instead of reusing the values
  // read before the loop
  int lane = (int)threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int g = lane >> 5;
  const __bf16* qrow = qb + (int64_t)(min(qpos0 + (lane & 31), Sq - 1) - qpos0) * kHeads * kD;
  bf16x8 qf[HPW][kD / 16];
  load_q<HPW>(qrow, g, alpha, qf);
  int kro[8];
  k_read_offsets<DV>(lane & 31, g, kro);
  const int lim = lim0 - 8 * g;
  constexpr bool MUL = CAP && !FUSED;
  float am[HPW];  // the tile's cell multipliers (compact bias with the cap), from its slot
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
    am[hh] = MUL ? cap_multiplier(cell_read<DV, C, true>(smem, head0 + hh), beta_mul, den_a) : den_a;
  // QK of both halves first, so that Q and the K offsets are dead before
  // the value fragments are read
  f32x16 sc[2][HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    sc[0][hh] = MUL ? f32x16{} : beta_acc<HPW, C, 0, DV>(smem, xbl, hh);
    sc[1][hh] = MUL ? f32x16{} : beta_acc<HPW, C, 1, DV>(smem, xbl, hh);
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) mfma(sc[kb][hh], kfrag<DV, C>(smem, kro, kb, kc), qf[hh][kc]);
    }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 P[HPW][2];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
      softmax_any<CAP, true, DV / 32>(sc[kb][hh], den_a,
                                      MUL ? (kb == 0 ? half_multipliers<0>(am[hh]) : half_multipliers<1>(am[hh]))
                                          : f32x2{den_a, den_a},
                                      rowsum[hh], mref[hh], O[hh], P[hh], lim - 32 * kb);
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 a = vfrag<DV, C>(smem, vro, db, 2 * kb + half);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) mfma(O[hh][db], a, P[hh][half]);
      }
  }
}

// Grid (Sq / 32, B, kv_splits).  With SPLIT, workgroup z covers key tiles
// [z n, (z + 1) n) and writes its unnormalised numerator and denominator to
// the workspace instead of the output (merged by merge_partials_kernel).
// TAIL: S not a multiple of 64 or Sq not a multiple of 32.  The tile that
// ends the sequence is copied with its rows past the end clamped to its last
// row and those keys masked (p = 0); query rows past Sq read row Sq - 1 and
// store nothing.
// CAP: the soft cap with its fixed maximum; otherwise the online softmax
// with a running reference maximum per row (bias, value width 128).
template <int HPW, int DV, bool SPLIT, bool TAIL, bool FUSED, bool CAP>
__device__ __forceinline__ void fast_attention(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                               const __bf16* __restrict__ v, const float* __restrict__ bias,
                                               const __bf16* __restrict__ pair, const __bf16* __restrict__ wt,
                                               __bf16* __restrict__ out, float* __restrict__ ws, int Sq,
                                               int S, int q_offset, int tiles_per_split,
                                               int64_t bias_batch_stride, int bias_group, float alpha,
                                               float beta_mul, float den_a) {
  static_assert(CAP || (DV == 128 && !FUSED), "without the cap: value width 128, compact bias");
  using L = FP<DV>;
  using Ctx = FastCtx<HPW, DV, FUSED>;
  constexpr int NT = 64 * (kHeads / HPW);
  constexpr int NPV = DV / 32;
  __shared__ __attribute__((aligned(16))) char smem[L::SMEM];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r = lane & 31;
  const int g = lane >> 5;
  const int b = blockIdx.y;
  const int split = blockIdx.z;
  const int qpos0 = blockIdx.x * kBlockPos;  // first row of this block in q / out
  const int pos0 = q_offset + qpos0;         // its position in the sequence
  const int P = (S + 15) >> 4;
  const int n = tiles_per_split;
  const int last = n - 1;
  const int64_t key0 = (int64_t)split * tiles_per_split * kTileKeys;  // first key of the range
  const int klim = S - (int)key0;  // keys of the sequence from key0 on
  const int kv_end = S - kTileKeys * ((S + kTileKeys - 1) / kTileKeys - 1);  // keys in the last tile

  Ctx c;
  c.kb_ptr = reinterpret_cast<const char*>(k + ((int64_t)b * S + key0) * kD);
  c.vb_ptr = reinterpret_cast<const char*>(v + ((int64_t)b * S + key0) * DV);
  c.beta_mul = beta_mul;
  c.wave = __builtin_amdgcn_readfirstlane(w);
  c.tile_end = (TAIL && split == (int)gridDim.z - 1 && kv_end < kTileKeys) ? last : -1;
  c.kv_end = kv_end;
  if constexpr (!FUSED) {
    // bias cell of lane l: head l>>3, query block (l>>2)&1, key block l&3
    const int bh = lane >> 3, pb = (lane >> 2) & 1, cell = lane & 3;
    const int qrow = min((pos0 >> 4) + pb, P - 1);  // clamped: query rows past the end
    const float* row = bias + (int64_t)(b / bias_group) * bias_batch_stride + ((int64_t)bh * P + qrow) * P;
    c.bias_lane = row + cell + (key0 >> 4);
    c.bias_cap = P - 1 - cell - (int)(key0 >> 4);
  }
  if constexpr (FUSED) {
    // pair [., P, P, 128] of this item: waves 0 and 1 copy query cell
    // (pos0 >> 4) + wave (clamped), key cells from key0 >> 4 on
    const int qc = min((pos0 >> 4) + min(c.wave, 1), P - 1);
    c.pr_base = reinterpret_cast<const char*>(pair + (int64_t)(b / bias_group) * bias_batch_stride +
                                              (int64_t)qc * P * 128);
    c.pr_cell = (int)(key0 >> 4) + (lane >> 4);
    c.pm1 = P - 1;
    const unsigned short* w16 = reinterpret_cast<const unsigned short*>(wt);
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ch = 16 * (lane & 7) + 2 * i, h = c.wave * HPW + hh;
        c.wreg[hh][i] = (uint32_t)w16[ch * kHeads + h] | ((uint32_t)w16[(ch + 1) * kHeads + h] << 16);
      }
  }
#pragma unroll
  for (int j = 0; j < Ctx::LPW_K; ++j) {
    const int qs = (Ctx::LPW_K * w + j) * 64 + lane;  // 16-byte slot of this lane in a K tile
    const int row = qs >> 4, pc = qs & 15;
    const int key = (row & 32) | key_perm(row & 31);
    c.goff_k[j] = key * L::KROW + ((pc ^ (row & 15)) * 16);
  }
#pragma unroll
  for (int j = 0; j < Ctx::LPW_V; ++j) {
    const int qs = (Ctx::LPW_V * w + j) * 64 + lane;  // 16-byte slot of this lane in a V tile
    const int row = qs / (L::VROW / 16), pc = qs % (L::VROW / 16);
    c.goff_v[j] = row * L::VROW + (2 * v_logical_slot<DV>(pc >> 1, row) + (pc & 1)) * 16;
  }
  int kro[8];
  k_read_offsets<DV>(r, g, kro);
  int vro[NPV];
  {
    const int i16 = lane & 15, grp = lane >> 4;
    const int row = 8 * (grp >> 1) + (i16 >> 2);
#pragma unroll
    for (int db = 0; db < NPV; ++db)
      vro[db] = L::V0 + row * L::VROW + v_physical_slot<DV>(2 * db + (grp & 1), row) * 32 + 8 * (i16 & 3);
  }
  int xbl[HPW];  // this lane's expanded exponent offsets: head, query cell r >> 4
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) xbl[hh] = L::XB0 + (w * HPW + hh) * 256 + (r >> 4) * 64;

  // the wave's first head in the block's first query row, and in this
  // lane's row (rows past Sq read row Sq - 1)
  const __bf16* qb = q + (((int64_t)b * Sq + qpos0) * kHeads + c.wave * HPW) * kD;
  bf16x8 qf[HPW][kD / 16];
  load_q<HPW>(qb + (int64_t)((TAIL ? min(qpos0 + r, Sq - 1) : qpos0 + r) - qpos0) * kHeads * kD, g, alpha, qf);

  f32x16 O[HPW][NPV];
  float rowsum[HPW];
  float mref[HPW];  // reference maximum of the row without the cap (base 2)
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    rowsum[hh] = 0.f;
    mref[hh] = -1e30f;
#pragma unroll
    for (int db = 0; db < NPV; ++db) O[hh][db] = f32x16{};
  }

  // ---- prologue: K/V of tiles 0 and 1, cells of tiles 0..2 ---------------------
  issue_kv<HPW, DV, TAIL, FUSED, 0>(smem, c, 0);
  issue_kv<HPW, DV, TAIL, FUSED, 1>(smem, c, min(1, last));
  issue_cells<HPW, DV, TAIL, FUSED, 0>(smem, c, 0);
  issue_cells<HPW, DV, TAIL, FUSED, 1>(smem, c, min(1, last));
  issue_cells<HPW, DV, TAIL, FUSED, 2>(smem, c, min(2, last));
  tile_barrier();
  // tiles 0 and 1: with the cap and the compact bias the cell multipliers of
  // each lane (iteration t reads tile t+2's), otherwise the expanded exponent
  // offsets (iteration t expands or projects tile t+2's)
  constexpr bool MUL = CAP && !FUSED;
  float amA[HPW], amB[HPW];  // multipliers of tiles t and t+1 (MUL)
  if constexpr (FUSED) {
    bf16x8 pv[2];
    pair_load<DV, 0>(smem, pv);
    pair_store<HPW, DV, 0>(smem, pv, c.wreg, c.wave, beta_mul);
    pair_load<DV, 1>(smem, pv);
    pair_store<HPW, DV, 1>(smem, pv, c.wreg, c.wave, beta_mul);
  } else if constexpr (!CAP) {
    expand_bias<HPW, DV, 0>(smem, c.wave, beta_mul);
    expand_bias<HPW, DV, 1>(smem, c.wave, beta_mul);
  } else {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      amA[hh] = cap_multiplier(cell_read<DV, 0>(smem, c.wave * HPW + hh), beta_mul, den_a);
      amB[hh] = cap_multiplier(cell_read<DV, 1>(smem, c.wave * HPW + hh), beta_mul, den_a);
    }
  }

  f32x16 S0[HPW], S1[HPW];
  bf16x8 P0[HPW][2], P1[HPW][2];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    S0[hh] = MUL ? f32x16{} : beta_acc<HPW, 0, 0, DV>(smem, xbl, hh);
    S1[hh] = MUL ? f32x16{} : beta_acc<HPW, 0, 1, DV>(smem, xbl, hh);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      mfma(S0[hh], kfrag<DV, 0>(smem, kro, 0, kc), qf[hh][kc]);
      mfma(S1[hh], kfrag<DV, 0>(smem, kro, 1, kc), qf[hh][kc]);
    }
    softmax_any<CAP, TAIL, NPV>(S0[hh], den_a, MUL ? half_multipliers<0>(amA[hh]) : f32x2{den_a, den_a},
                                rowsum[hh], mref[hh], O[hh], P0[hh], klim - 8 * g);
  }
  // iteration 0 copies tile 3's cells into slot 0, which other waves may
  // still be reading for tile 0 above (later slots are two barriers past
  // their last read when they are overwritten)
  __syncthreads();
  bf16x8 ring[4];
#pragma unroll
  for (int j = 0; j < 3; ++j) ring[j] = vfrag<DV, 0>(smem, vro, j, 0);

  // ---- main loop, unrolled over the three stages -------------------------------------
  // A last tile that ends the sequence early (tile_end > 0) is left out of
  // the pipeline (it is still prefetched with the others) and taken on its
  // own at the end; with a single tile (tile_end == 0) the prologue and the
  // tail mask it instead.
  const int lastp = (TAIL && c.tile_end > 0) ? last - 1 : last;
  int t = 0;
  while (true) {
    if (t >= lastp) break;
    fast_iter<HPW, DV, TAIL, FUSED, CAP, 0>(smem, c, t, last, kro, vro, xbl, qf, O, S0, S1, P0, P1, den_a, rowsum,
                                            mref, ring, amA, amB);
    ++t;
    if (t >= lastp) break;
    fast_iter<HPW, DV, TAIL, FUSED, CAP, 1>(smem, c, t, last, kro, vro, xbl, qf, O, S0, S1, P0, P1, den_a, rowsum,
                                            mref, ring, amA, amB);
    ++t;
    if (t >= lastp) break;
    fast_iter<HPW, DV, TAIL, FUSED, CAP, 2>(smem, c, t, last, kro, vro, xbl, qf, O, S0, S1, P0, P1, den_a, rowsum,
                                            mref, ring, amA, amB);
    ++t;
  }
  switch (lastp % 3) {
    case 0: fast_tail<HPW, DV, TAIL, CAP, 0, FUSED>(klim - 64 * lastp - 32, smem, vro, O, S1, P0, den_a, rowsum, mref, c.wave * HPW, beta_mul); break;
    case 1: fast_tail<HPW, DV, TAIL, CAP, 1, FUSED>(klim - 64 * lastp - 32, smem, vro, O, S1, P0, den_a, rowsum, mref, c.wave * HPW, beta_mul); break;
    default: fast_tail<HPW, DV, TAIL, CAP, 2, FUSED>(klim - 64 * lastp - 32, smem, vro, O, S1, P0, den_a, rowsum, mref, c.wave * HPW, beta_mul); break;
  }
  if constexpr (TAIL) {
    if (c.tile_end > 0) {  // uniform; the tile was loaded and its offsets expanded before
      switch (last % 3) {
        case 0: fast_partial<HPW, DV, CAP, 0, FUSED>(klim - 64 * last, qb, qpos0, Sq, smem, vro, xbl, O, alpha, den_a, rowsum,
                                           mref, c.wave * HPW, beta_mul); break;
        case 1: fast_partial<HPW, DV, CAP, 1, FUSED>(klim - 64 * last, qb, qpos0, Sq, smem, vro, xbl, O, alpha, den_a, rowsum,
                                           mref, c.wave * HPW, beta_mul); break;
        default: fast_partial<HPW, DV, CAP, 2, FUSED>(klim - 64 * last, qb, qpos0, Sq, smem, vro, xbl, O, alpha, den_a, rowsum,
                                           mref, c.wave * HPW, beta_mul); break;
      }
    }
  }
  if constexpr (SPLIT) {
    // partial rows [split][b][pos][h][DV], each normalised by its own row
    // sum and rounded to bf16 (every value a weighted mean of V rows, so in
    // range and with bf16's own 8-bit exponent per value), then one float per
    // row [split][b][pos][h]: the row sum with the cap, reference +
    // log2(row sum) without it.  Lane (r, g) holds channels
    // 32 db + 8 j + 4 g .. + 3 of its row (32 x 32 accumulator layout).
    const int64_t rows = (int64_t)gridDim.y * Sq * kHeads;
    const int64_t row0 = ((int64_t)split * gridDim.y + b) * Sq * kHeads;
    __bf16* wn = reinterpret_cast<__bf16*>(ws) + row0 * DV;
    float* wd = reinterpret_cast<float*>(reinterpret_cast<__bf16*>(ws) + (int64_t)gridDim.z * rows * DV) + row0;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const int h = w * HPW + hh;
      const float tot = rowsum[hh] + __shfl_xor(rowsum[hh], 32);
      const float inv = 1.f / tot;
      if (TAIL && qpos0 + r >= Sq) continue;
      __bf16* nrow = wn + ((int64_t)(qpos0 + r) * kHeads + h) * DV + 4 * g;
#pragma unroll
      for (int db = 0; db < NPV; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2 lo = {O[hh][db][4 * j] * inv, O[hh][db][4 * j + 1] * inv};
          const f32x2 hi = {O[hh][db][4 * j + 2] * inv, O[hh][db][4 * j + 3] * inv};
          u32x2 pk;
          pk.x = __builtin_bit_cast(unsigned int, __builtin_convertvector(lo, bf16x2));
          pk.y = __builtin_bit_cast(unsigned int, __builtin_convertvector(hi, bf16x2));
          *reinterpret_cast<u32x2*>(nrow + 32 * db + 8 * j) = pk;
        }
      if (g == 0) wd[(int64_t)(qpos0 + r) * kHeads + h] = CAP ? tot : mref[hh] + __builtin_amdgcn_logf(tot);
    }
  } else {
    __syncthreads();  // the output staging reuses the tile buffers
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) stage_output<__bf16, DV>(smem, O[hh], rowsum[hh], r, g, w * HPW + hh);
    __syncthreads();
    copy_output<__bf16, NT, DV>(smem, out + ((int64_t)b * Sq + qpos0) * kHeads * DV, tid,
                                TAIL ? min(kBlockPos, Sq - qpos0) : kBlockPos);
  }
}

template <int HPW, int DV, bool SPLIT, bool TAIL, bool FUSED>
__global__ __launch_bounds__(64 * (kHeads / HPW), 1)
void biased_mqa_fwd_bf16_capped_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                       const __bf16* __restrict__ v, const float* __restrict__ bias,
                                       const __bf16* __restrict__ pair, const __bf16* __restrict__ wt,
                                       __bf16* __restrict__ out, float* __restrict__ ws, int Sq,
                                       int S, int q_offset, int tiles_per_split,
                                       int64_t bias_batch_stride, int bias_group, float alpha,
                                       float beta_mul, float den_a) {
  fast_attention<HPW, DV, SPLIT, TAIL, FUSED, true>(q, k, v, bias, pair, wt, out, ws, Sq, S, q_offset,
                                                    tiles_per_split, bias_batch_stride, bias_group,
                                                    alpha, beta_mul, den_a);
}
template <int HPW, bool SPLIT, bool TAIL>
__global__ __launch_bounds__(64 * (kHeads / HPW), 1)
void biased_mqa_fwd_bf16_uncapped_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                         const __bf16* __restrict__ v, const float* __restrict__ bias,
                                         const __bf16* __restrict__ pair, const __bf16* __restrict__ wt,
                                         __bf16* __restrict__ out, float* __restrict__ ws, int Sq,
                                         int S, int q_offset, int tiles_per_split,
                                         int64_t bias_batch_stride, int bias_group, float alpha,
                                         float beta_mul, float den_a) {
  fast_attention<HPW, 128, SPLIT, TAIL, false, false>(q, k, v, bias, pair, wt, out, ws, Sq, S, q_offset,
                                                      tiles_per_split, bias_batch_stride, bias_group,
                                                      alpha, beta_mul, den_a);
}

// Merge of the key ranges' partial states into the output (one thread per 4
// channels of a row; HBM-bound), per the page's update equations for two
// states (m, d, n) -> (max m, sum d e^(m - max m), sum n e^(m - max m)):
//   * ranges computed with the same fixed maximum (the cap): numerators n_z
//     and denominators d_z, which add: out = sum_z n_z / sum_z d_z;
//   * LSE, ranges with their own running maxima m_z: normalised rows
//     o_z = n_z / d_z and l_z = m_z + log2 d_z (base 2); with M = max_z l_z,
//     out = sum_z 2^(l_z - M) o_z / sum_z 2^(l_z - M).
template <int DV, typename T, bool LSE>
__global__ __launch_bounds__(256)
void merge_partials_kernel(const float* __restrict__ ws, T* __restrict__ out, int64_t rows,
                           int splits) {
  constexpr int Q = DV / 4;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * Q) return;
  const int64_t row = id / Q;
  const int c4 = (int)(id - row * Q);
  const float* wd = ws + (int64_t)splits * rows * DV;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if constexpr (LSE) {
    float mx = -__builtin_inff();
    for (int z = 0; z < splits; ++z) mx = __builtin_fmaxf(mx, wd[(int64_t)z * rows + row]);
    for (int z = 0; z < splits; ++z) {
      const float wz = __builtin_amdgcn_exp2f(wd[(int64_t)z * rows + row] - mx);
      num += wz * *reinterpret_cast<const f32x4*>(ws + ((int64_t)z * rows + row) * DV + 4 * c4);
      den += wz;
    }
  } else {
    for (int z = 0; z < splits; ++z) {
      num += *reinterpret_cast<const f32x4*>(ws + ((int64_t)z * rows + row) * DV + 4 * c4);
      den += wd[(int64_t)z * rows + row];
    }
  }
  const float inv = 1.0f / den;
  if constexpr (sizeof(T) == 2) {
    const f32x2 a = {num[0] * inv, num[1] * inv};
    const f32x2 c = {num[2] * inv, num[3] * inv};
    u32x2 wv;
    wv.x = __builtin_bit_cast(unsigned int, __builtin_convertvector(a, bf16x2));
    wv.y = __builtin_bit_cast(unsigned int, __builtin_convertvector(c, bf16x2));
    *reinterpret_cast<u32x2*>(out + row * DV + 4 * c4) = wv;
  } else {
    *reinterpret_cast<f32x4*>(out + row * DV + 4 * c4) = num * inv;
  }
}

// The same merge for the bf16 kernels' partials (rows normalised by their
// range's row sum, in bf16; one float per row): with weights w_z = d_z (the
// cap) or 2^(l_z - M), M = max_z l_z (without it),
// out = sum_z w_z o_z / sum_z w_z.  bf16 output.
template <int DV, bool LSE>
__global__ __launch_bounds__(256)
void merge_partials_bf16_kernel(const void* __restrict__ ws, __bf16* __restrict__ out, int64_t rows,
                                int splits) {
  constexpr int Q = DV / 4;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= rows * Q) return;
  const int64_t row = id / Q;
  const int c4 = (int)(id - row * Q);
  const __bf16* wn = static_cast<const __bf16*>(ws);
  const float* wd = reinterpret_cast<const float*>(wn + (int64_t)splits * rows * DV);
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f, mx = -__builtin_inff();
  if constexpr (LSE) {
    for (int z = 0; z < splits; ++z) mx = __builtin_fmaxf(mx, wd[(int64_t)z * rows + row]);
  }
  for (int z = 0; z < splits; ++z) {
    const float d = wd[(int64_t)z * rows + row];
    const u32x2 pk = *reinterpret_cast<const u32x2*>(wn + ((int64_t)z * rows + row) * DV + 4 * c4);
    const float wz = LSE ? __builtin_amdgcn_exp2f(d - mx) : d;
    const f32x4 x = {__builtin_bit_cast(float, pk.x << 16), __builtin_bit_cast(float, pk.x & 0xffff0000u),
                     __builtin_bit_cast(float, pk.y << 16), __builtin_bit_cast(float, pk.y & 0xffff0000u)};
    num += wz * x;
    den += wz;
  }
  const float inv = 1.0f / den;
  const f32x2 a = {num[0] * inv, num[1] * inv};
  const f32x2 c = {num[2] * inv, num[3] * inv};
  u32x2 wv;
  wv.x = __builtin_bit_cast(unsigned int, __builtin_convertvector(a, bf16x2));
  wv.y = __builtin_bit_cast(unsigned int, __builtin_convertvector(c, bf16x2));
  *reinterpret_cast<u32x2*>(out + row * DV + 4 * c4) = wv;
}

template <int DV, bool TAIL, bool FUSED, bool CAP>
hipError_t launch_fast_t(const AttnLaunch& a, hipStream_t stream, float alpha, float beta_mul,
                         float den_a) {
  constexpr int HPW = kFastHeadsPerWave;
  const int splits = (int)a.kv_splits;
  const int tiles = (int)((a.Sk + kTileKeys - 1) / kTileKeys) / splits;
  dim3 grid((unsigned)((a.Sq + kBlockPos - 1) / kBlockPos), (unsigned)a.B, (unsigned)splits);
  const __bf16* q = static_cast<const __bf16*>(a.q);
  const __bf16* k = static_cast<const __bf16*>(a.k);
  const __bf16* v = static_cast<const __bf16*>(a.v);
  __bf16* out = static_cast<__bf16*>(a.out);
  const __bf16* pair = static_cast<const __bf16*>(a.pair);
  const __bf16* wt = static_cast<const __bf16*>(a.weight);
  constexpr auto kern1 = CAP ? biased_mqa_fwd_bf16_capped_kernel<HPW, DV, false, TAIL, FUSED>
                             : biased_mqa_fwd_bf16_uncapped_kernel<HPW, false, TAIL>;
  constexpr auto kernz = CAP ? biased_mqa_fwd_bf16_capped_kernel<HPW, DV, true, TAIL, FUSED>
                             : biased_mqa_fwd_bf16_uncapped_kernel<HPW, true, TAIL>;
  if (splits == 1) {
    hipLaunchKernelGGL(kern1, grid,
                       dim3(64 * (kHeads / HPW)), 0, stream, q, k, v, a.bias, pair, wt, out, nullptr,
                       (int)a.Sq, (int)a.Sk, (int)a.q_offset, tiles, a.bias_batch_stride,
                       (int)a.bias_group, alpha, beta_mul, den_a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(kernz, grid,
                     dim3(64 * (kHeads / HPW)), 0, stream, q, k, v, a.bias, pair, wt, out, a.ws,
                     (int)a.Sq, (int)a.Sk, (int)a.q_offset, tiles, a.bias_batch_stride,
                     (int)a.bias_group, alpha, beta_mul, den_a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = a.B * a.Sq * kHeads;
  const int64_t threads = rows * (DV / 4);
  hipLaunchKernelGGL((merge_partials_bf16_kernel<DV, !CAP>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     stream, a.ws, out, rows, splits);
  return hipGetLastError();
}

template <int DV, bool CAP>
hipError_t launch_fast(const AttnLaunch& a, hipStream_t stream, float alpha, float beta_mul,
                       float den_a) {
  const bool tail = a.Sk % kTileKeys != 0 || a.Sq % kBlockPos != 0;
  if constexpr (CAP) {
    if (a.pair)  // bias projected in the kernel from the pair representation
      return tail ? launch_fast_t<DV, true, true, true>(a, stream, alpha, beta_mul, den_a)
                  : launch_fast_t<DV, false, true, true>(a, stream, alpha, beta_mul, den_a);
  }
  return tail ? launch_fast_t<DV, true, false, CAP>(a, stream, alpha, beta_mul, den_a)
              : launch_fast_t<DV, false, false, CAP>(a, stream, alpha, beta_mul, den_a);
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
  if constexpr (CAPPED && sizeof(T) == 2) {
    return a.Dv == 192 ? launch_fast<192, true>(a, stream, alpha, beta_mul, den_a)
                       : launch_fast<128, true>(a, stream, alpha, beta_mul, den_a);
  } else if constexpr (sizeof(T) == 2) {
    // bf16 without the cap (value width 128, compact bias: the only form the
    // boundary accepts): the same kernel with the online softmax
    return launch_fast<128, false>(a, stream, alpha, beta_mul, den_a);
  } else {
    const bool tail = a.Sk % kTileKeys != 0 || a.Sq % kBlockPos != 0;
    const int splits = (int)a.kv_splits;
    const int tiles = (int)((a.Sk + kTileKeys - 1) / kTileKeys) / splits;
    dim3 grid((unsigned)((a.Sq + kBlockPos - 1) / kBlockPos), (unsigned)a.B, (unsigned)splits);
    auto kern = splits > 1 ? (tail ? biased_mqa_fwd_kernel<T, CAPPED, true, true>
                                   : biased_mqa_fwd_kernel<T, CAPPED, false, true>)
                           : (tail ? biased_mqa_fwd_kernel<T, CAPPED, true, false>
                                   : biased_mqa_fwd_kernel<T, CAPPED, false, false>);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.bias,
                       static_cast<T*>(a.out), a.ws, (int)a.Sq, (int)a.Sk, (int)a.q_offset, tiles,
                       a.bias_batch_stride, (int)a.bias_group, alpha, beta_mul, den_a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t threads = a.B * a.Sq * kHeads * (kD / 4);
    hipLaunchKernelGGL((merge_partials_kernel<kD, T, !CAPPED>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, stream, a.ws, static_cast<T*>(a.out), a.B * a.Sq * kHeads,
                       splits);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_biased_mqa_fwd(const AttnLaunch& a, hipStream_t stream) {
  const bool capped = a.softcap > 0.f;
  if (a.dtype == ABG_BF16)
    return capped ? launch_typed<__bf16, true>(a, stream) : launch_typed<__bf16, false>(a, stream);
  return capped ? launch_typed<float, true>(a, stream) : launch_typed<float, false>(a, stream);
}

}  // namespace abg
