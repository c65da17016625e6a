// Pair-bias projection for gfx950 (MI355X):
//   bias[b, h, p, r] = sum_c pair[b, p, r, c] * weight[c, h],   h < 8
// The compact pair representation (one cell per 16 x 16 positions) is
// projected to one compact bias plane per query head, as described on the web
// page "Making Full-Context AlphaGenome Fit on an RTX 3090", section
// "Profiling pointed at one very large object" (the dense path then repeats it
// 16x along both sequence axes; here it stays compact).
//
// The pass is bound by HBM bandwidth: every pair cell (C values) is read once
// and 8 floats are written per cell.  Layout of the work:
//   * a wave owns 64 consecutive cells per step; it copies their C values
//     (64 * C * E contiguous bytes) from HBM into its own LDS slice with
//     16-byte, fully coalesced loads, then each lane reads back the row of one
//     cell (XOR-swizzled 16-byte chunks, conflict-free) and forms the 8 dot
//     products in float32;
//   * the weight is staged once per workgroup in LDS as float32 [C][8] and
//     read with broadcast loads (every lane of a wave reads the same address);
//   * the 8 results of a lane go to 8 planes; for each plane the 64 lanes
//     write 64 consecutive floats (256 bytes, coalesced);
//   * a persistent grid walks the cells in wave-sized steps.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "abg_internal.h"

namespace abg {
namespace {

constexpr int kH = 8;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxC = 512;
// Per-wave LDS slice for 64 cells: 64 * CHUNK_C * E bytes, staged in pieces of
// 8 KiB (several workgroups per CU keep enough loads in flight).
constexpr int kSliceBytes = 8192;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T>
__global__ __launch_bounds__(kThreads)
void pair_bias_project_kernel(const T* __restrict__ pair, const T* __restrict__ weight,
                              float* __restrict__ bias, int64_t n_cells_per_item,
                              int64_t n_items, int C) {
  constexpr int E = sizeof(T);
  // Channels per staged piece so that 64 cells fit the slice.
  constexpr int PIECE_C = kSliceBytes / (64 * E);  // 64 (bf16) or 32 (f32)
  __shared__ float w_lds[kMaxC * kH];
  __shared__ __attribute__((aligned(16))) char stage[kWaves * kSliceBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  for (int i = tid; i < C * kH; i += kThreads) {
    if constexpr (E == 2) {
      const uint16_t bits = reinterpret_cast<const uint16_t*>(weight)[i];
      w_lds[i] = __uint_as_float((uint32_t)bits << 16);
    } else {
      w_lds[i] = reinterpret_cast<const float*>(weight)[i];
    }
  }
  __syncthreads();

  char* slice = stage + wave * kSliceBytes;
  const int64_t total = n_cells_per_item * n_items;
  const int64_t n_steps = (total + 63) / 64;
  const int64_t wave_id = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t n_waves = (int64_t)gridDim.x * kWaves;

  for (int64_t step = wave_id; step < n_steps; step += n_waves) {
    const int64_t cell0 = step * 64;
    const int ncell = (int)((total - cell0) < 64 ? (total - cell0) : 64);
    float acc[kH];
#pragma unroll
    for (int h = 0; h < kH; ++h) acc[h] = 0.f;

    for (int c0 = 0; c0 < C; c0 += PIECE_C) {
      const int pc = (C - c0) < PIECE_C ? (C - c0) : PIECE_C;  // channels in this piece
      const int row_chunks = pc * E / 16;                       // 16-B chunks per cell row
      // XOR swizzle of the chunks of a row when their count is a power of two.
      const int swz = ((row_chunks & (row_chunks - 1)) == 0) ? row_chunks - 1 : 0;
      // Coalesced copy of the piece: cell-major rows of row_chunks chunks.
      const int n_chunks = ncell * row_chunks;
      const char* src = reinterpret_cast<const char*>(pair + cell0 * C + c0);
      for (int id = lane; id < n_chunks; id += 64) {
        const int cell = id / row_chunks, c = id - cell * row_chunks;
        const uint4 val = *reinterpret_cast<const uint4*>(src + (int64_t)cell * C * E + c * 16);
        *reinterpret_cast<uint4*>(slice + cell * (row_chunks * 16) + ((c ^ (cell & swz)) * 16)) = val;
      }
      // The slice is private to this wave: wait for its LDS writes, no
      // workgroup barrier (waves run different numbers of steps).
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      if (lane < ncell) {
        const char* row = slice + lane * (row_chunks * 16);
        for (int c = 0; c < row_chunks; ++c) {
          const uint4 val = *reinterpret_cast<const uint4*>(row + ((c ^ (lane & swz)) * 16));
          float x[16 / E];
          if constexpr (E == 2) {
            x[0] = bf16_lo(val.x); x[1] = bf16_hi(val.x);
            x[2] = bf16_lo(val.y); x[3] = bf16_hi(val.y);
            x[4] = bf16_lo(val.z); x[5] = bf16_hi(val.z);
            x[6] = bf16_lo(val.w); x[7] = bf16_hi(val.w);
          } else {
            x[0] = __uint_as_float(val.x); x[1] = __uint_as_float(val.y);
            x[2] = __uint_as_float(val.z); x[3] = __uint_as_float(val.w);
          }
          const float* wrow = w_lds + (c0 + c * (16 / E)) * kH;
#pragma unroll
          for (int m = 0; m < 16 / E; ++m)
#pragma unroll
            for (int h = 0; h < kH; ++h) acc[h] = __builtin_fmaf(x[m], wrow[m * kH + h], acc[h]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }

    if (lane < ncell) {
      const int64_t cell = cell0 + lane;
      const int64_t item = cell / n_cells_per_item;
      const int64_t pr = cell - item * n_cells_per_item;
      float* dst = bias + item * kH * n_cells_per_item + pr;
#pragma unroll
      for (int h = 0; h < kH; ++h) dst[h * n_cells_per_item] = acc[h];
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 inputs with C a multiple of 32: the projection as a skinny matrix
// product on the matrix cores, D = W^T . pair^T per 16 cells, with the
// 16x16x32 bf16 MFMA (float32 accumulation):
//   * A (16 x 32) = W^T for one 32-channel step: row m = head (rows 8..15
//     are zero), lane l holds row l % 16, channels 8 (l >> 4) .. + 7;
//     the C / 32 fragments stay in registers for the whole kernel;
//   * B (32 x 16) = pair^T: column n = cell, lane l holds cell l % 16,
//     channels 8 (l >> 4) .. + 7 of the step -- one 16-byte load per lane
//     straight from HBM (each cell row is C * 2 contiguous bytes);
//   * D (16 x 16): lane l holds cell l % 16, heads 4 (l >> 4) .. + 3 (lanes
//     32..63 hold the zero rows).
// A wave takes 16 cells per step: it issues the loads of all its fragments
// at once (C / 32 of them) and then runs the MFMAs; the D values go through
// the wave's own LDS slice so that every lane then stores, 4 heads x 16
// cells per instruction.  With 16 cells a step there are more waves than fit
// a CU at once, so the stores of some overlap the loads of others: measured
// against 64 cells a step with the stores straight from D, 16.3 against
// 16.9 us per full layer on cold inputs.  The pass is bound by HBM.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaMaxC = 256;

template <int NKS>  // C / 32
__global__ __launch_bounds__(kThreads)
void pair_bias_project_mfma_kernel(const __bf16* __restrict__ pair, const __bf16* __restrict__ weight,
                                   float* __restrict__ bias, int64_t n_cells_per_item,
                                   int64_t n_items) {
  constexpr int C = NKS * 32;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, kg = lane >> 4;
  __shared__ float res[kWaves][kH * 16];  // per wave: [head][cell] of a step

  bf16x8_t a[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      a[ks][i] = col < kH ? weight[(ks * 32 + 8 * kg + i) * kH + col] : (__bf16)0.0f;
  }

  const int64_t total = n_cells_per_item * n_items;
  const int64_t n_steps = (total + 15) / 16;
  const int64_t n_waves = (int64_t)gridDim.x * kWaves;
  for (int64_t step = (int64_t)blockIdx.x * kWaves + wave; step < n_steps; step += n_waves) {
    const int64_t cell0 = step * 16;
    bf16x8_t b[NKS];
    {
      int64_t cell = cell0 + col;
      cell = cell < total ? cell : total - 1;  // past the end: load a valid cell, store nothing
      const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(pair + cell * C + 8 * kg);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) b[ks] = src[ks * 4];
    }
    f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], b[ks], d, 0, 0, 0);
    if (kg < 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) res[wave][(4 * kg + i) * 16 + col] = d[i];
    }
    // a wave's LDS accesses run in order: its reads below see its writes
    __builtin_amdgcn_wave_barrier();
    const int64_t cell = cell0 + col;
    if (cell < total) {
      const int64_t item = cell / n_cells_per_item;
      const int64_t pr = cell - item * n_cells_per_item;
      float* dst = bias + item * kH * n_cells_per_item + pr;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int h = 4 * hh + kg;
        dst[h * n_cells_per_item] = res[wave][h * 16 + col];
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_pair_bias_project(const void* pair, const void* weight, float* bias,
                                    int64_t Bp, int64_t P, int64_t C, abg_dtype dtype,
                                    hipStream_t stream) {
  const int64_t cells = P * P;
  const int64_t steps = (cells * Bp + 63) / 64;
  int64_t blocks = (steps + kWaves - 1) / kWaves;
  const int64_t max_blocks = 256 * 8;  // 8 workgroups per CU is plenty for a stream
  if (blocks > max_blocks) blocks = max_blocks;
  if (dtype == ABG_BF16 && C % 32 == 0 && C <= kMfmaMaxC) {
    const int64_t wsteps = (cells * Bp + 15) / 16;
    int64_t mblocks = (wsteps + kWaves - 1) / kWaves;
    if (mblocks > 65536) mblocks = 65536;
    const __bf16* p = static_cast<const __bf16*>(pair);
    const __bf16* w = static_cast<const __bf16*>(weight);
    switch (C / 32) {
      case 1: hipLaunchKernelGGL(pair_bias_project_mfma_kernel<1>, dim3((unsigned)mblocks), dim3(kThreads), 0, stream, p, w, bias, cells, Bp); break;
      case 2: hipLaunchKernelGGL(pair_bias_project_mfma_kernel<2>, dim3((unsigned)mblocks), dim3(kThreads), 0, stream, p, w, bias, cells, Bp); break;
      case 3: hipLaunchKernelGGL(pair_bias_project_mfma_kernel<3>, dim3((unsigned)mblocks), dim3(kThreads), 0, stream, p, w, bias, cells, Bp); break;
      case 4: hipLaunchKernelGGL(pair_bias_project_mfma_kernel<4>, dim3((unsigned)mblocks), dim3(kThreads), 0, stream, p, w, bias, cells, Bp); break;
      case 5: hipLaunchKernelGGL(pair_bias_project_mfma_kernel<5>, dim3((unsigned)mblocks), dim3(kThreads), 0, stream, p, w, bias, cells, Bp); break;
      case 6: hipLaunchKernelGGL(pair_bias_project_mfma_kernel<6>, dim3((unsigned)mblocks), dim3(kThreads), 0, stream, p, w, bias, cells, Bp); break;
      case 7: hipLaunchKernelGGL(pair_bias_project_mfma_kernel<7>, dim3((unsigned)mblocks), dim3(kThreads), 0, stream, p, w, bias, cells, Bp); break;
      default: hipLaunchKernelGGL(pair_bias_project_mfma_kernel<8>, dim3((unsigned)mblocks), dim3(kThreads), 0, stream, p, w, bias, cells, Bp); break;
    }
  } else if (dtype == ABG_BF16) {
    hipLaunchKernelGGL(pair_bias_project_kernel<__bf16>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, static_cast<const __bf16*>(pair), static_cast<const __bf16*>(weight),
                       bias, cells, Bp, (int)C);
  } else {
    hipLaunchKernelGGL(pair_bias_project_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, static_cast<const float*>(pair), static_cast<const float*>(weight),
                       bias, cells, Bp, (int)C);
  }
  return hipGetLastError();
}

}  // namespace abg
