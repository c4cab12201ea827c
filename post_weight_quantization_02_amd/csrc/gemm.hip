// Out-of-block correction of the lazy batch on fp32 matrix cores:
//   W[:, i+B:] -= E U[i:i+B, i+B:]
// (itwiki "GPTQ", three-changes table, change 2, and the last line of
// Algorithm 1).  K = B <= 128, M = d_row, N = the columns after the block.
//
// E arrives transposed (Et [B x d_row], written that way by the panel kernel)
// so that both operands stage with 16-byte loads along the M or N direction
// and land in LDS as [k][m] / [k][n]: the v_mfma_f32_32x32x2f32 operands are
// then one LDS word per lane with 32 consecutive lanes on consecutive words.
// 128x128 output tile per work-group (4 waves, 64x64 each), K in two 64-deep
// phases (67 KB LDS, two work-groups per CU); the C tile is read into
// registers at the start of the last K phase (its latency hides under that
// phase's MFMAs) and written once.  Tiles are mapped so that each XCD runs a contiguous range.
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kT = 128, kKP = 64, kP = kT + 4, kThreads = 256;

__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t total) {
  const int64_t q = total / 8, r = total % 8;
  const int64_t x = bid % 8, i = bid / 8;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void trail_kernel(float* __restrict__ C, int64_t ldc,
                                                         int M, int N, int K,
                                                         const float* __restrict__ Et, int64_t lde,
                                                         const float* __restrict__ Ub, int64_t ldu,
                                                         int64_t tiles_m, int64_t tiles_n) {
  __shared__ __attribute__((aligned(16))) float SA[kKP * kP];
  __shared__ __attribute__((aligned(16))) float SB[kKP * kP];
  const int64_t lid = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int m0 = (int)(lid / tiles_n) * kT, n0 = (int)(lid % tiles_n) * kT;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w & 1, wn = w >> 1;

  // staging: thread t covers k rows t/32 + 8 i (i < 8) and 4 columns at (t % 32) * 4
  const int sk = t >> 5, sc = (t & 31) * 4;
  auto load4 = [&](const float* __restrict__ base, int64_t ld, int k, int x0, int lim) {
    f32x4 v;
    const int x = x0 + sc;
    if (VEC && k < K && x + 3 < lim) {
      v = *(const f32x4*)(base + (int64_t)k * ld + x);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (k < K && x + e < lim) ? base[(int64_t)k * ld + x + e] : 0.f;
    }
    return v;
  };
  f32x4 ra[8], rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + sk + 8 * i;
      ra[i] = load4(Et, lde, k, m0, M);
      rb[i] = load4(Ub, ldu, k, n0, N);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *(f32x4*)&SA[(sk + 8 * i) * kP + sc] = ra[i];
      *(f32x4*)&SB[(sk + 8 * i) * kP + sc] = rb[i];
    }
  };

  // C tile in the MFMA output layout, read at the start of the last K phase
  // (the staging registers are free by then; its latency hides under the MFMAs)
  float c[2][2][16];
  auto cload = [&]() {
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = n0 + wn * 64 + fn * 32 + (lane & 31);
          c[fm][fn][r] = (row < M && col < N) ? C[(int64_t)row * ldc + col] : 0.f;
        }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  auto mfma_phase = [&](int kn) {
#pragma unroll 4
    for (int kk = 0; kk < kKP / 2; ++kk) {
      if (2 * kk >= kn) break;
      const int k = 2 * kk + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        a[f] = SA[k * kP + wm * 64 + f * 32 + (lane & 31)];
        b[f] = SB[k * kP + wn * 64 + f * 32 + (lane & 31)];
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
  };
  // K <= 128: one or two straight-line phases of 64
  gload(0);
  lstore();
  __syncthreads();
  if (K > kKP) {
    gload(kKP);
    mfma_phase(kKP);
    __syncthreads();
    lstore();
    __syncthreads();
    cload();
    mfma_phase(K - kKP);
  } else {
    cload();
    mfma_phase(K);
  }
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = n0 + wn * 64 + fn * 32 + (lane & 31);
        if (row < M && col < N) C[(int64_t)row * ldc + col] = c[fm][fn][r] - acc[fm][fn][r];
      }
}

}  // namespace

hipError_t trail_update_launch(float* C, int64_t ldc, int M, int N, int K, const float* Et,
                               int64_t lde, const float* Ub, int64_t ldu, hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  const int64_t tm = cdiv(M, kT), tn = cdiv(N, kT);
  const bool vec = (lde % 4 == 0) && (ldu % 4 == 0) && (((uintptr_t)Et & 15) == 0) &&
                   (((uintptr_t)Ub & 15) == 0);
  if (vec)
    hipLaunchKernelGGL(trail_kernel<true>, dim3((unsigned)(tm * tn)), dim3(kThreads), 0, s, C, ldc,
                       M, N, K, Et, lde, Ub, ldu, tm, tn);
  else
    hipLaunchKernelGGL(trail_kernel<false>, dim3((unsigned)(tm * tn)), dim3(kThreads), 0, s, C, ldc,
                       M, N, K, Et, lde, Ub, ldu, tm, tn);
  return hipGetLastError();
}

}  // namespace gptq
