// fp32 matrix-core GEMM: C = alpha * A B (+ C), row-major, batched.
//
// Used for the out-of-block correction of the lazy batch, W[:, i+B:] -= E *
// U[i:i+B, i+B:] (itwiki "GPTQ", three-changes table change 2 and the last line
// of Algorithm 1), and for the products of the triangular inverse.
//
// 128x128 output tile per work-group (4 waves, 64x64 each, 2x2 fragments of
// v_mfma_f32_32x32x2f32), 16-deep k stages with a register prefetch of the
// next stage.  A is staged as [m][k] with an odd pitch (17): the MFMA reads one
// A value per lane down a column, which then touches 32 distinct banks.  B is
// staged as [k][n].  Tiles are mapped so that each XCD runs a contiguous range
// of output tiles (shared A rows stay in that XCD's L2).
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kT = 128, kK = 16, kPA = kK + 1, kPB = kT + 4, kThreads = 256;

__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t total) {
  const int64_t q = total / 8, r = total % 8;
  const int64_t x = bid % 8, i = bid / 8;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float* p, bool row_ok, int64_t k, int64_t kend) {
  if (VEC && row_ok && k + 3 < kend) return *(const f32x4*)p;
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (row_ok && k + e < kend) ? p[e] : 0.f;
  return v;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmBatch g, int64_t tiles_m,
                                                            int64_t tiles_n) {
  __shared__ __attribute__((aligned(16))) float SA[kT * kPA];
  __shared__ __attribute__((aligned(16))) float SB[kK * kPB];
  const int64_t total = tiles_m * tiles_n;
  const int64_t lid = xcd_remap(blockIdx.x, total);
  const int64_t mt = lid / tiles_n, nt = lid % tiles_n;
  const int64_t bz = blockIdx.y;
  const float* A = g.A + bz * g.sA;
  const float* B = g.B + bz * g.sB;
  float* C = g.C + bz * g.sC;
  const int64_t m0 = mt * kT, n0 = nt * kT;
  int64_t kbeg = 0, kend = g.K;
  if (g.kmode == 1) kbeg = n0;
  if (g.kmode == 2) kend = std::min<int64_t>(g.K, m0 + kT);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w & 1, wn = w >> 1;
  // staging assignments
  const int am = t >> 1, ak = (t & 1) * 8;      // A: row am, k offset ak..ak+7
  const int bk = t >> 4, bn = (t & 15) * 8;      // B: k row bk, n offset bn..bn+7
  const bool arow = (m0 + am) < g.M;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  f32x4 ra[2], rb[2];
  auto gload = [&](int64_t k0) {
    const float* pa = A + (m0 + am) * g.lda + k0 + ak;
    ra[0] = load4<VEC>(pa, arow, k0 + ak, kend);
    ra[1] = load4<VEC>(pa + 4, arow, k0 + ak + 4, kend);
    const int64_t kr = k0 + bk;
    const bool bok = kr < kend;
    const float* pb = B + kr * g.ldb + n0 + bn;
    rb[0] = load4<VEC>(pb, bok, n0 + bn, g.N);
    rb[1] = load4<VEC>(pb + 4, bok, n0 + bn + 4, g.N);
  };
  if (kbeg < kend) gload(kbeg);
  for (int64_t k0 = kbeg; k0 < kend; k0 += kK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      SA[am * kPA + ak + e] = ra[0][e];
      SA[am * kPA + ak + 4 + e] = ra[1][e];
    }
    *(f32x4*)&SB[bk * kPB + bn] = rb[0];
    *(f32x4*)&SB[bk * kPB + bn + 4] = rb[1];
    __syncthreads();
    if (k0 + kK < kend) gload(k0 + kK);
#pragma unroll
    for (int kk = 0; kk < kK / 2; ++kk) {
      const int k = 2 * kk + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        a[f] = SA[(wm * 64 + f * 32 + (lane & 31)) * kPA + k];
        b[f] = SB[k * kPB + wn * 64 + f * 32 + (lane & 31)];
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = n0 + wn * 64 + fn * 32 + (lane & 31);
        if (row < g.M && col < g.N) {
          float* c = C + row * g.ldc + col;
          *c = g.beta_zero ? g.alpha * acc[fm][fn][r] : (*c + g.alpha * acc[fm][fn][r]);
        }
      }
}

}  // namespace

hipError_t gemm_f32_launch(const GemmBatch& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  const int64_t tm = cdiv(g.M, kT), tn = cdiv(g.N, kT);
  const bool vec = (g.lda % 4 == 0) && (g.ldb % 4 == 0) && (g.sA % 4 == 0) && (g.sB % 4 == 0) &&
                   (((uintptr_t)g.A & 15) == 0) && (((uintptr_t)g.B & 15) == 0);
  dim3 grid((unsigned)(tm * tn), (unsigned)g.batch);
  if (vec)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, dim3(kThreads), 0, s, g, tm, tn);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, dim3(kThreads), 0, s, g, tm, tn);
  return hipGetLastError();
}

}  // namespace gptq
