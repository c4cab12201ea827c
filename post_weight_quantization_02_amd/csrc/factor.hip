// Damping and the inverse-Hessian factor U (upper, U^T U = (H + lambda I)^-1).
//
// itwiki "GPTQ": three-changes table, change 3 (Cholesky form of H^-1, damping
// by 1% of the mean diagonal, computed once up front); Algorithm 1 first line;
// minimal implementation, damping and factor lines.
//
// Route: U is the inverse of the upper factor Ut of H_l = Ut Ut^T.  With J the
// index reversal, J H_l J = L L^T (ordinary lower Cholesky) and Ut = J L J, so
// U = J L^-1 J.  This costs d^3/3 (Cholesky) + d^3/3 (triangular inverse)
// instead of the d^3 of Cholesky -> inverse -> Cholesky, and gives the same U
// by uniqueness of the Cholesky factor.
//
// Precision: the Cholesky runs in fp64 (fp64 MFMA for its trailing updates);
// fp32 there misses a 1e-4 relative factor tolerance at d = 4096 with
// condition numbers ~1e4.  The triangular inverse of the fp64 factor runs in
// fp32 (MFMA), whose error stays ~1e-6.
//
// Kernels: damp (lambda, info = 0) -> reversed fp64 copy with lambda on the
// diagonal -> per 64-column block: diagonal factor + its inverse in LDS (one
// work-group), panel solve and trailing update (fp64 MFMA 16x16x4) -> fp32
// conversion -> triangular inverse by recursive doubling on the fp32 MFMA GEMM
// -> reversed write of U.
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kNB = 64;
constexpr int kThreads = 256;

// Output layout of v_mfma_f64_16x16x4f64: lane l, register r holds
// D[l / 16 + 4 r][l % 16] (checked on gfx950 against a host product).
__device__ __forceinline__ int f64_row(int lane, int r) { return (lane >> 4) + 4 * r; }

__global__ __launch_bounds__(kThreads) void damp_kernel(const float* __restrict__ H, int64_t d,
                                                        float percdamp, double* lam64,
                                                        float* lambda_out, int32_t* info) {
  __shared__ double red[kThreads];
  const int t = threadIdx.x;
  double s = 0.0;
  for (int64_t i = t; i < d; i += kThreads) s += (double)H[i * (d + 1)];
  red[t] = s;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  if (t == 0) {
    const double lam = (double)percdamp * (red[0] / (double)d);
    *lam64 = lam;
    *lambda_out = (float)lam;
    *info = 0;
  }
}

// A[i][j] = H[d-1-i][d-1-j] (+ lambda on the diagonal), lower 64x64 tiles only
__global__ __launch_bounds__(kThreads) void rev_copy_kernel(const float* __restrict__ H, int64_t d,
                                                            const double* lam64,
                                                            double* __restrict__ A) {
  const int bj = blockIdx.x, bi = blockIdx.y;
  if (bj > bi) return;
  const double lam = *lam64;
  const int t = threadIdx.x;
  const int64_t j = (int64_t)bj * 64 + (t & 63);
  for (int k = 0; k < 16; ++k) {
    const int64_t i = (int64_t)bi * 64 + (t >> 6) + 4 * k;
    if (i < d && j < d && j <= i) {
      double v = (double)H[(d - 1 - i) * d + (d - 1 - j)];
      if (i == j) v += lam;
      A[i * d + j] = v;
    }
  }
}

// Factor the diagonal block A[k0:k0+nbe, k0:k0+nbe] = L L^T in LDS, write L back
// and L^-1 (lower, zeros above) to Dinv.  The first non-positive pivot sets
// info to (its natural column index) + 1 if info is still 0.
__global__ __launch_bounds__(kThreads) void potrf_diag_kernel(double* __restrict__ A, int64_t d,
                                                              int64_t k0, int nbe,
                                                              double* __restrict__ Dinv,
                                                              int32_t* info) {
  __shared__ double L[kNB][kNB + 1];
  __shared__ double X[kNB][kNB + 1];
  __shared__ int fail;
  const int t = threadIdx.x;
  for (int idx = t; idx < kNB * kNB; idx += kThreads) {
    const int r = idx / kNB, c = idx % kNB;
    double v;
    if (r < nbe && c < nbe) v = (c <= r) ? A[(k0 + r) * d + k0 + c] : 0.0;
    else v = (r == c) ? 1.0 : 0.0;  // identity padding of a ragged last block
    L[r][c] = v;
    X[r][c] = (r == c) ? 1.0 : 0.0;
  }
  if (t == 0) fail = -1;
  __syncthreads();
  for (int j = 0; j < kNB; ++j) {
    if (t == 0) {
      const double p = L[j][j];
      if (!(p > 0.0) && fail < 0) fail = j;
      L[j][j] = sqrt(p);
    }
    __syncthreads();
    const double ljj = L[j][j];
    for (int i = j + 1 + t; i < kNB; i += kThreads) L[i][j] /= ljj;
    __syncthreads();
    for (int i = j + 1 + (t >> 4); i < kNB; i += 16) {
      const double lij = L[i][j];
      for (int c = j + 1 + (t & 15); c <= i; c += 16) L[i][c] -= lij * L[c][j];
    }
    __syncthreads();
  }
  // X = L^-1 by row elimination: X[j] /= L[j][j]; X[i] -= L[i][j] X[j] for i > j
  for (int j = 0; j < kNB; ++j) {
    const double rl = 1.0 / L[j][j];
    for (int c = t; c <= j; c += kThreads) X[j][c] *= rl;
    __syncthreads();
    for (int i = j + 1 + (t >> 4); i < kNB; i += 16) {
      const double lij = L[i][j];
      for (int c = (t & 15); c <= j; c += 16) X[i][c] -= lij * X[j][c];
    }
    __syncthreads();
  }
  for (int idx = t; idx < kNB * kNB; idx += kThreads) {
    const int r = idx / kNB, c = idx % kNB;
    if (r < nbe && c <= r) A[(k0 + r) * d + k0 + c] = L[r][c];
    Dinv[idx] = (c <= r) ? X[r][c] : 0.0;
  }
  if (t == 0 && fail >= 0 && *info == 0) *info = (int32_t)(d - (k0 + fail));
}

// fp64 64x64 tile product on MFMA: C = beta C + alpha * sum_k Am[m][k] Bn[n][k]
// with K = 64.  mode 0: panel solve, tile row tr of rows below the diagonal
// block: C = A21 (in place) * Dinv^T.  mode 1: trailing update of lower tile
// (ti >= tj) of the trailing matrix: C -= L21[ti] L21[tj]^T.
__global__ __launch_bounds__(kThreads) void chol_tile_kernel(double* __restrict__ A, int64_t d,
                                                             int64_t k0, int mode,
                                                             const double* __restrict__ Dinv) {
  __shared__ double SA[kNB][kNB + 1];
  __shared__ double SB[kNB][kNB + 1];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int64_t base = k0 + kNB;  // first row/col of the trailing matrix
  int64_t R0, C0;
  if (mode == 0) {
    R0 = base + (int64_t)blockIdx.x * kNB;
    C0 = k0;
  } else {
    const int64_t tt = blockIdx.x;
    int i = (int)((sqrt(8.0 * (double)tt + 1.0) - 1.0) * 0.5);
    while ((int64_t)(i + 1) * (i + 2) / 2 <= tt) ++i;
    while ((int64_t)i * (i + 1) / 2 > tt) --i;
    const int j = (int)(tt - (int64_t)i * (i + 1) / 2);
    R0 = base + (int64_t)i * kNB;
    C0 = base + (int64_t)j * kNB;
  }
  for (int idx = t; idx < kNB * kNB; idx += kThreads) {
    const int r = idx / kNB, c = idx % kNB;
    if (mode == 0) {
      SA[r][c] = (R0 + r < d) ? A[(R0 + r) * d + k0 + c] : 0.0;
      SB[r][c] = Dinv[idx];
    } else {
      SA[r][c] = (R0 + r < d) ? A[(R0 + r) * d + k0 + c] : 0.0;
      SB[r][c] = (C0 + r < d) ? A[(C0 + r) * d + k0 + c] : 0.0;
    }
  }
  __syncthreads();
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll 4
  for (int k4 = 0; k4 < kNB / 4; ++k4) {
    const int k = 4 * k4 + (lane >> 4);
    double a[2], b[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      a[f] = SA[wm * 32 + f * 16 + (lane & 15)][k];
      b[f] = SB[wn * 32 + f * 16 + (lane & 15)][k];
    }
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
  }
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = R0 + wm * 32 + fm * 16 + f64_row(lane, r);
        const int64_t col = C0 + wn * 32 + fn * 16 + (lane & 15);
        if (row >= d || col >= d) continue;
        if (mode == 0) {
          A[row * d + col] = acc[fm][fn][r];
        } else if (col <= row) {
          A[row * d + col] -= acc[fm][fn][r];
        }
      }
}

// L32 := fp32(L) (lower; zeros above) and Linv := blockdiag(fp32(Dinv_k)), zeros elsewhere
__global__ __launch_bounds__(kThreads) void cvt_kernel(const double* __restrict__ A, int64_t d,
                                                       const double* __restrict__ Dinv,
                                                       float* __restrict__ L32,
                                                       float* __restrict__ Linv) {
  const int bj = blockIdx.x, bi = blockIdx.y;
  const int t = threadIdx.x;
  const int c = t & 63;
  const int64_t j = (int64_t)bj * 64 + c;
  for (int k = 0; k < 16; ++k) {
    const int r = (t >> 6) + 4 * k;
    const int64_t i = (int64_t)bi * 64 + r;
    if (i >= d || j >= d) continue;
    L32[i * d + j] = (j <= i) ? (float)A[i * d + j] : 0.f;
    Linv[i * d + j] = (bi == bj) ? (float)Dinv[(int64_t)bi * kNB * kNB + r * kNB + c] : 0.f;
  }
}

// U[i][j] = Linv[d-1-i][d-1-j] for j >= i, else 0
__global__ __launch_bounds__(kThreads) void rev_out_kernel(const float* __restrict__ Linv, int64_t d,
                                                           float* __restrict__ U) {
  const int bj = blockIdx.x, bi = blockIdx.y;
  const int t = threadIdx.x;
  const int64_t j = (int64_t)bj * 64 + (t & 63);
  for (int k = 0; k < 16; ++k) {
    const int64_t i = (int64_t)bi * 64 + (t >> 6) + 4 * k;
    if (i >= d || j >= d) continue;
    U[i * d + j] = (j >= i) ? Linv[(d - 1 - i) * d + (d - 1 - j)] : 0.f;
  }
}

}  // namespace

FactorPlan factor_plan(int64_t d) {
  FactorPlan p{};
  p.d = d;
  p.nb = kNB;
  p.nblk = cdiv(d, kNB);
  size_t off = 0;
  p.off_a64 = off;
  off = align_up(off + (size_t)d * d * sizeof(double), 256);
  p.off_dinv = off;
  off = align_up(off + (size_t)p.nblk * kNB * kNB * sizeof(double), 256);
  p.off_tmp = off;  // Linv (d*d fp32) then the recursive-doubling temporary (d*d/2 fp32)
  off = align_up(off + (size_t)d * d * sizeof(float) + (size_t)d * ((d + 1) / 2) * sizeof(float), 256);
  p.off_lam = off;
  off = align_up(off + 64, 256);
  p.ws_bytes = off;
  return p;
}

hipError_t factor_launch(const FactorPlan& p, const float* H, float percdamp, float* U,
                         float* lambda_out, int32_t* info, void* ws, hipStream_t s) {
  const int64_t d = p.d;
  char* base = (char*)ws;
  double* A = (double*)(base + p.off_a64);
  double* Dinv = (double*)(base + p.off_dinv);
  float* Linv = (float*)(base + p.off_tmp);
  float* Tmp = Linv + (size_t)d * d;
  double* lam = (double*)(base + p.off_lam);
  hipError_t e;
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(kThreads), 0, s, H, d, percdamp, lam, lambda_out, info);
  const unsigned nt = (unsigned)p.nblk;
  hipLaunchKernelGGL(rev_copy_kernel, dim3(nt, nt), dim3(kThreads), 0, s, H, d, lam, A);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int64_t k = 0; k < p.nblk; ++k) {
    const int64_t k0 = k * kNB;
    const int nbe = (int)std::min<int64_t>(kNB, d - k0);
    hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(kThreads), 0, s, A, d, k0, nbe,
                       Dinv + k * kNB * kNB, info);
    const int64_t rest = p.nblk - k - 1;
    if (rest > 0) {
      hipLaunchKernelGGL(chol_tile_kernel, dim3((unsigned)rest), dim3(kThreads), 0, s, A, d, k0, 0,
                         (const double*)(Dinv + k * kNB * kNB));
      hipLaunchKernelGGL(chol_tile_kernel, dim3((unsigned)(rest * (rest + 1) / 2)), dim3(kThreads), 0,
                         s, A, d, k0, 1, (const double*)nullptr);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  float* L32 = U;  // U doubles as fp32 L storage until the final write
  hipLaunchKernelGGL(cvt_kernel, dim3(nt, nt), dim3(kThreads), 0, s, A, d, Dinv, L32, Linv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // recursive doubling: for adjacent diagonal blocks A (first) and C (second) of
  // size S, Linv[C, A] = -Linv[C,C] * (L[C, A] * Linv[A, A])
  for (int64_t S = kNB; S < d; S *= 2) {
    const int64_t nfull = d / (2 * S);
    const int64_t rag0 = nfull * 2 * S;        // start of a trailing partial pair
    const int64_t rag2 = d - (rag0 + S);       // its second-block size
    for (int part = 0; part < 2; ++part) {
      int64_t M, npairs, off0;
      if (part == 0) { M = S; npairs = nfull; off0 = 0; }
      else { M = rag2; npairs = (rag2 > 0) ? 1 : 0; off0 = rag0; }
      if (npairs == 0 || M <= 0) continue;
      GemmBatch g1{};
      g1.A = L32 + (off0 + S) * d + off0; g1.lda = d; g1.sA = 2 * S * d + 2 * S;
      g1.B = Linv + off0 * d + off0;      g1.ldb = d; g1.sB = 2 * S * d + 2 * S;
      g1.C = Tmp;                         g1.ldc = S; g1.sC = M * S;
      g1.M = (int)M; g1.N = (int)S; g1.K = (int)S; g1.batch = (int)npairs;
      g1.alpha = 1.f; g1.beta_zero = 1; g1.kmode = 1;
      if ((e = gemm_f32_launch(g1, s)) != hipSuccess) return e;
      GemmBatch g2{};
      g2.A = Linv + (off0 + S) * d + (off0 + S); g2.lda = d; g2.sA = 2 * S * d + 2 * S;
      g2.B = Tmp;                                 g2.ldb = S; g2.sB = M * S;
      g2.C = Linv + (off0 + S) * d + off0;        g2.ldc = d; g2.sC = 2 * S * d + 2 * S;
      g2.M = (int)M; g2.N = (int)S; g2.K = (int)M; g2.batch = (int)npairs;
      g2.alpha = -1.f; g2.beta_zero = 1; g2.kmode = 2;
      if ((e = gemm_f32_launch(g2, s)) != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(rev_out_kernel, dim3(nt, nt), dim3(kThreads), 0, s, Linv, d, U);
  return hipGetLastError();
}

}  // namespace gptq
