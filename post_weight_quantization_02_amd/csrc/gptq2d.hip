// Two-sided adaptive rounding (blog.secrett2633.cloud, "[논문리뷰] GPTQ-2D:
// Cubic-Time Two-Sided Adaptive Rounding", sections 1-3): round X [m x n] on one
// k-bit grid so as to minimise ||A (Z - X) B||_F^2, given the upper factors U_Q
// (U_Q^T U_Q = (A^T A)^-1, m x m) and U_P (U_P^T U_P = (B B^T)^-1, n x n).
//
// With column-major vec the one-sided loop's factor is U_P kron U_Q, so entry
// (i, j) feeds back only to entries (i' >= i, j' >= j) and the entries of an
// anti-diagonal are independent.  With M = E U_P over the entries already rounded,
// entry (i, j) is rounded from X_ij - (U_Q^T M)_ij and its error
// e = (value - q) / (U_Q[i][i] U_P[j][j]) adds e U_P[j][j:] to row i of M.
//
// MI355X: the matrix is cut into 32 x 32 tiles swept by tile anti-diagonals (the
// tiles of one are independent: tile (I, J) needs only tiles above and to the left
// of it).  Three launches per tile anti-diagonal:
//   corr2d  the correction C = sum over I' <= I of U_Q(I', I)^T M(I', J), split in
//           chunks of 8 tile-rows, one work-group per (tile, chunk), on fp32 MFMA
//           (v_mfma_f32_32x32x2f32) with every load issued before the products;
//   tile2d  per tile: the chunks' partial sums added in order, then the tile's own
//           63 anti-diagonals on 256 threads (eight lanes per row share its dot
//           product and its update), writing codes, E and M(I, J);
//   feed2d  M(I, J'') += E(I, J) U_P(J, J'') for the tiles to the right, one
//           work-group per (tile, 8 tiles of J''), on fp32 MFMA.
// The grid comes from a min / max reduction first; every tile's sum of e^2 is
// kept in fp64 and the sums are added in a fixed order at the end.
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kT = 32;            // tile edge
constexpr int kTh = 256;          // threads per work-group
constexpr int kMinMaxWgs = 1024;  // work-groups of the min / max pass

template <typename T>
__global__ __launch_bounds__(kTh) void minmax_kernel(const T* __restrict__ X, int64_t ldx, int64_t m, int64_t n,
                                                     float* __restrict__ part) {
  __shared__ float lo_s[kTh], hi_s[kTh];
  float lo = INFINITY, hi = -INFINITY;
  const int64_t total = m * n;
  for (int64_t id = (int64_t)blockIdx.x * kTh + threadIdx.x; id < total; id += (int64_t)gridDim.x * kTh) {
    const float v = (float)X[(id / n) * ldx + id % n];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  lo_s[threadIdx.x] = lo;
  hi_s[threadIdx.x] = hi;
  __syncthreads();
  for (int o = kTh / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      lo_s[threadIdx.x] = fminf(lo_s[threadIdx.x], lo_s[threadIdx.x + o]);
      hi_s[threadIdx.x] = fmaxf(hi_s[threadIdx.x], hi_s[threadIdx.x + o]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = lo_s[0];
    part[2 * blockIdx.x + 1] = hi_s[0];
  }
}

// scale = max(max - min, 1e-8) / maxq and zero = round(-min / scale) in fp64 (the
// one-sided grid rule over every entry); gridv = {scale, zero} as floats for the sweep
__global__ __launch_bounds__(kTh) void grid_kernel(const float* __restrict__ part, int nwg, int maxq,
                                                   float* __restrict__ scale_out, int32_t* __restrict__ zero_out,
                                                   float* __restrict__ gridv) {
  __shared__ float lo_s[kTh], hi_s[kTh];
  float lo = INFINITY, hi = -INFINITY;
  for (int i = threadIdx.x; i < nwg; i += kTh) {
    lo = fminf(lo, part[2 * i]);
    hi = fmaxf(hi, part[2 * i + 1]);
  }
  lo_s[threadIdx.x] = lo;
  hi_s[threadIdx.x] = hi;
  __syncthreads();
  for (int o = kTh / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      lo_s[threadIdx.x] = fminf(lo_s[threadIdx.x], lo_s[threadIdx.x + o]);
      hi_s[threadIdx.x] = fmaxf(hi_s[threadIdx.x], hi_s[threadIdx.x + o]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double s = fmax((double)hi_s[0] - (double)lo_s[0], 1e-8) / (double)maxq;
    const double z = rint(-(double)lo_s[0] / s);
    *scale_out = (float)s;
    *zero_out = (int32_t)z;
    gridv[0] = (float)s;
    gridv[1] = (float)z;
  }
}

__global__ __launch_bounds__(kTh) void fill_zero_kernel(float* __restrict__ p, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * kTh + threadIdx.x; i < count; i += (int64_t)gridDim.x * kTh) p[i] = 0.f;
}

constexpr int kChunk = 8;   // tiles per work-group in the correction and the feedback

// KA: partial corrections.  Work-group (tile, chunk) of the anti-diagonal adds
// U_Q(I', I)^T M(I', J) over I' in [8 chunk, 8 chunk + 8) and I' <= I, into
// part[(tile * nchunk + chunk)], on v_mfma_f32_32x32x2f32: wave w takes I' = 8
// chunk + w and + w + 4, with both operands read straight from memory (lane l
// reads row k = 2 kk + l / 32 of the two tiles at column l % 32: 128 contiguous
// bytes per half-wave), all of a wave's loads issued before its products; the
// four waves' sums are added in LDS in wave order.
__global__ __launch_bounds__(kTh) void corr2d_kernel(int m, int n, const float* __restrict__ UQ,
                                                     const float* __restrict__ M, float* __restrict__ part,
                                                     int K, int I_lo, int nchunk) {
  __shared__ float red[kTh / 64][16][64];
  const int tile = (int)blockIdx.x / nchunk, ch = (int)blockIdx.x % nchunk;
  const int I = I_lo + tile, J = K - I;
  const int i0 = ch * kChunk, i1 = min(i0 + kChunk, I + 1);
  if (i0 >= i1) return;
  const int r0 = I * kT, c0 = J * kT;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, col = lane & 31, kh = lane >> 5;
  float av[2][16], bv[2][16];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int Ip = i0 + w + 4 * u;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int gr = Ip * kT + 2 * kk + kh;
      const bool ok = Ip < i1 && gr < m;
      av[u][kk] = (ok && r0 + col < m && gr <= r0 + col) ? UQ[(int64_t)gr * m + r0 + col] : 0.f;   // upper part only
      bv[u][kk] = (ok && c0 + col < n) ? M[(int64_t)gr * n + c0 + col] : 0.f;
    }
  }
  f32x16 acc = {};
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[u][kk], bv[u][kk], acc, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) red[w][r][lane] = acc[r];
  __syncthreads();
  if (w == 0) {
    float* out = part + ((int64_t)tile * nchunk + ch) * (kT * kT);
    // lane l, register r: D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = ((red[0][r][lane] + red[1][r][lane]) + red[2][r][lane]) + red[3][r][lane];
      out[(8 * (r >> 2) + 4 * kh + (r & 3)) * kT + col] = v;
    }
  }
}

// KB: one work-group per tile of the anti-diagonal: C = the partial corrections
// added in chunk order, then the tile's own 63 anti-diagonals.
template <typename T>
__global__ __launch_bounds__(kTh) void tile2d_kernel(const T* __restrict__ X, int64_t ldx, int m, int n,
                                                     const float* __restrict__ UQ, const float* __restrict__ UP,
                                                     float* __restrict__ M, float* __restrict__ E,
                                                     const float* __restrict__ part, const float* __restrict__ gridv,
                                                     int maxq, uint8_t* __restrict__ codes, int64_t ldc,
                                                     double* __restrict__ errp, int K, int I_lo, int Nb, int nchunk) {
  __shared__ float xs[kT][kT + 1];      // X - C, then the tile's E
  __shared__ float ml[kT][kT + 1];      // the tile's part of M: E_tile U_P(J, J)
  __shared__ float uq[kT][kT + 1], up[kT][kT + 1];
  __shared__ double red[kTh];
  const int tile = (int)blockIdx.x, I = I_lo + tile, J = K - I;
  const int r0 = I * kT, c0 = J * kT;
  const int t = threadIdx.x, rr = t >> 3, cb = (t & 7) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int nc = (I + kChunk) / kChunk;   // chunks that hold tile-rows <= I
  for (int ch = 0; ch < nc; ++ch) {
    const float* pp = part + ((int64_t)tile * nchunk + ch) * (kT * kT) + rr * kT + cb;
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += pp[u];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int gi = r0 + rr, gj = c0 + cb + u;
    xs[rr][cb + u] = (gi < m && gj < n) ? (float)X[(int64_t)gi * ldx + gj] - acc[u] : 0.f;
  }
  for (int e = t; e < kT * kT; e += kTh) {
    const int i = e >> 5, j = e & 31;
    uq[i][j] = (r0 + i < m && r0 + j < m) ? (i <= j ? UQ[(int64_t)(r0 + i) * m + r0 + j] : 0.f) : (i == j ? 1.f : 0.f);
    up[i][j] = (c0 + i < n && c0 + j < n) ? (i <= j ? UP[(int64_t)(c0 + i) * n + c0 + j] : 0.f) : (i == j ? 1.f : 0.f);
    ml[i][j] = 0.f;
  }
  __syncthreads();
  const float scale = gridv[0], zero = gridv[1], fmaxq = (float)maxq;
  const float rs = 1.f / scale;
  // row i of the tile belongs to the eight lanes 8 i .. 8 i + 7 (a wave holds eight
  // rows): lane p takes every eighth term of the row's dot product and owns the
  // row's columns p, p + 8, p + 16, p + 24 of the tile's part of M in registers
  // (published to LDS for the other rows' dot products); the eight partial sums
  // meet by DPP moves, so all eight lanes round the same value.  A step's
  // entries never read each other's updates (a row is read by other rows only at
  // columns below its own entry); the barrier after each step publishes the row
  // to the other waves.
  const int i = t >> 3, p = t & 7;
  const float rq = 1.f / uq[i][i];
  float mr[kT / 8] = {0.f, 0.f, 0.f, 0.f};
  double eacc = 0.0;
  for (int s = 0; s < 2 * kT - 1; ++s) {
    const int j = s - i;
    const bool on = j >= 0 && j < kT && r0 + i < m && c0 + j < n;
    float d = 0.f;
    if (on) {
#pragma unroll
      for (int u = 0; u < kT / 8; ++u) {
        const int ip = p + 8 * u;
        d = fmaf(ip <= i ? uq[ip][i] : 0.f, ml[ip][j], d);
      }
    }
    // the eight lanes' sum by DPP: quad_perm [1,0,3,2], quad_perm [2,3,0,1], then
    // row_half_mirror (lane k of an 8-lane group reads lane 7 - k: the other quad)
    d += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, d), 0xB1, 0xF, 0xF, false));
    d += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, d), 0x4E, 0xF, 0xF, false));
    d += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, d), 0x141, 0xF, 0xF, false));
    if (on) {
      const float v = xs[i][j] - d;
      const float c = fminf(fmaxf(rintf(v * rs) + zero, 0.f), fmaxq);
      const float e = (v - scale * (c - zero)) * (rq / up[j][j]);
      if (p == 0) {
        codes[(int64_t)(r0 + i) * ldc + c0 + j] = (uint8_t)c;
        eacc += (double)e * (double)e;
        xs[i][j] = e;
      }
#pragma unroll
      for (int u = 0; u < kT / 8; ++u) {
        const int jj = p + 8 * u;
        if (jj >= j) {
          mr[u] = fmaf(e, up[j][jj], mr[u]);
          ml[i][jj] = mr[u];
        }
      }
    }
    __syncthreads();
  }
  // E tile to the workspace, M(I, J) += ml
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int gi = r0 + rr, gj = c0 + cb + u;
    if (gi < m && gj < n) {
      E[(int64_t)gi * n + gj] = xs[rr][cb + u];
      M[(int64_t)gi * n + gj] += ml[rr][cb + u];
    }
  }
  red[t] = eacc;
  __syncthreads();
  for (int o = kTh / 2; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  if (t == 0) errp[(int64_t)I * Nb + J] = red[0];
}

// KC: feedback to the tiles to the right.  Work-group (tile, chunk) adds
// E(I, J) U_P(J, J'') to M(I, J'') for J'' in J + 1 + [8 chunk, 8 chunk + 8), on
// v_mfma_f32_32x32x2f32: E from LDS, U_P rows straight from memory (coalesced),
// wave w taking J'' = j0 + w and + w + 4 and writing its own output tiles.
__global__ __launch_bounds__(kTh) void feed2d_kernel(int m, int n, const float* __restrict__ UP,
                                                     float* __restrict__ M, const float* __restrict__ E, int K,
                                                     int I_lo, int Nb, int nchunk) {
  __shared__ float se[kT][kT + 1];
  const int tile = (int)blockIdx.x / nchunk, ch = (int)blockIdx.x % nchunk;
  const int I = I_lo + tile, J = K - I;
  const int j0 = J + 1 + ch * kChunk, j1 = min(j0 + kChunk, Nb);
  if (j0 >= j1) return;
  const int r0 = I * kT, c0 = J * kT;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, col = lane & 31, kh = lane >> 5;
  float bv[2][16];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int Jp = j0 + w + 4 * u;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int gk = c0 + 2 * kk + kh, gc = Jp * kT + col;
      bv[u][kk] = (Jp < j1 && gk < n && gc < n) ? UP[(int64_t)gk * n + gc] : 0.f;
    }
  }
  // the output tiles' current values, loaded with the operands (lane l, register
  // r: D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] of v_mfma_f32_32x32x2f32)
  float mv[2][16];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int Jp = j0 + w + 4 * u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gi = r0 + 8 * (r >> 2) + 4 * kh + (r & 3), gj = Jp * kT + col;
      mv[u][r] = (Jp < j1 && gi < m && gj < n) ? M[(int64_t)gi * n + gj] : 0.f;
    }
  }
  for (int e = t; e < kT * kT; e += kTh) {
    const int k = e >> 5, c = e & 31;
    se[k][c] = (r0 + k < m && c0 + c < n) ? E[(int64_t)(r0 + k) * n + c0 + c] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int Jp = j0 + w + 4 * u;
    if (Jp >= j1) break;
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(se[col][2 * kk + kh], bv[u][kk], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gi = r0 + 8 * (r >> 2) + 4 * kh + (r & 3), gj = Jp * kT + col;
      if (gi < m && gj < n) M[(int64_t)gi * n + gj] = mv[u][r] + acc[r];
    }
  }
}

__global__ __launch_bounds__(kTh) void err2d_kernel(const double* __restrict__ errp, int64_t count,
                                                    double* __restrict__ out) {
  __shared__ double red[kTh];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < count; i += kTh) s += errp[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = kTh / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

}  // namespace

Plan2D plan2d(int64_t m, int64_t n) {
  Plan2D p;
  p.m = m;
  p.n = n;
  p.Mb = cdiv(m, kT);
  p.Nb = cdiv(n, kT);
  p.off_m = 0;
  p.off_e = align_up(p.off_m + (size_t)m * (size_t)n * sizeof(float), 256);
  p.nchunk_a = cdiv(p.Mb, kChunk);
  p.off_cpart = align_up(p.off_e + (size_t)m * (size_t)n * sizeof(float), 256);
  p.off_err = align_up(p.off_cpart + (size_t)std::min(p.Mb, p.Nb) * (size_t)p.nchunk_a * kT * kT * sizeof(float),
                       256);
  p.off_part = align_up(p.off_err + (size_t)p.Mb * (size_t)p.Nb * sizeof(double), 256);
  p.off_grid = align_up(p.off_part + 2 * kMinMaxWgs * sizeof(float), 256);
  p.ws_bytes = align_up(p.off_grid + 4 * sizeof(float), 256);
  return p;
}

hipError_t quantize2d_launch(const Plan2D& p, const void* X, int x_dtype, int64_t ldx, const float* UQ,
                             const float* UP, int bits, uint8_t* codes, int64_t ldc, float* scale, int32_t* zero,
                             double* out_err, void* ws, hipStream_t s) {
  char* w = (char*)ws;
  float* M = (float*)(w + p.off_m);
  double* errp = (double*)(w + p.off_err);
  float* part = (float*)(w + p.off_part);
  float* gridv = (float*)(w + p.off_grid);
  const int maxq = (1 << bits) - 1;
  const int64_t mn = p.m * p.n;
  const int mm_wgs = (int)std::min<int64_t>(kMinMaxWgs, cdiv(mn, kTh));
  if (x_dtype == 1)
    hipLaunchKernelGGL(minmax_kernel<_Float16>, dim3(mm_wgs), dim3(kTh), 0, s, (const _Float16*)X, ldx, p.m, p.n,
                       part);
  else
    hipLaunchKernelGGL(minmax_kernel<float>, dim3(mm_wgs), dim3(kTh), 0, s, (const float*)X, ldx, p.m, p.n, part);
  hipLaunchKernelGGL(grid_kernel, dim3(1), dim3(kTh), 0, s, part, mm_wgs, maxq, scale, zero, gridv);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<int64_t>(4096, cdiv(mn, kTh))), dim3(kTh), 0, s, M,
                     mn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* E = (float*)(w + p.off_e);
  float* cpart = (float*)(w + p.off_cpart);
  const int Mb = (int)p.Mb, Nb = (int)p.Nb;
  for (int K = 0; K <= Mb + Nb - 2; ++K) {
    const int lo = std::max(0, K - Nb + 1), hi = std::min(K, Mb - 1), ntile = hi - lo + 1;
    const int nca = (hi + kChunk) / kChunk;              // correction chunks of the deepest tile
    hipLaunchKernelGGL(corr2d_kernel, dim3(ntile * nca), dim3(kTh), 0, s, (int)p.m, (int)p.n, UQ, M, cpart, K, lo,
                       nca);
    if (x_dtype == 1)
      hipLaunchKernelGGL(tile2d_kernel<_Float16>, dim3(ntile), dim3(kTh), 0, s, (const _Float16*)X, ldx, (int)p.m,
                         (int)p.n, UQ, UP, M, E, cpart, gridv, maxq, codes, ldc, errp, K, lo, Nb, nca);
    else
      hipLaunchKernelGGL(tile2d_kernel<float>, dim3(ntile), dim3(kTh), 0, s, (const float*)X, ldx, (int)p.m,
                         (int)p.n, UQ, UP, M, E, cpart, gridv, maxq, codes, ldc, errp, K, lo, Nb, nca);
    const int ncc = (Nb - (K - hi) - 1 + kChunk - 1) / kChunk;   // feedback chunks of the leftmost tile
    if (ncc > 0)
      hipLaunchKernelGGL(feed2d_kernel, dim3(ntile * ncc), dim3(kTh), 0, s, (int)p.m, (int)p.n, UP, M, E, K, lo, Nb,
                         ncc);
  }
  hipLaunchKernelGGL(err2d_kernel, dim3(1), dim3(kTh), 0, s, errp, p.Mb * p.Nb, out_err);
  return hipGetLastError();
}

}  // namespace gptq
