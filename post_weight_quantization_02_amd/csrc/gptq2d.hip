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
// of it).  Two launches per tile anti-diagonal K:
//   fc2d    the partial corrections C = sum over I' <= I of U_Q(I', I)^T M(I', J)
//           of anti-diagonal K, split in chunks of 8 tile-rows, one work-group per
//           (tile, chunk), together with the feedback of anti-diagonal K - 1,
//           M(I, J'') += E(I, J) U_P(J, J'') for J'' >= J + 2, one work-group per
//           (tile, 8 tiles of J''); both on fp32 MFMA (v_mfma_f32_32x32x2f32) with
//           every load issued before the products;
//   tile2d  per tile: the chunks' partial sums added in order, then the tile's own
//           63 anti-diagonals on one wave (one column per pair of lanes), writing
//           codes, E and M(I, J), and the right neighbour's feedback
//           M(I, J + 1) += E(I, J) U_P(J, J + 1), which the next correction needs.
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
__device__ __forceinline__ void corr2d_body(int bid, int m, int n, const float* __restrict__ UQ,
                                            const float* __restrict__ M, float* __restrict__ part, int K, int I_lo,
                                            int nchunk) {
  __shared__ float red[kTh / 64][16][64];
  const int tile = bid / nchunk, ch = bid % nchunk;
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
// added in chunk order (all four waves), then the tile's own 63 anti-diagonals on
// wave 0, one column per pair of lanes (j and j + 32, rows 0-15 and 16-31).  A
// pair keeps column j of the tile's part of M in registers; at step s its entry
// is row i = s - j, whose dot product sum_{i' <= i} U_Q[i'][i] M[i'][j] needs only
// its own column (U_Q's column i comes from LDS, stored transposed; the two halves
// meet by a lane swap, so both round the same value), and the step's errors, one
// per row, meet in a 32-word LDS vector from which every lane adds
// e_k U_P[s - k][j] to its rows k.  The factors U_P[s - k][j] for a lane's 16 rows
// are one contiguous run of column j of U_P stored reversed, kept in four copies
// shifted by one word so that every step reads its run with aligned 16-byte
// loads.  No barrier inside the sweep, and the step loop stays rolled.
template <typename T>
__global__ __launch_bounds__(kTh) void tile2d_kernel(const T* __restrict__ X, int64_t ldx, int m, int n,
                                                     const float* __restrict__ UQ, const float* __restrict__ UP,
                                                     float* __restrict__ M, float* __restrict__ E,
                                                     const float* __restrict__ part, const float* __restrict__ gridv,
                                                     int maxq, uint8_t* __restrict__ codes, int64_t ldc,
                                                     double* __restrict__ errp, int K, int I_lo, int Nb, int nchunk) {
  constexpr int kH = kT / 2;             // rows per lane
  constexpr int kUQ = kT + 4;            // pitch of uqt: rows 16-byte aligned, row reads spread over banks
  constexpr int kRun = 2 * kT - 1;       // reversed column j of U_P: rv[z] = U_P[kRun - 1 - z][j]
  constexpr int kUW = 3 * kT + 4;        // pitch of a reversed column (a run starts at z <= 62, ends <= 93)
  __shared__ float xs[kT + 1][kT];       // X - C, then the tile's E (pitch 32: an anti-diagonal's
                                         // entries fall in 32 different banks); row 32 takes the
                                         // sweep's discarded writes
  __shared__ __attribute__((aligned(16))) float uqt[kT][kUQ];      // uqt[i][i'] = U_Q(I, I)[i'][i]
  __shared__ __attribute__((aligned(16))) float upw[4][kT][kUW];   // upw[r][j][z] = rv_j[z + r]
  __shared__ float up[kT][kT + 1];       // U_P(J, J), staged for upw; then the tile's part of M
  __shared__ float fac[kT][kT];          // (1 / U_Q[i][i]) / U_P[j][j]
  __shared__ __attribute__((aligned(16))) float es[kT + 4];        // the step's errors, by row (+ a
                                                                   // slot for discarded writes)
  __shared__ uint8_t cs[kT + 1][kT];     // codes (row 32: discarded writes)
  __shared__ float upn[kT][kT + 1];      // U_P(J, J + 1), for the right neighbour's feedback
  __shared__ float mo[2][kT][kT];        // M(I, J) and M(I, J + 1) as they stand
  __shared__ double red[kTh];
  const int tile = (int)blockIdx.x, I = I_lo + tile, J = K - I;
  const int r0 = I * kT, c0 = J * kT;
  const int t = threadIdx.x, rr = t >> 3, cb = (t & 7) * 4;
  // every global load of the set-up is issued before the values are used:
  // addresses are clamped into the matrix and the results selected afterwards
  float xv[4], qv[4], pv[4], qd[4], pd[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int gi = min(r0 + rr, m - 1), gj = min(c0 + cb + u, n - 1);
    xv[u] = (float)X[(int64_t)gi * ldx + gj];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = t + kTh * q, i = e >> 5, j = e & 31;
    const int qi = min(r0 + i, m - 1), qj = min(r0 + j, m - 1), pi = min(c0 + i, n - 1), pj = min(c0 + j, n - 1);
    qv[q] = UQ[(int64_t)qi * m + qj];
    pv[q] = UP[(int64_t)pi * n + pj];
    qd[q] = UQ[(int64_t)qi * m + qi];
    pd[q] = UP[(int64_t)pj * n + pj];
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int nc = (I + kChunk) / kChunk;   // chunks that hold tile-rows <= I
  const float* pp = part + (int64_t)tile * nchunk * (kT * kT) + rr * kT + cb;
  int ch = 0;
  for (; ch + 8 <= nc; ch += 8) {   // eight chunks' loads in flight, added in chunk order
    f32x4 x[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = *(const f32x4*)(pp + (ch + q) * (kT * kT));
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] += x[q][u];
  }
  for (; ch < nc; ++ch) {
    const f32x4 x = *(const f32x4*)(pp + ch * (kT * kT));
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += x[u];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int gi = r0 + rr, gj = c0 + cb + u;
    xs[rr][cb + u] = (gi < m && gj < n) ? xv[u] - acc[u] : 0.f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = t + kTh * q, i = e >> 5, j = e & 31;
    // the tiles' upper parts; the identity outside the matrix
    uqt[j][i] = (r0 + i < m && r0 + j < m) ? (i <= j ? qv[q] : 0.f) : (i == j ? 1.f : 0.f);
    up[i][j] = (c0 + i < n && c0 + j < n) ? (i <= j ? pv[q] : 0.f) : (i == j ? 1.f : 0.f);
    fac[i][j] = (1.f / (r0 + i < m ? qd[q] : 1.f)) / (c0 + j < n ? pd[q] : 1.f);
  }
  if (t < kT) es[t] = 0.f;
  // the reversed columns of U_P in four shifted copies: zeros first, then the
  // 32 values of each column (rv_j[y] = U_P[62 - y][j] for y = 31 .. 62) into
  // every copy r at z = y - r
  {
    float* w = &upw[0][0][0];
    for (int e = t; e < 4 * kT * kUW / 4; e += kTh) *(f32x4*)(w + 4 * e) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  {
    const int j = t & 31, c0w = (t >> 5) * 4;   // rows c0w .. c0w + 3 of column j
    float cv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) cv[q] = up[c0w + q][j];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int y = kRun - 1 - (c0w + q);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (y - r >= 0) upw[r][j][y - r] = cv[q];
    }
  }
  __syncthreads();
  double eacc = 0.0;
  if (t < 64) {
    const int j = t & 31, h = t >> 5;
    float mc[kH];
#pragma unroll
    for (int k = 0; k < kH; ++k) mc[k] = 0.f;
    const float scale = gridv[0], zero = gridv[1], fmaxq = (float)maxq;
    const float rs = 1.f / scale;
    const bool colv = c0 + j < n;
    // the operands of a step that do not depend on the previous step (U_Q's
    // column, X - C, the error factor) are read one step ahead, under the
    // previous step's error exchange
    f32x4 un[kH / 4];
    float xn, fn;
    auto fetch = [&](int sn) __attribute__((always_inline)) {
      const int ic = min(max(sn - j, 0), kT - 1);
      xn = xs[ic][j];
      fn = fac[ic][j];
      const f32x4* urow = (const f32x4*)&uqt[ic][kH * h];
#pragma unroll
      for (int q = 0; q < kH / 4; ++q) un[q] = urow[q];
    };
    fetch(0);
    for (int s = 0; s < kRun; ++s) {
      // every lane runs every instruction of a step (no branches): a lane whose
      // column has no entry on this anti-diagonal computes on row ic's operands
      // and sends its writes to the spare row and slot
      const int i = s - j;
      const bool inr = (unsigned)i < (unsigned)kT;
      const bool val = inr && colv && r0 + i < m;
      // dot product over i' <= i (U_Q upper: uqt[i][i'] = 0 past i), each half
      // over its 16 rows, the halves added by a swap of lanes j and j + 32
      float dq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < kH / 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[r] = fmaf(un[q][r], mc[4 * q + r], dq[r]);
      const float dh = (dq[0] + dq[1]) + (dq[2] + dq[3]);
      // swap the upper half of one copy with the lower half of another: the
      // first result then holds rows 0-15's sum and the second rows 16-31's, in
      // both halves (the results are copied out as scalars before the casts)
      const unsigned du = __builtin_bit_cast(unsigned, dh);
      const auto sw = __builtin_amdgcn_permlane32_swap(du, du, false, false);
      const unsigned lo = sw[0], hi = sw[1];
      const float d = __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
      const float v = xn - d;
      const float c = fminf(fmaxf(rintf(v * rs) + zero, 0.f), fmaxq);
      const float e = val ? (v - scale * (c - zero)) * fn : 0.f;
      const int iw = (val && h == 0) ? i : kT;
      cs[iw][j] = (uint8_t)c;
      xs[iw][j] = e;
      es[(inr && h == 0) ? i : kT] = e;
      // row s - 32 had its last entry (column 31) in the previous step
      es[(t == kT - 1 && s >= kT) ? s - kT : kT] = 0.f;
      // the writes above come before the reads below in this wave's LDS queue,
      // which the hardware keeps in order; only the compiler must not move them
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      f32x4 ev[kH / 4], uv[kH / 4];
#pragma unroll
      for (int q = 0; q < kH / 4; ++q) ev[q] = *(const f32x4*)&es[kH * h + 4 * q];
      {
        // U_P[s - k][j] = rv_j[kRun - 1 - s + k] for this lane's rows k = 16 h + k'
        const int o = kRun - 1 - s, r = o & 3;
        const f32x4* run = (const f32x4*)&upw[r][j][o - r + kH * h];
#pragma unroll
        for (int q = 0; q < kH / 4; ++q) uv[q] = run[q];
      }
      fetch(s + 1);   // past the last step it reads a clamped row and is not used
      // M[k][j] += e_k U_P[s - k][j]; rows without an entry in this step have
      // e_k = 0, and U_P[s - k][j] = 0 where s - k is not in 0 .. j
#pragma unroll
      for (int q = 0; q < kH / 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) mc[4 * q + r] = fmaf(ev[q][r], uv[q][r], mc[4 * q + r]);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
#pragma unroll
    for (int k = 0; k < kH; ++k) up[kH * h + k][j] = mc[k];
  } else if (t >= 64) {
    // waves 1-3, idle during the sweep, stage U_P(J, J + 1), M(I, J) and M(I, J + 1)
    // (no other work-group of this launch writes these two tiles of M)
    for (int e = t - 64; e < kT * kT; e += kTh - 64) {
      const int k = e >> 5, c = e & 31;
      const int gi = min(r0 + k, m - 1), gj = min(c0 + c, n - 1), gn = min(c0 + kT + c, n - 1);
      const float u = UP[(int64_t)min(c0 + k, n - 1) * n + gn];
      const float a = M[(int64_t)gi * n + gj], b = M[(int64_t)gi * n + gn];
      upn[k][c] = (c0 + k < n && c0 + kT + c < n) ? u : 0.f;
      mo[0][k][c] = a;
      mo[1][k][c] = b;
    }
  }
  __syncthreads();
  // E (and its squares, in fp64), codes and M(I, J) += the tile's part of M
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int gi = r0 + rr, gj = c0 + cb + u;
    if (gi < m && gj < n) {
      const float e = xs[rr][cb + u];
      E[(int64_t)gi * n + gj] = e;
      eacc += (double)e * (double)e;
      codes[(int64_t)gi * ldc + gj] = cs[rr][cb + u];
      M[(int64_t)gi * n + gj] = mo[0][rr][cb + u] + up[rr][cb + u];
    }
  }
  // the right neighbour's feedback, M(I, J + 1) += E(I, J) U_P(J, J + 1), before
  // its correction is formed in the next launch
  if (J + 1 < Nb) {
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int k = 0; k < kT; ++k) {
      const float ev = xs[rr][k];
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = fmaf(ev, upn[k][cb + u], o[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int gi = r0 + rr, gj = c0 + kT + cb + u;
      if (gi < m && gj < n) M[(int64_t)gi * n + gj] = mo[1][rr][cb + u] + o[u];
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

// KC: feedback to the tiles to the right but one (the tile kernel itself feeds
// its right neighbour, J + 1).  Work-group (tile, chunk) adds E(I, J) U_P(J, J'')
// to M(I, J'') for J'' in J + 2 + [8 chunk, 8 chunk + 8), on
// v_mfma_f32_32x32x2f32: E from LDS, U_P rows straight from memory (coalesced),
// wave w taking J'' = j0 + w and + w + 4 and writing its own output tiles.
__device__ __forceinline__ void feed2d_body(int bid, int m, int n, const float* __restrict__ UP,
                                            float* __restrict__ M, const float* __restrict__ E, int K, int I_lo,
                                            int Nb, int nchunk) {
  __shared__ float se[kT][kT + 1];
  const int tile = bid / nchunk, ch = bid % nchunk;
  const int I = I_lo + tile, J = K - I;
  const int j0 = J + 2 + ch * kChunk, j1 = min(j0 + kChunk, Nb);
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

// One launch between two tile sweeps: the feedback of anti-diagonal K - 1 (the
// first nfeed work-groups) and the partial corrections of anti-diagonal K.  They
// touch disjoint parts of M: the correction of tile (I, K - I) reads M(I', K - I)
// for I' <= I, which the feedback of anti-diagonal K - 1 (tile (I', K - 1 - I')
// to J'' >= K + 1 - I') never writes.
__global__ __launch_bounds__(kTh) void fc2d_kernel(int m, int n, const float* __restrict__ UQ,
                                                   const float* __restrict__ UP, float* __restrict__ M,
                                                   const float* __restrict__ E, float* __restrict__ part, int Kf,
                                                   int lo_f, int ncc, int nfeed, int K, int lo, int nca, int Nb) {
  const int b = (int)blockIdx.x;
  if (b < nfeed)
    feed2d_body(b, m, n, UP, M, E, Kf, lo_f, Nb, ncc);
  else
    corr2d_body(b - nfeed, m, n, UQ, M, part, K, lo, nca);
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
    // feedback of anti-diagonal K - 1 past the right neighbours, in the same launch
    int lo_f = 0, ncc = 0, nfeed = 0;
    if (K >= 1) {
      const int Kf = K - 1, hi_f = std::min(Kf, Mb - 1);
      lo_f = std::max(0, Kf - Nb + 1);
      ncc = (Nb - (Kf - hi_f) - 2 + kChunk - 1) / kChunk;   // chunks of the leftmost tile
      nfeed = ncc > 0 ? (hi_f - lo_f + 1) * ncc : 0;
    }
    hipLaunchKernelGGL(fc2d_kernel, dim3(nfeed + ntile * nca), dim3(kTh), 0, s, (int)p.m, (int)p.n, UQ, UP, M, E,
                       cpart, K - 1, lo_f, std::max(ncc, 1), nfeed, K, lo, nca, Nb);
    if (x_dtype == 1)
      hipLaunchKernelGGL(tile2d_kernel<_Float16>, dim3(ntile), dim3(kTh), 0, s, (const _Float16*)X, ldx, (int)p.m,
                         (int)p.n, UQ, UP, M, E, cpart, gridv, maxq, codes, ldc, errp, K, lo, Nb, nca);
    else
      hipLaunchKernelGGL(tile2d_kernel<float>, dim3(ntile), dim3(kTh), 0, s, (const float*)X, ldx, (int)p.m,
                         (int)p.n, UQ, UP, M, E, cpart, gridv, maxq, codes, ldc, errp, K, lo, Nb, nca);
  }
  hipLaunchKernelGGL(err2d_kernel, dim3(1), dim3(kTh), 0, s, errp, p.Mb * p.Nb, out_err);
  return hipGetLastError();
}

}  // namespace gptq
