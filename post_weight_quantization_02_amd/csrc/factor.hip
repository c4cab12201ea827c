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
// diagonal -> one launch per 64-column block (blocked Cholesky with look-ahead;
// each diagonal block's inverse comes out of its factorization).  Up to 16
// blocks every step updates the whole trailing triangle.  From 17 to 96 blocks
// a block column receives the updates of all earlier steps late, two launches
// before its own factorization, as split-K partial products that the next
// launch folds in, so every launch carries about the same update work; past 96
// blocks the trailing updates of each step are confined to its group of eight
// blocks (512 columns), with one rank-512 update of the rest of the matrix
// after each group -> recursive-doubling triangular inverse, two batched fp32
// MFMA products per level -> reversed write of U.
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kNB = 64;
constexpr int kThreads = 256;
constexpr int kP = kNB + 1;  // LDS pitch (elements) of 64x64 tiles

// Output layout of v_mfma_f64_16x16x4f64: lane l, register r holds
// D[l / 16 + 4 r][l % 16] (checked on gfx950 against a host product).
__device__ __forceinline__ int f64_row(int lane, int r) { return (lane >> 4) + 4 * r; }

// A[i][j] = Hp[d-1-i][d-1-j] (+ lambda on the diagonal), lower 64x64 tiles only;
// Hp = H, or H with rows and columns taken in the order perm (Hp[a][b] =
// H[perm[a]][perm[b]]; indices clamped into range).  lambda = percdamp times
// the mean of diag(H) (the same under any perm), summed in fp64 by every
// diagonal-tile work-group in one fixed order, so all of them add the same
// value; work-group (0, 0) also writes lambda out and clears info.
__global__ __launch_bounds__(kThreads) void rev_copy_kernel(const float* __restrict__ H, int64_t d,
                                                            float percdamp,
                                                            const int32_t* __restrict__ perm,
                                                            double* __restrict__ A, float* lambda_out,
                                                            int32_t* info) {
  const int bj = blockIdx.x, bi = blockIdx.y;
  if (bj > bi) return;
  const int t = threadIdx.x;
  double lam = 0.0;
  if (bi == bj) {
    __shared__ double red[kThreads];
    double s = 0.0;
    for (int64_t i = t; i < d; i += kThreads) s += (double)H[i * (d + 1)];
    red[t] = s;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
      if (t < o) red[t] += red[t + o];
      __syncthreads();
    }
    lam = (double)percdamp * (red[0] / (double)d);
    if (bi == 0 && t == 0) {
      *lambda_out = (float)lam;
      *info = 0;
    }
  }
  const int64_t j = (int64_t)bj * 64 + (t & 63);
  for (int k = 0; k < 16; ++k) {
    const int64_t i = (int64_t)bi * 64 + (t >> 6) + 4 * k;
    if (i < d && j < d && j <= i) {
      int64_t si = d - 1 - i, sj = d - 1 - j;
      if (perm) {
        si = min<int64_t>(max<int32_t>(perm[si], 0), d - 1);
        sj = min<int64_t>(max<int32_t>(perm[sj], 0), d - 1);
      }
      double v = (double)H[si * d + sj];
      if (i == j) v += lam;
      A[i * d + j] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// One step of the blocked Cholesky (64-column blocks) with look-ahead.  Launch
// k (k = -1 .. nblk-2) runs independent work-groups of the kinds below; every
// input a work-group reads was finished by an earlier launch, so no work-group
// ever waits on another:
//   P  (rows r = k+1 .. nblk-1): apply step k to column block c = k+1 (tile
//      (r, c) and the diagonal tile (c, c)), factor the diagonal tile in LDS
//      (each P work-group redundantly), and solve its own tile:
//      L[r][c] = T Lcc^-T.  The r == c work-group writes Lcc^-1 as the
//      diagonal block of L^-1 (Lcc itself is never needed again).
// and either (deferred updates, 17 to 96 blocks)
//   RED (tiles (i, k+2), i >= k+2): A[i][k+2] -= (the partial products of steps
//      0 .. k-1 that the previous launch left, chunk by chunk) + L[i][k] L[k+2][k]^T,
//      which brings block column k+2 up to date for the next launch's P;
//   DEF (tiles (i, k+3), i >= k+3, one chunk of kDefSteps steps each): the
//      partial product  sum_{s in chunk} L[i][s] L[k+3][s]^T  of steps 0 .. k,
//      into this launch's half of a double buffer;
// block column j thus receives steps 0 .. j-3 as DEF products in launch j-3,
// folds them in with step j-2 in launch j-2 (RED), and takes step j-1 in the
// P work-groups of launch j-1.  No tile is written by two work-groups of one
// launch, and every launch's update work is about (rows left) x (steps done).
// or (right-looking updates: one group spanning the matrix up to 16 blocks,
// groups of eight blocks past 96)
//   UC (tiles (i, j), i >= j >= k+2, j < jend): A[i][j] -= L[i][k] L[j][k]^T
//      (fp64 MFMA); jend is the end of the step's column group, whose steps
//      reach the block columns past it in one rank-512 update instead.  The
//      first launch of a group (skip_step) finds step k already applied.
// ---------------------------------------------------------------------------
constexpr int kDefSteps = 4;        // steps per deferred partial product (K = 256)
constexpr int kDeferMinBlocks = 17;  // deferred updates from 17 to 96 blocks (1025 .. 6144 columns)
constexpr int kDeferMaxBlocks = 96;
inline bool deferred_updates(int64_t nblk) { return nblk >= kDeferMinBlocks && nblk <= kDeferMaxBlocks; }

struct StepArgs {
  double* A;
  float* Linv;
  int32_t* info;
  int d, nblk, k;
  int np, nuc, nred, ndef;
  int red_chunks;        // partial products RED folds in (chunks of the previous launch)
  const double* part_r;  // the previous launch's partial products
  double* part_w;        // this launch's
  int jend;       // update tiles only in block columns < jend
  int skip_step;  // step k already applied (by the column group's rank-512 update)
};

// C[m][n] (this wave's 32x32 quadrant) += sum_k SA[m][k] SB[n][k], fp64 MFMA
__device__ __forceinline__ void mma_nt_f64(const double* SA, const double* SB, f64x4 (&acc)[2][2],
                                           int lane, int wm, int wn) {
#pragma unroll 4
  for (int k4 = 0; k4 < kNB / 4; ++k4) {
    const int k = 4 * k4 + (lane >> 4);
    double a[2], b[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      a[f] = SA[(wm * 32 + f * 16 + (lane & 15)) * kP + k];
      b[f] = SB[(wn * 32 + f * 16 + (lane & 15)) * kP + k];
    }
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
  }
}

// tile coordinates held by acc[fm][fn][r] of mma_nt_f64
__device__ __forceinline__ int nt_row(int lane, int wm, int fm, int r) {
  return wm * 32 + fm * 16 + f64_row(lane, r);
}
__device__ __forceinline__ int nt_col(int lane, int wn, int fn) { return wn * 32 + fn * 16 + (lane & 15); }

__device__ __forceinline__ void zero_acc(f64x4 (&acc)[2][2]) {
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
}

// a 64x64 fp64 tile (rows R0.., cols C0..) into registers, zeros outside d
__device__ __forceinline__ void load_tile_regs(double (&v)[16], const double* __restrict__ A, int64_t d,
                                               int64_t R0, int64_t C0, int t) {
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int idx = t + u * kThreads;
    const int r = idx >> 6, c = idx & 63;
    v[u] = (R0 + r < d && C0 + c < d) ? A[(R0 + r) * d + C0 + c] : 0.0;
  }
}
__device__ __forceinline__ void store_tile_lds(double* S, const double (&v)[16], int t) {
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int idx = t + u * kThreads;
    S[(idx >> 6) * kP + (idx & 63)] = v[u];
  }
}

// load a 64x64 fp64 tile into LDS [row][col], zeros outside d.
// All global loads are issued before any LDS store (one memory round trip).
__device__ __forceinline__ void load_tile_f64(double* S, const double* __restrict__ A, int64_t d,
                                              int64_t R0, int64_t C0, int t) {
  double v[16];
  load_tile_regs(v, A, d, R0, C0, t);
  store_tile_lds(S, v, t);
}

// 1/x: the hardware estimate (relative error below 2^-22) refined by one
// Newton step (error squared: below 2^-44)
__device__ __forceinline__ double rcp_f64(double x) {
  const double r = __builtin_amdgcn_rcp(x);
  return fma(r, fma(-x, r, 1.0), r);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// ---------------------------------------------------------------------------
// Stacked LDL^T elimination of a 64-column block.
//
// S0 holds the symmetric diagonal block Dm (lower part; the upper part is free
// space), S1 holds 64 further rows T that receive the same eliminations (the
// rows of the block below the diagonal, or the identity).  Eliminating pivot j
// turns row i into row i - m_ij * (pivot row j), m_ij = a_ij / d_j; for the
// stacked rows that is Gaussian elimination of [Dm; T], whose multipliers are
//   m_T = T (D M^T)^-1,   M = unit lower factor of Dm = M D M^T.
// Hence T M^-T D^-1/2 = m_T D^1/2: the Cholesky tile of T, and for T = I the
// transpose of D^-1/2 M^-1, the inverse of the diagonal Cholesky factor.
//
// Pivots go in panels of 8 columns.  Wave 0 eliminates the diagonal block Dm
// alone, one row per lane in registers (pivot-row values by readlane:
// a_jc = a_cj sits in lane c), and stores
//   W  = pivot-time column values a_ij (i >= j) in the lower part of S0,
//   M^T in the upper part of S0 (row j, columns i > j); d_j is W's diagonal.
// Wave 0 stores without branches: a lane's store that has no place in S0 goes
// to its own slot of a sink array that nothing reads.
// The rank-8 update of Dm right of the panel runs on fp64 MFMA in 16x16 tiles:
// wave 0 takes the next 16 columns and goes on to the next panel at once.
// The stacked rows T follow one panel behind, off wave 0's path: each of waves
// 1-3 owns fixed 16-row blocks of T (wave 1 two, waves 2 and 3 one each), turns
// their panel columns into multipliers m_T by forward substitution with the
// panel's W and 1/d, and applies the rank-8 update to its own rows; waves 2 and
// 3 also take the Dm tiles right of the next 16 columns.  One barrier per panel;
// within a panel step no wave reads what another writes.
// ---------------------------------------------------------------------------
enum : int { kTileDm = 0, kTileT = 1, kTileNone = -1 };
struct TileDesc {
  int kind, R, C;
};

// C[R+m][C+n] -= sum_{k<8} A[R+m][J0+k] B[C+n][J0+k] for the tiles desc(0..NT-1);
// indices past 63 are clamped on load and masked on store.
template <int J0, int NT, typename Desc>
__device__ __forceinline__ void rank8_tiles(double* S0, double* S1, int lane, Desc desc) {
  double cv[NT][4], av[NT][2], bv[NT][2];
  TileDesc td[NT];
  const int m = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    td[u] = desc(u);
    const bool isT = td[u].kind == kTileT;
    const double* Cb = isT ? S1 : S0;
    const int am = min(td[u].R + m, kNB - 1), bn = min(td[u].C + m, kNB - 1);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      cv[u][r] = Cb[min(td[u].R + f64_row(lane, r), kNB - 1) * kP + bn];
#pragma unroll
    for (int k4 = 0; k4 < 2; ++k4) {
      const int k = J0 + 4 * k4 + kq;
      // A: M[i][k] = S0[k][i] (transposed multipliers) or m_T[i][k] = S1[i][k]
      av[u][k4] = -(isT ? S1[am * kP + k] : S0[k * kP + am]);
      bv[u][k4] = S0[bn * kP + k];  // W[c][k]
    }
  }
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    f64x4 acc = {cv[u][0], cv[u][1], cv[u][2], cv[u][3]};
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[u][0], bv[u][0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[u][1], bv[u][1], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) cv[u][r] = acc[r];
  }
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    if (td[u].kind == kTileNone) continue;
    const bool isT = td[u].kind == kTileT;
    double* Cb = isT ? S1 : S0;
    const int col = td[u].C + m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = td[u].R + f64_row(lane, r);
      if (row < kNB && col < kNB && (isT || col <= row)) Cb[row * kP + col] = cv[u][r];
    }
  }
}

// wave 0: eliminate panel P (columns 8P .. 8P+7) of Dm, one row per lane
template <int P>
__device__ __forceinline__ void ldl_dm_panel(double* S0, double* sink, int lane) {
  constexpr int J0 = 8 * P;
  double v[8], mu[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) v[c] = S0[lane * kP + J0 + c];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const double dj = readlane_f64(v[jj], J0 + jj);
    double s[8];
#pragma unroll
    for (int j2 = jj + 1; j2 < 8; ++j2) s[j2] = readlane_f64(v[jj], J0 + j2);  // a_{j, j2}
    const double rd = rcp_f64(dj);
    mu[jj] = (lane > J0 + jj) ? v[jj] * rd : 0.0;
#pragma unroll
    for (int j2 = jj + 1; j2 < 8; ++j2) v[j2] = fma(-mu[jj], s[j2], v[j2]);
  }
  // W (lower part, with d_j = W[j][j]), then M^T (upper part): disjoint places
#pragma unroll
  for (int c = 0; c < 8; ++c) *((lane >= J0 + c) ? &S0[lane * kP + J0 + c] : &sink[lane]) = v[c];
#pragma unroll
  for (int c = 0; c < 8; ++c) *((lane > J0 + c) ? &S0[(J0 + c) * kP + lane] : &sink[lane]) = mu[c];
}

// rows row0 .. row0 + nrows - 1 of T (one per lane): the same eliminations of
// panel P, t_j <- t_j / d_j, then t_j2 -= t_j a_{j, j2} (a_{j, j2} = W[j2][j]),
// leaving the multipliers m_T in the panel columns.  1/d_j is formed here from
// W's diagonal, as wave 0 formed it from the same d_j.
template <int P>
__device__ __forceinline__ void t_panel(const double* S0, double* S1, int lane, int row0, int nrows) {
  constexpr int J0 = 8 * P;
  if (lane >= nrows) return;
  double* r = S1 + (row0 + lane) * kP + J0;
  double tv[8], rd[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) tv[c] = r[c];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) rd[jj] = rcp_f64(S0[(J0 + jj) * kP + J0 + jj]);
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    tv[jj] *= rd[jj];
#pragma unroll
    for (int j2 = jj + 1; j2 < 8; ++j2) tv[j2] = fma(-tv[jj], S0[(J0 + j2) * kP + J0 + jj], tv[j2]);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) r[c] = tv[c];
}

// triangular index (a, b), 1 <= b <= a, in order (1,1) (2,1) (2,2) (3,1) ...
__device__ __forceinline__ void tri_ab(int i, int& a, int& b) {
  a = 1 + (i >= 1) + (i >= 3);
  b = i - (a - 1) * a / 2 + 1;
}

__device__ __forceinline__ void ldl_stacked(double* S0, double* S1, double* sink, int t) {
  const int lane = t & 63, w = t >> 6;
  if (w == 0) ldl_dm_panel<0>(S0, sink, lane);
  __syncthreads();
  static_for<0, kNB / 8>([&](auto PP) {
    constexpr int P = decltype(PP)::value;
    constexpr int J0 = 8 * P, T0 = J0 + 8;
    constexpr int nT = (kNB - T0 + 15) / 16;  // 16-wide column blocks right of the panel
    constexpr int nDm = nT * (nT - 1) / 2;    // Dm tiles outside column block 0
    if (w == 0) {
      if constexpr (nT > 0) {
        rank8_tiles<J0, nT>(S0, S1, lane, [&](int u) { return TileDesc{kTileDm, T0 + 16 * u, T0}; });
        ldl_dm_panel<P + 1>(S0, sink, lane);
      }
    } else if (w == 1) {
      t_panel<P>(S0, S1, lane, 0, 32);
      if constexpr (nT > 0)
        rank8_tiles<J0, 2 * nT>(S0, S1, lane, [&](int u) {
          return TileDesc{kTileT, 16 * (u / nT), T0 + 16 * (u % nT)};
        });
    } else {
      const int q = w;  // T rows 16 q .. 16 q + 15 (q = 2, 3)
      t_panel<P>(S0, S1, lane, 16 * q, 16);
      if constexpr (nT > 0)
        rank8_tiles<J0, nT + (nDm + 1) / 2>(S0, S1, lane, [&](int u) {
          if (u < nT) return TileDesc{kTileT, 16 * q, T0 + 16 * u};
          const int i = 2 * (u - nT) + (q - 2);
          if (i >= nDm) return TileDesc{kTileNone, 0, 0};
          int a, b;
          tri_ab(i, a, b);
          return TileDesc{kTileDm, T0 + 16 * a, T0 + 16 * b};
        });
    }
    __syncthreads();
  });
}

// ---------------------------------------------------------------------------
// acc (this wave's 32x32 quadrant of a 64x64 tile) +=
//   A[R0 .. R0+63][K0 .. K0+nk) A[C0 .. C0+63][K0 .. K0+nk)^T   (fp64 MFMA),
// rows past d read as zeros.  K is staged kGK columns at a time through S0 and
// S1 ([64][kGP] each, few registers live), the next stage loading into
// registers under the current products.  nk is a multiple of kGK; the LDS is
// free again on return.
// ---------------------------------------------------------------------------
constexpr int kGK = 32;       // K columns per stage
constexpr int kGP = kGK + 1;  // LDS pitch (doubles) of the [row][k] stages

__device__ __forceinline__ void mma_nt_stream(const double* __restrict__ A, int64_t d, int64_t R0, int64_t C0,
                                              int64_t K0, int nk, double* S0, double* S1, f64x4 (&acc)[2][2],
                                              int t) {
  const int lane = t & 63, w = t >> 6, wm = w & 1, wn = w >> 1;
  // staging: thread t covers row t / 4 of a [64][32] stage, columns 8 (t % 4) .. + 7
  const int sr = t >> 2, sc = 8 * (t & 3);
  double va[8], vb[8];
  auto gload = [&](double (&v)[8], int64_t row0, int64_t k0) {
    const int64_t row = row0 + sr;
    const bool ok = row < d;
    const double* src = A + (ok ? row : 0) * d + k0 + sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ok ? src[e] : 0.0;
  };
  gload(va, R0, K0);
  gload(vb, C0, K0);
  const int nst = nk / kGK;
  for (int st = 0; st < nst; ++st) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      S0[sr * kGP + sc + e] = va[e];
      S1[sr * kGP + sc + e] = vb[e];
    }
    __syncthreads();
    if (st + 1 < nst) {
      gload(va, R0, K0 + (int64_t)(st + 1) * kGK);
      gload(vb, C0, K0 + (int64_t)(st + 1) * kGK);
    }
#pragma unroll
    for (int k4 = 0; k4 < kGK / 4; ++k4) {
      const int k = 4 * k4 + (lane >> 4);
      double a[2], bb[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        a[f] = S0[(wm * 32 + f * 16 + (lane & 15)) * kGP + k];
        bb[f] = S1[(wn * 32 + f * 16 + (lane & 15)) * kGP + k];
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[fm], bb[fn], acc[fm][fn], 0, 0, 0);
    }
    __syncthreads();
  }
}

struct PanelSmem {
  double S0[kNB * kP], S1[kNB * kP];
  double sink[kNB], sq[kNB], rsq[kNB];   // sink: the LDL's discarded stores
  int fail;
};

// Step k applied to column block c1 = k+1, then the stacked elimination of
// [A[c1][c1]; A[r][c1]] (or [A[c1][c1]; I] for r == c1).
// S0: L[c1][k], then Dm.   S1: L[r][k], then T (or I), then m_T.
__device__ __forceinline__ void task_panel(const StepArgs a, int b, PanelSmem& sm) {
  // the panel chain is the critical path of the whole factorization: its waves
  // take issue priority over update work-groups sharing the CU
  __builtin_amdgcn_s_setprio(3);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w & 1, wn = w >> 1;
  const int64_t d = a.d;
  const int c1 = a.k + 1;
  const int r = c1 + b;
  const bool own = (r == c1);
  const int64_t R0 = (int64_t)r * kNB, C0 = (int64_t)c1 * kNB, K0 = (int64_t)a.k * kNB;
  const int nbe = (int)std::min<int64_t>(kNB, d - C0);
  // tiles A[c1][c1] (lower part) and A[r][c1] in the MFMA output layout; their
  // loads are in flight during the step-k product
  double gD[16], gT[16];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = (fm * 2 + fn) * 4 + q;
        const int rr = nt_row(lane, wm, fm, q), cc = nt_col(lane, wn, fn);
        gD[u] = (cc <= rr && rr < nbe) ? a.A[(C0 + rr) * d + C0 + cc] : 0.0;
        gT[u] = (!own && R0 + rr < d && cc < nbe) ? a.A[(R0 + rr) * d + C0 + cc] : 0.0;
      }
  f64x4 accD[2][2], accT[2][2];
  zero_acc(accD);
  zero_acc(accT);
  if (a.k >= 0 && !a.skip_step) {
    load_tile_f64(sm.S0, a.A, d, C0, K0, t);            // L[c1][k]
    if (!own) load_tile_f64(sm.S1, a.A, d, R0, K0, t);  // L[r][k]
    __syncthreads();
    mma_nt_f64(sm.S0, sm.S0, accD, lane, wm, wn);
    if (!own) mma_nt_f64(sm.S1, sm.S0, accT, lane, wm, wn);
    __syncthreads();
  }
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = (fm * 2 + fn) * 4 + q;
        const int rr = nt_row(lane, wm, fm, q), cc = nt_col(lane, wn, fn);
        // identity past the end of the matrix keeps the padded pivots at 1
        sm.S0[rr * kP + cc] = (rr < nbe) ? gD[u] - accD[fm][fn][q] : (rr == cc ? 1.0 : 0.0);
        sm.S1[rr * kP + cc] = own ? (rr == cc ? 1.0 : 0.0) : gT[u] - accT[fm][fn][q];
      }
  if (t == 0) sm.fail = kNB;
  __syncthreads();
  ldl_stacked(sm.S0, sm.S1, sm.sink, t);
  if (t < kNB) {
    const double dj = sm.S0[t * kP + t];
    if (!(dj > 0.0)) atomicMin(&sm.fail, t);
    sm.sq[t] = sqrt(dj);
    sm.rsq[t] = 1.0 / sm.sq[t];
  }
  __syncthreads();
  if (own) {
    // Lcc^-1 = (m_T D^1/2)^T, the diagonal block of L^-1.  Lcc itself is not
    // stored: nothing reads the diagonal blocks of L again, and the other panel
    // work-groups of this launch may still be reading A[c1][c1] (with more of
    // them than the GPU runs at once, late ones start after this one ends).
    // two adjacent columns per thread: 8-byte stores where d is even
    for (int idx = t; idx < kNB * kNB / 2; idx += kThreads) {
      const int i = idx >> 5, c = 2 * (idx & 31);
      if (C0 + i >= d) continue;
      float v[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) v[e] = (c + e <= i) ? (float)(sm.S1[(c + e) * kP + i] * sm.sq[i]) : 0.f;
      float* dst = a.Linv + (C0 + i) * d + C0 + c;
      if ((d & 1) == 0 && C0 + c + 1 < d) {
        *(float2*)dst = make_float2(v[0], v[1]);
      } else {
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (C0 + c + e < d) dst[e] = v[e];
      }
    }
    if (t == 0 && sm.fail < nbe && *a.info == 0) *a.info = (int32_t)(d - (C0 + sm.fail));
    return;
  }
  // L[r][c1] = m_T D^1/2, and its fp32 rounding at the same place of L^-1's
  // buffer: the block is read there by the one triangular-inverse product that
  // needs it, before the product after it overwrites the block with L^-1's.
  // Two adjacent columns per thread: 16- and 8-byte stores where d is even.
  for (int idx = t; idx < kNB * kNB / 2; idx += kThreads) {
    const int i = idx >> 5, c = 2 * (idx & 31);
    if (R0 + i >= d || c >= nbe) continue;
    double v[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) v[e] = sm.S1[i * kP + c + e] * sm.sq[c + e];
    double* da = a.A + (R0 + i) * d + C0 + c;
    float* dl = a.Linv + (R0 + i) * d + C0 + c;
    if ((d & 1) == 0 && c + 1 < nbe) {
      *(f64x2*)da = f64x2{v[0], v[1]};
      *(float2*)dl = make_float2((float)v[0], (float)v[1]);
    } else {
      da[0] = v[0];
      dl[0] = (float)v[0];
      if (c + 1 < nbe) {
        da[1] = v[1];
        dl[1] = (float)v[1];
      }
    }
  }
}

__device__ __forceinline__ void task_update_chol(const StepArgs a, int b, PanelSmem& sm) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w & 1, wn = w >> 1;
  const int64_t d = a.d;
  // tiles (i, j), j = 0 .. jend - base - 1, i = j .. nblk - base - 1, column by column
  const int base = a.k + 2, m = a.nblk - base;
  int j = 0;
  while (b >= m - j) {
    b -= m - j;
    ++j;
  }
  const int i = j + b;
  const int64_t R0 = (int64_t)(base + i) * kNB, C0 = (int64_t)(base + j) * kNB,
                K0 = (int64_t)a.k * kNB;
  load_tile_f64(sm.S0, a.A, d, R0, K0, t);
  load_tile_f64(sm.S1, a.A, d, C0, K0, t);
  __syncthreads();
  f64x4 acc[2][2];
  zero_acc(acc);
  double c[16];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = R0 + nt_row(lane, wm, fm, q), col = C0 + nt_col(lane, wn, fn);
        c[(fm * 2 + fn) * 4 + q] = (row < d && col <= row) ? a.A[row * d + col] : 0.0;
      }
  mma_nt_f64(sm.S0, sm.S1, acc, lane, wm, wn);
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = R0 + nt_row(lane, wm, fm, q), col = C0 + nt_col(lane, wn, fn);
        if (row < d && col <= row) a.A[row * d + col] = c[(fm * 2 + fn) * 4 + q] - acc[fm][fn][q];
      }
}

// Partial products keep each thread's 16 accumulator values in MFMA layout:
// value u of thread t at [u * kThreads + t] of the tile's 4096 doubles.
__device__ __forceinline__ int64_t part_tile(int chunk, int ntile, int ti) {
  return ((int64_t)chunk * ntile + ti) * (kNB * kNB);
}

// RED: tile row i = k+2+b of block column j = k+2
__device__ __forceinline__ void task_reduce(const StepArgs a, int b, PanelSmem& sm) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w & 1, wn = w >> 1;
  const int64_t d = a.d;
  const int j = a.k + 2, nt = a.nblk - j;
  const int64_t R0 = (int64_t)(j + b) * kNB, C0 = (int64_t)j * kNB, K0 = (int64_t)a.k * kNB;
  load_tile_f64(sm.S0, a.A, d, R0, K0, t);
  load_tile_f64(sm.S1, a.A, d, C0, K0, t);
  double c[16];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = R0 + nt_row(lane, wm, fm, q), col = C0 + nt_col(lane, wn, fn);
        c[(fm * 2 + fn) * 4 + q] = (row < d && col <= row) ? a.A[row * d + col] : 0.0;
      }
  // the deferred steps, chunk by chunk in step order
  for (int ch = 0; ch < a.red_chunks; ++ch) {
    const double* p = a.part_r + part_tile(ch, nt, b);
#pragma unroll
    for (int u = 0; u < 16; ++u) c[u] -= p[u * kThreads + t];
  }
  __syncthreads();
  f64x4 acc[2][2];
  zero_acc(acc);
  mma_nt_f64(sm.S0, sm.S1, acc, lane, wm, wn);
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = R0 + nt_row(lane, wm, fm, q), col = C0 + nt_col(lane, wn, fn);
        if (row < d && col <= row) a.A[row * d + col] = c[(fm * 2 + fn) * 4 + q] - acc[fm][fn][q];
      }
}

// DEF: block column j = k+3; work-group b takes tile row i = j + b % nt and
// steps [kDefSteps c, kDefSteps (c+1)) of 0 .. k, c = b / nt
__device__ __forceinline__ void task_deferred(const StepArgs a, int b, PanelSmem& sm) {
  const int t = threadIdx.x;
  const int j = a.k + 3, nt = a.nblk - j;
  const int ch = b / nt, ti = b % nt;
  const int s0 = ch * kDefSteps, s1 = std::min(s0 + kDefSteps, a.k + 1);
  f64x4 acc[2][2];
  zero_acc(acc);
  mma_nt_stream(a.A, a.d, (int64_t)(j + ti) * kNB, (int64_t)j * kNB, (int64_t)s0 * kNB, (s1 - s0) * kNB, sm.S0,
                sm.S1, acc, t);
  double* p = a.part_w + part_tile(ch, nt, ti);
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) p[((fm * 2 + fn) * 4 + q) * kThreads + t] = acc[fm][fn][q];
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void chol_step_kernel(StepArgs a) {
  __shared__ PanelSmem sm;
  int b = blockIdx.x;
  if (b < a.np) {
    task_panel(a, b, sm);
    return;
  }
  b -= a.np;
  if (b < a.nred) {
    task_reduce(a, b, sm);
    return;
  }
  b -= a.nred;
  if (b < a.ndef) {
    task_deferred(a, b, sm);
    return;
  }
  b -= a.ndef;
  if (b < a.nuc) task_update_chol(a, b, sm);
}

// ---------------------------------------------------------------------------
// The steps of one column group (blocks jb .. je-1) applied at once to the block
// columns past it: A[i][j] -= sum_s L[i][s] L[j][s]^T, je <= j <= i (fp64 MFMA,
// K = 64 (je - jb)).  One 64x64 tile per work-group, C read and written once
// after the products; 34 KB of LDS and few registers, so four work-groups share
// a CU.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void chol_group_update_kernel(
    double* __restrict__ A, int d, int jb, int je) {
  __shared__ double S0[kNB * kGP], S1[kNB * kGP];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w & 1, wn = w >> 1;
  const int b = blockIdx.x;
  int i = (int)((sqrt(8.0 * (double)b + 1.0) - 1.0) * 0.5);
  while ((i + 1) * (i + 2) / 2 <= b) ++i;
  while (i * (i + 1) / 2 > b) --i;
  const int j = b - i * (i + 1) / 2;
  const int64_t dd = d;
  const int64_t R0 = (int64_t)(je + i) * kNB, C0 = (int64_t)(je + j) * kNB;
  f64x4 acc[2][2];
  zero_acc(acc);
  mma_nt_stream(A, dd, R0, C0, (int64_t)jb * kNB, (je - jb) * kNB, S0, S1, acc, t);
  // C after the products (few registers live across the K loop)
  double c[16];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = R0 + nt_row(lane, wm, fm, q), col = C0 + nt_col(lane, wn, fn);
        c[(fm * 2 + fn) * 4 + q] = A[std::min(row, dd - 1) * dd + std::min(col, dd - 1)];
      }
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = R0 + nt_row(lane, wm, fm, q), col = C0 + nt_col(lane, wn, fn);
        if (row < dd && col <= row) A[row * dd + col] = c[(fm * 2 + fn) * 4 + q] - acc[fm][fn][q];
      }
}

// ---------------------------------------------------------------------------
// Triangular inverse L^-1 by recursive doubling over the 64-blocks (fp32 MFMA).
// A diagonal super-block [[A, 0], [B, C]] of L has the inverse
//   [[A^-1, 0], [-C^-1 B A^-1, C^-1]].
// Level sb (sb = 1, 2, 4, ... blocks) pairs A = blocks [2 p sb, 2 p sb + sb)
// with C = the next sb blocks (clipped at the end of the matrix).  With A^-1
// and C^-1 from the levels below it runs two batched products:
//   mode 0:  T = B A^-1   (B = L[C][A], the fp64 factor rounded to fp32, which
//                          the Cholesky left at the same place of L^-1's buffer; A^-1
//                          is lower triangular, so output block column j sums
//                          k = j .. sb-1)
//   mode 1:  X = -C^-1 T  (C^-1 lower: output block row i sums k = 0 .. i)
// X is L^-1[C][A]; T goes to a scratch buffer.  The one block that may stop
// short of d (the last) can only sit in a C range -- an A range there has no C
// and is skipped -- so masking rows and columns >= d of C is enough.
// ---------------------------------------------------------------------------
struct TriArgs {
  float* Linv;      // ld d
  float* Tw;        // scratch: pair p at p (64 sb)^2, ld 64 sb
  int64_t d;
  int nblk, sb, npairs;
  int nsub;         // output blocks per work-group (1, or 2 with complementary K ranges)
};

constexpr int kTK = kNB / 2;    // K per stage (half a block: small LDS, many work-groups per CU)
constexpr int kTPa = kTK + 1;   // LDS pitch of the [m][k] operand stage
constexpr int kTPb = kNB + 32;  // LDS pitch of the [k][n] operand stage (the two k rows of one read use disjoint banks)

template <int MODE, bool VEC>
__device__ __forceinline__ void tri_block(const TriArgs& a, float* SA, float* SB, int p, int bi, int bj, int A0,
                                          int C0) {
  const int sb = a.sb;
  const int64_t d = a.d;
  const int64_t ldt = (int64_t)kNB * sb;
  float* Tp = a.Tw + (int64_t)p * ldt * ldt;
  const int kb0 = (MODE == 0) ? bj : 0, kb1 = (MODE == 0) ? sb : bi + 1;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w & 1, wn = w >> 1;
  // K in stages of half a block: the A stage is [64 m][32 k] (thread t: row t / 4,
  // 8 k from 8 (t % 4)), the B stage [32 k][64 n] (thread t: k-row t / 8, 8 n from 8 (t % 8))
  const int ar = t >> 2, ac = 8 * (t & 3), br = t >> 3, bc = 8 * (t & 7);
  const int64_t arow = (int64_t)(C0 + bi) * kNB + ar;
  float ra[8], rb[8];
  auto gload = [&](int st) {
    const int kb = kb0 + (st >> 1), kh = (st & 1) * kTK;
    // A: mode 0 L[C0+bi][A0+kb] rounded to fp32 (in L^-1's buffer; columns inside
    // the A range, < d), mode 1 L^-1[C0+bi][C0+kb] (columns may pass d in the last block)
    const int64_t acol = (int64_t)((MODE == 0 ? A0 : C0) + kb) * kNB + kh + ac;
    const float* src = a.Linv + (arow < d ? arow : 0) * d + acol;
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      if (VEC && arow < d && (MODE == 0 || acol + e + 3 < d)) {
        const f32x4 v = *(const f32x4*)(src + e);
        ra[e] = v[0]; ra[e + 1] = v[1]; ra[e + 2] = v[2]; ra[e + 3] = v[3];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) ra[e + u] = (arow < d && acol + e + u < d) ? src[e + u] : 0.f;
      }
    }
    // B: mode 0 L^-1[A0+kb][A0+bj] (inside the A range), mode 1 T[kb][bj] of this pair
    const float* bsrc = (MODE == 0)
                            ? a.Linv + ((int64_t)(A0 + kb) * kNB + kh + br) * d + (int64_t)(A0 + bj) * kNB + bc
                            : Tp + ((int64_t)kb * kNB + kh + br) * ldt + (int64_t)bj * kNB + bc;
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      if (VEC) {
        const f32x4 v = *(const f32x4*)(bsrc + e);
        rb[e] = v[0]; rb[e + 1] = v[1]; rb[e + 2] = v[2]; rb[e + 3] = v[3];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) rb[e + u] = bsrc[e + u];
      }
    }
  };
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int nst = 2 * (kb1 - kb0);
  gload(0);
  for (int st = 0; st < nst; ++st) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) SA[ar * kTPa + ac + e] = ra[e];
#pragma unroll
    for (int e = 0; e < 8; e += 4)
      *(f32x4*)&SB[br * kTPb + bc + e] = f32x4{rb[e], rb[e + 1], rb[e + 2], rb[e + 3]};
    __syncthreads();
    if (st + 1 < nst) gload(st + 1);
#pragma unroll 8
    for (int kk = 0; kk < kTK / 2; ++kk) {
      const int k = 2 * kk + (lane >> 5);
      const float av = SA[(wm * 32 + (lane & 31)) * kTPa + k];
      const float bv = SB[k * kTPb + wn * 32 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
  }
  // v_mfma_f32_32x32x2f32 output: lane l, register r holds D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), col = wn * 32 + (lane & 31);
    if (MODE == 0) {
      Tp[((int64_t)bi * kNB + row) * ldt + (int64_t)bj * kNB + col] = acc[r];
    } else {
      const int64_t grow = (int64_t)(C0 + bi) * kNB + row;
      if (grow < d) a.Linv[grow * d + (int64_t)(A0 + bj) * kNB + col] = -acc[r];
    }
  }
}

// On levels with many blocks each work-group takes two output blocks whose
// triangular K ranges add up to sb + 1 blocks (block columns j and sb - 1 - j in
// mode 0, block rows i and sb - 1 - i in mode 1), so every work-group of the
// level carries the same work and no CU is left with the longest ranges; on
// the others one block each (longest ranges first).
template <int MODE, bool VEC>
__global__ __launch_bounds__(kThreads) void tri_gemm_kernel(TriArgs a) {
  __shared__ float SA[kNB * kTPa];
  __shared__ __attribute__((aligned(16))) float SB[kTK * kTPb];
  const int sb = a.sb, np = a.npairs;
  const int nsub = a.nsub;
  const int outer = blockIdx.x / (np * sb), rem = blockIdx.x % (np * sb);
  const int p = rem / sb, q = rem % sb;
  const int A0 = 2 * p * sb, C0 = A0 + sb;
  const int nC = min(sb, a.nblk - C0);
  for (int sub = 0; sub < nsub; ++sub) {
    const int o = (sub == 0) ? outer : sb - 1 - outer;
    const int bi = (MODE == 0) ? q : sb - 1 - o;
    const int bj = (MODE == 0) ? o : q;
    if (bi < nC) tri_block<MODE, VEC>(a, SA, SB, p, bi, bj, A0, C0);
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

namespace {
// Act-order (itwiki "GPTQ", practical variants: the columns with the largest
// Hessian diagonal are quantized first).  Column j goes to position
// #{i : key_i > key_j} with the 64-bit key (ord(diag_i) << 32) | ~i, where
// ord maps floats to unsigned integers in the same order (-0 taken as +0, NaN
// as -inf): descending diagonal, equal diagonals in ascending index order.
// The keys are distinct, so the ranks are always a permutation.
__device__ __forceinline__ uint64_t act_order_key(float v, uint32_t i) {
  if (v != v) v = -INFINITY;
  if (v == 0.f) v = 0.f;
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(~i);
}

constexpr int kRankTile = 128;    // columns j per work-group (one per thread)
constexpr int kKeyTile = 4096;    // keys staged in LDS at a time (32 KB)
__global__ __launch_bounds__(kRankTile) void act_order_rank_kernel(const float* __restrict__ H,
                                                                   int64_t d,
                                                                   int32_t* __restrict__ perm) {
  __shared__ __attribute__((aligned(16))) uint64_t key[kKeyTile];
  const int j = blockIdx.x * kRankTile + threadIdx.x;  // d <= 2^20
  const uint64_t kj = (j < d) ? act_order_key(H[(int64_t)j * (d + 1)], (uint32_t)j) : ~0ull;
  int rank = 0;
  for (int i0 = 0; i0 < d; i0 += kKeyTile) {
    __syncthreads();
    // this tile's keys: every thread's loads in flight together; entries past
    // d get key 0, below every real key, so they never count
    constexpr int kPer = kKeyTile / kRankTile;
    uint64_t kv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = i0 + threadIdx.x + u * kRankTile;
      kv[u] = (i < d) ? act_order_key(H[(int64_t)i * (d + 1)], (uint32_t)i) : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) key[threadIdx.x + u * kRankTile] = kv[u];
    __syncthreads();
    const int n = (int)min<int64_t>(kKeyTile, d - i0);
    const int n2 = (n + 1) & ~1;
#pragma unroll 8
    for (int u = 0; u < n2; u += 2) {
      const uint64_t a0 = key[u], a1 = key[u + 1];
      rank += (int)(a0 > kj) + (int)(a1 > kj);
    }
  }
  if (j < d) perm[rank] = j;
}
}  // namespace

hipError_t act_order_launch(const float* H, int64_t d, int32_t* perm, hipStream_t s) {
  hipLaunchKernelGGL(act_order_rank_kernel, dim3((unsigned)cdiv(d, kRankTile)), dim3(kRankTile), 0, s, H, d,
                     perm);
  return hipGetLastError();
}

// pairs of level sb of the recursive inverse (those whose C range is not empty)
static int64_t tri_pairs(int64_t nblk, int64_t sb) { return (nblk > sb) ? cdiv(nblk - sb, 2 * sb) : 0; }

FactorPlan factor_plan(int64_t d) {
  FactorPlan p{};
  p.d = d;
  p.nb = kNB;
  p.nblk = cdiv(d, kNB);
  // scratch for T: pair p at p (64 sb)^2; the last pair holds only its nC block rows
  size_t tw = 0;
  for (int64_t sb = 1; sb < p.nblk; sb *= 2) {
    const int64_t np = tri_pairs(p.nblk, sb);
    const int64_t nc_last = std::min<int64_t>(sb, p.nblk - ((np - 1) * 2 * sb + sb));
    const size_t e = (size_t)kNB * (size_t)sb;
    tw = std::max(tw, (size_t)(np - 1) * e * e + (size_t)nc_last * kNB * e);
  }
  // deferred partial products (up to 96 blocks): per launch k, nblk - k - 3
  // tiles of block column k+3 times cdiv(k + 1, kDefSteps) chunks, two launches'
  // worth (double buffer)
  size_t part_tiles = 0;
  if (deferred_updates(p.nblk))
    for (int64_t k = 0; k + 3 < p.nblk; ++k)
      part_tiles = std::max(part_tiles, (size_t)(p.nblk - k - 3) * (size_t)cdiv(k + 1, kDefSteps));
  p.part_slot = part_tiles * kNB * kNB;
  size_t off = 0;
  p.off_a64 = off;
  off = align_up(off + (size_t)d * d * sizeof(double), 256);
  p.off_part = off;
  off = align_up(off + 2 * p.part_slot * sizeof(double), 256);
  p.off_tw = off;
  off = align_up(off + tw * sizeof(float), 256);
  p.off_tmp = off;  // L^-1 (d*d fp32)
  off = align_up(off + (size_t)d * d * sizeof(float), 256);
  p.ws_bytes = off;
  return p;
}

hipError_t factor_launch(const FactorPlan& p, const float* H, const int32_t* perm, float percdamp,
                         float* U, float* lambda_out, int32_t* info, void* ws, hipStream_t s) {
  const int64_t d = p.d;
  char* base = (char*)ws;
  double* A = (double*)(base + p.off_a64);
  double* part = (double*)(base + p.off_part);
  float* Tw = (float*)(base + p.off_tw);
  float* Linv = (float*)(base + p.off_tmp);
  hipError_t e;
  const unsigned nt = (unsigned)p.nblk;
  hipLaunchKernelGGL(rev_copy_kernel, dim3(nt, nt), dim3(kThreads), 0, s, H, d, percdamp, perm, A, lambda_out,
                     info);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nblk = (int)p.nblk;
  if (deferred_updates(nblk)) {
    for (int k = -1; k <= nblk - 2; ++k) {
      StepArgs a{};
      a.A = A;
      a.Linv = Linv;
      a.info = info;
      a.d = (int)d;
      a.nblk = nblk;
      a.k = k;
      a.np = nblk - (k + 1);
      a.jend = nblk;
      // RED on block column k+2 with the chunks the previous launch's DEF wrote
      // (steps 0 .. k-1); DEF on block column k+3 with steps 0 .. k
      a.nred = (k >= 0 && k + 2 < nblk) ? nblk - (k + 2) : 0;
      a.red_chunks = (a.nred > 0 && k >= 1) ? (int)cdiv(k, kDefSteps) : 0;
      a.ndef = (k >= 0 && k + 3 < nblk) ? (nblk - (k + 3)) * (int)cdiv(k + 1, kDefSteps) : 0;
      a.part_w = part + (size_t)(k & 1) * p.part_slot;
      a.part_r = part + (size_t)((k + 1) & 1) * p.part_slot;
      hipLaunchKernelGGL(chol_step_kernel, dim3((unsigned)(a.np + a.nred + a.ndef)), dim3(kThreads), 0, s, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  } else {
    // up to 16 blocks every step updates the whole trailing triangle (measured:
    // 2% faster than the deferred scheme at 512 columns, equal at 1024); past
    // 96 blocks groups of 8 blocks (512 columns): each step updates the tiles of
    // its own group, and one rank-512 update per group reaches the rest of the
    // matrix (the deferred launches would outgrow the panel chain there)
    const int kGroup = nblk > kDeferMaxBlocks ? 8 : nblk;
    for (int jb = 0; jb < nblk; jb += kGroup) {
      const int je = std::min(jb + kGroup, nblk);
      for (int k = jb - 1; k < je - 1; ++k) {
        StepArgs a{};
        a.A = A;
        a.Linv = Linv;
        a.info = info;
        a.d = (int)d;
        a.nblk = nblk;
        a.k = k;
        a.np = nblk - (k + 1);
        a.jend = je;
        a.skip_step = (jb > 0 && k == jb - 1) ? 1 : 0;
        const int m = nblk - (k + 2);  // block rows past column k+1
        const int w = je - (k + 2);    // block columns of the group past column k+1
        a.nuc = (k >= 0 && !a.skip_step && w > 0) ? w * m - w * (w - 1) / 2 : 0;
        hipLaunchKernelGGL(chol_step_kernel, dim3((unsigned)(a.np + a.nuc)), dim3(kThreads), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      if (je < nblk) {
        const int m = nblk - je;
        hipLaunchKernelGGL(chol_group_update_kernel, dim3((unsigned)(m * (m + 1) / 2)), dim3(kThreads), 0, s, A,
                           (int)d, jb, je);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
  }
  const bool vec = (d % 4) == 0;
  for (int64_t sb = 1; sb < p.nblk; sb *= 2) {
    TriArgs t{Linv, Tw, d, nblk, (int)sb, (int)tri_pairs(p.nblk, sb), 1};
    // two blocks per work-group from 1024 blocks (four per CU) up: measured 1-2%
    // faster factors at 4096-12288 columns (U bitwise the same), and 2-5% slower
    // at 512-2048 columns when the smaller levels were paired too
    t.nsub = (sb >= 2 && (int64_t)t.npairs * sb * sb >= 1024) ? 2 : 1;
    const dim3 grid((unsigned)(t.npairs * sb * (sb / t.nsub)));
    if (vec) {
      hipLaunchKernelGGL((tri_gemm_kernel<0, true>), grid, dim3(kThreads), 0, s, t);
      hipLaunchKernelGGL((tri_gemm_kernel<1, true>), grid, dim3(kThreads), 0, s, t);
    } else {
      hipLaunchKernelGGL((tri_gemm_kernel<0, false>), grid, dim3(kThreads), 0, s, t);
      hipLaunchKernelGGL((tri_gemm_kernel<1, false>), grid, dim3(kThreads), 0, s, t);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(rev_out_kernel, dim3(nt, nt), dim3(kThreads), 0, s, Linv, d, U);
  return hipGetLastError();
}

}  // namespace gptq
