// Hessian accumulation H += 2 X^T X on gfx950 matrix cores.
//
// Blog "GPTQ를 밑바닥부터 구현하며 배운 것들", section 3: H = 2 X^T X over the
// calibration inputs; itwiki "GPTQ", minimal implementation: the same line.
//
// Design (MI355X): only the upper triangle of square tiles is computed.  The
// calibration rows are split into row ranges ("splits"); every (tile, split)
// pair is one work-group that accumulates in fp32 on MFMA and writes a partial
// tile.  A reduce kernel adds the partials in split order (bitwise
// reproducible, no float atomics), scales by 2, adds to H and mirrors the
// tile into the lower triangle through LDS so both triangles are written with
// coalesced stores.
//
// fp16 X: v_mfma_f32_32x32x16_f16, 256x256 tiles, 64 rows per stage.  X is
// stored row-major (features contiguous), the MFMA wants 8 consecutive rows
// per lane, so each thread loads an 8x8 block (8 rows x 16 bytes), transposes
// it in registers and writes 8 features' 16-byte row chunks to LDS.  LDS rows
// are 128 bytes; the 16-byte chunk c of feature m is stored at chunk
// c ^ ((m ^ (m >> 3)) & 7), which keeps both these staging writes (lanes 8
// features apart) and the fragment reads (consecutive features) free of bank
// conflicts.
// fp32 X: v_mfma_f32_32x32x2f32 reads one row value per lane, so the natural
// [row][feature] LDS layout needs no transpose; 128x128 tiles.
#include "gptq_internal.h"

#include <numeric>

namespace gptq {
namespace {

constexpr int kThreads = 256;

// upper-triangle tile enumeration t = tj (tj + 1) / 2 + ti with ti <= tj
__device__ __forceinline__ void tile_of(int64_t t, int& ti, int& tj) {
  int j = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while ((int64_t)(j + 1) * (j + 2) / 2 <= t) ++j;
  while ((int64_t)j * (j + 1) / 2 > t) --j;
  tj = j;
  ti = (int)(t - (int64_t)j * (j + 1) / 2);
}

// work-group -> (tile, split).  Splits are visited in order by the whole GPU
// (split-major), so at any time the running work-groups read the same few
// split row ranges and those stay in the Infinity Cache while every tile
// passes over them.  When the tile count is a multiple of 8, XCD x (work-groups
// are dispatched round-robin over the 8 XCDs) takes the contiguous tile range
// [x * ntiles / 8, (x + 1) * ntiles / 8) of each split, so tiles that share
// column blocks share that XCD's L2.
__device__ __forceinline__ void wg_map(int64_t ntiles, int64_t nsplit, int64_t& tile,
                                       int64_t& split) {
  const int64_t bid = blockIdx.x;
  if ((ntiles & 7) == 0) {
    const int64_t per = ntiles >> 3;
    const int64_t j = bid >> 3;
    split = j / per;
    tile = (bid & 7) * per + j % per;
  } else {
    split = bid / ntiles;
    tile = bid % ntiles;
  }
}

// ------------------------------------------------------------------ fp16
constexpr int kBT16 = 256, kKS16 = 64;

__device__ __forceinline__ int sw16(int m, int c) {
  return m * kKS16 + ((c ^ ((m ^ (m >> 3)) & 7)) << 3);
}

// Software pipeline per 64-row stage s (LDS double-buffered, one barrier):
//   k-substep 0..3 each issue 16 MFMAs (this wave's 4x4 32x32 fragments) with
//   the next substep's fragments read from LDS underneath;
//   substep 1 also transposes the registers holding stage s+1 into LDS buffer
//   (s+1)&1, substep 2 issues the global loads of stage s+2 into those
//   registers; the barrier sits between substeps 2 and 3 so that substep 3 can
//   already read stage s+1's first fragments.  sched_group_barrier pins the
//   interleave (one MFMA, then a few memory or transpose instructions).
// Full stages load unmasked from a uniform per-stage base with 32-bit offsets;
// only a split's tail stage (or a partial last column tile) takes the masked
// path.
#define GPTQ_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
constexpr int kSgMFMA = 0x008, kSgVALU = 0x002, kSgVMEMR = 0x020, kSgDSR = 0x100, kSgDSW = 0x200;

template <bool VEC>
__global__ __launch_bounds__(kThreads) void syrk_f16_kernel(
    const _Float16* __restrict__ X, int64_t ldx, int64_t n, int d, int64_t ntiles,
    int64_t nsplit, int64_t rps, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[2][2][kBT16 * kKS16];
  int64_t tile, split;
  wg_map(ntiles, nsplit, tile, split);
  int ti, tj;
  tile_of(tile, ti, tj);
  const bool diag = (ti == tj);
  const int I0 = ti * kBT16, J0 = tj * kBT16;
  const int64_t r0 = split * rps;
  const int64_t r1 = min(n, r0 + rps);
  const int nrows = (int)(r1 - r0);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int mg = t & 31, kg = t >> 5;
  const bool full_cols = VEC && (I0 + kBT16 <= d) && (J0 + kBT16 <= d);
  const _Float16* __restrict__ Xs = X + r0 * ldx;   // this split's first row
  const uint32_t offA = (uint32_t)(kg * 8 * ldx + I0 + mg * 8);
  const uint32_t offB = (uint32_t)(kg * 8 * ldx + J0 + mg * 8);
  const uint32_t ld32 = (uint32_t)ldx;

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  half8 ra[8], rb[8];
  auto gload_fast = [&](int st, uint32_t off, half8* r) {
    const _Float16* __restrict__ p = Xs + (int64_t)(st * kKS16) * ldx;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = *(const half8*)(p + off + i * ld32);
  };
  auto gload_masked = [&](int st, int col0, half8* r) {
    const int k0 = st * kKS16;
    const int col = col0 + mg * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = k0 + kg * 8 + i;
      const bool ok = row < nrows;
      const int64_t rowc = ok ? row : 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool cok = col + e < d;
        const _Float16 v = Xs[rowc * ldx + (cok ? col + e : 0)];
        r[i][e] = (ok && cok) ? v : (_Float16)0.f;
      }
    }
  };
  auto lstore = [&](_Float16* L, const half8* r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      half8 v;
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = r[k][i];
      *(half8*)(L + sw16(mg * 8 + i, kg)) = v;
    }
  };
  auto frags = [&](const _Float16* LA, const _Float16* LB, int kk, half8* fa, half8* fb) {
    const int c = 2 * kk + (lane >> 5);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      fa[f] = *(const half8*)(LA + sw16(wm * 128 + f * 32 + (lane & 31), c));
      fb[f] = *(const half8*)(LB + sw16(wn * 128 + f * 32 + (lane & 31), c));
    }
  };
  auto mfmas = [&](const half8* fa, const half8* fb) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[fm], fb[fn], acc[fm][fn], 0, 0, 0);
  };

  // full stages: pipelined, unmasked; indices are clamped so that every
  // iteration runs the same straight-line code (surplus loads/stores at the end
  // touch valid memory and an LDS buffer nobody reads afterwards)
  const int nfull = full_cols ? nrows / kKS16 : 0;
  half8 fa[2][4], fb[2][4];
  if (nfull > 0) {
    gload_fast(0, offA, ra);
    if (!diag) gload_fast(0, offB, rb);
    lstore(lds[0][0], ra);
    if (!diag) lstore(lds[0][1], rb);
    __syncthreads();
    const int s1 = nfull > 1 ? 1 : 0;
    gload_fast(s1, offA, ra);
    if (!diag) gload_fast(s1, offB, rb);
    frags(lds[0][0], diag ? lds[0][0] : lds[0][1], 0, fa[0], fb[0]);
  }
  for (int s = 0; s < nfull; ++s) {
    const int cur = s & 1;
    const _Float16* LA = lds[cur][0];
    const _Float16* LB = diag ? lds[cur][0] : lds[cur][1];
    const _Float16* NA = lds[cur ^ 1][0];
    const _Float16* NB = diag ? lds[cur ^ 1][0] : lds[cur ^ 1][1];
    const int s2 = min(s + 2, nfull - 1);
    // substep 0
    frags(LA, LB, 1, fa[1], fb[1]);
    mfmas(fa[0], fb[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) { GPTQ_SGB(kSgMFMA, 1); GPTQ_SGB(kSgDSR, 1); }
    GPTQ_SGB(kSgMFMA, 8);
    // substep 1: + transpose stage s+1 into the other buffer
    frags(LA, LB, 2, fa[0], fb[0]);
    lstore(lds[cur ^ 1][0], ra);
    if (!diag) lstore(lds[cur ^ 1][1], rb);
    mfmas(fa[1], fb[1]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      GPTQ_SGB(kSgMFMA, 1);
      if (i < 8) GPTQ_SGB(kSgDSR, 1);
      GPTQ_SGB(kSgVALU, 4);
      GPTQ_SGB(kSgDSW, 1);
    }
    // substep 2: + global loads of stage s+2
    frags(LA, LB, 3, fa[1], fb[1]);
    gload_fast(s2, offA, ra);
    if (!diag) gload_fast(s2, offB, rb);
    mfmas(fa[0], fb[0]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      GPTQ_SGB(kSgMFMA, 1);
      if (i < 8) GPTQ_SGB(kSgDSR, 1);
      GPTQ_SGB(kSgVMEMR, 1);
      GPTQ_SGB(kSgVALU, 2);
    }
    __syncthreads();
    // substep 3: + first fragments of stage s+1
    frags(NA, NB, 0, fa[0], fb[0]);
    mfmas(fa[1], fb[1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) { GPTQ_SGB(kSgMFMA, 1); GPTQ_SGB(kSgDSR, 1); }
    GPTQ_SGB(kSgMFMA, 8);
  }
  // tail stages (partial rows or partial column tiles): masked, not pipelined
  const int nst = (nrows + kKS16 - 1) / kKS16;
  for (int s = nfull; s < nst; ++s) {
    __syncthreads();
    gload_masked(s, I0, ra);
    if (!diag) gload_masked(s, J0, rb);
    lstore(lds[0][0], ra);
    if (!diag) lstore(lds[0][1], rb);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      frags(lds[0][0], diag ? lds[0][0] : lds[0][1], kk, fa[0], fb[0]);
      mfmas(fa[0], fb[0]);
    }
  }
  float* P = part + (split * ntiles + tile) * (int64_t)(kBT16 * kBT16);
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 128 + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * 128 + fn * 32 + (lane & 31);
        P[row * kBT16 + col] = acc[fm][fn][r];
      }
}

// ------------------------------------------------------------------ fp32
constexpr int kBT32 = 128, kKS32 = 16, kP32 = kBT32 + 4;

template <bool VEC>
__global__ __launch_bounds__(kThreads) void syrk_f32_kernel(
    const float* __restrict__ X, int64_t ldx, int64_t n, int d, int64_t ntiles, int64_t nsplit,
    int64_t rps, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float lds[2][kKS32 * kP32];
  int64_t tile, split;
  wg_map(ntiles, nsplit, tile, split);
  int ti, tj;
  tile_of(tile, ti, tj);
  const bool diag = (ti == tj);
  const int I0 = ti * kBT32, J0 = tj * kBT32;
  const int64_t r0 = split * rps;
  const int64_t r1 = min(n, r0 + rps);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w & 1, wn = w >> 1;
  const int c4 = t & 31, rr = t >> 5;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  f32x4 ra[2], rb[2];
  auto gload = [&](int64_t k0, int col0, f32x4* r) {
    const int col = col0 + c4 * 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t row = k0 + rr + 8 * i;
      if (VEC) {
        if (row < r1 && col < d) r[i] = *(const f32x4*)(X + row * ldx + col);
        else r[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[i][e] = (row < r1 && col + e < d) ? X[row * ldx + col + e] : 0.f;
      }
    }
  };
  auto lstore = [&](float* L, const f32x4* r) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *(f32x4*)(L + (rr + 8 * i) * kP32 + c4 * 4) = r[i];
  };

  const int64_t nst = (r1 > r0) ? (r1 - r0 + kKS32 - 1) / kKS32 : 0;
  if (nst > 0) {
    gload(r0, I0, ra);
    if (!diag) gload(r0, J0, rb);
  }
  for (int64_t s = 0; s < nst; ++s) {
    lstore(lds[0], ra);
    if (!diag) lstore(lds[1], rb);
    __syncthreads();
    if (s + 1 < nst) {
      gload(r0 + (s + 1) * kKS32, I0, ra);
      if (!diag) gload(r0 + (s + 1) * kKS32, J0, rb);
    }
    const float* LA = lds[0];
    const float* LB = diag ? lds[0] : lds[1];
#pragma unroll
    for (int kk = 0; kk < kKS32 / 2; ++kk) {
      const int k = 2 * kk + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        a[f] = LA[k * kP32 + wm * 64 + f * 32 + (lane & 31)];
        b[f] = LB[k * kP32 + wn * 64 + f * 32 + (lane & 31)];
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
    __syncthreads();
  }
  float* P = part + (split * ntiles + tile) * (int64_t)(kBT32 * kBT32);
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * 64 + fn * 32 + (lane & 31);
        P[row * kBT32 + col] = acc[fm][fn][r];
      }
}

// ------------------------------------------------------------------ reduce
// One work-group per 64x64 sub-block of an upper tile: H_sub += 2 * sum over
// splits (fixed order), and the mirror H_sub^T into the lower triangle.  On a
// diagonal tile only its upper triangle is used, so H stays exactly symmetric.
__global__ __launch_bounds__(kThreads) void syrk_reduce_kernel(
    const float* __restrict__ part, int64_t ntiles, int64_t nsplit, int bt, int d,
    float* __restrict__ H) {
  __shared__ float tr[64][65];
  const int nsub = bt / 64;
  const int64_t b = blockIdx.x;
  const int64_t tile = b / (nsub * nsub);
  const int sb = (int)(b % (nsub * nsub));
  const int sa = sb / nsub, sc = sb % nsub;
  int ti, tj;
  tile_of(tile, ti, tj);
  const bool diag = (ti == tj);
  if (diag && sa > sc) return;
  const bool subdiag = diag && sa == sc;
  const int64_t R0 = (int64_t)ti * bt + sa * 64, C0 = (int64_t)tj * bt + sc * 64;
  const int t = threadIdx.x;
  const int col = t & 63;
  const int64_t tsz = (int64_t)bt * bt;
  for (int i = 0; i < 16; ++i) {
    const int row = (t >> 6) + 4 * i;
    const float* p = part + tile * tsz + (int64_t)(sa * 64 + row) * bt + sc * 64 + col;
    float s = 0.f;
    for (int64_t sp = 0; sp < nsplit; ++sp) s += p[sp * ntiles * tsz];
    s *= 2.f;
    if (R0 + row < d && C0 + col < d && (!subdiag || row <= col)) H[(R0 + row) * d + C0 + col] += s;
    tr[row][col] = s;
  }
  __syncthreads();
  for (int i = 0; i < 16; ++i) {
    const int orow = t & 63;            // row of the upper element
    const int ocol = (t >> 6) + 4 * i;  // its column
    if (subdiag && !(orow < ocol)) continue;
    if (C0 + ocol < d && R0 + orow < d) H[(C0 + ocol) * d + R0 + orow] += tr[orow][ocol];
  }
}

}  // namespace

HessianPlan hessian_plan(int64_t d, int64_t n, int dtype) {
  HessianPlan p{};
  p.dtype = dtype;
  p.bt = (dtype == 1) ? kBT16 : kBT32;
  const int ks = (dtype == 1) ? kKS16 : kKS32;
  p.tiles_side = cdiv(d, p.bt);
  p.ntiles = p.tiles_side * (p.tiles_side + 1) / 2;
  if (n <= 0) {
    p.nsplit = 0;
    p.rows_per_split = 0;
    p.ws_bytes = 0;
    return p;
  }
  // At most 16384 rows per split (short fp32 accumulation chains).  When that
  // gives fewer than 16 rounds of work-groups over the 256 CUs, the split count
  // is raised to make tiles x splits a whole number of rounds (no idle tail),
  // keeping >= 2048 rows per split; each split's rows stay cache-resident while
  // all tiles pass over them.
  const int64_t cus = 256;
  const int64_t ns0 = cdiv(n, 16384);
  int64_t ns = ns0;
  if (p.ntiles * ns0 < 16 * cus) {
    const int64_t unit = cus / std::gcd<int64_t>(p.ntiles, cus);
    ns = cdiv(ns0, unit) * unit;
    const int64_t cap = std::max<int64_t>(1, cdiv(n, 2048));
    if (ns > cap) ns = std::max(ns0, std::min(cap, std::max<int64_t>(1, cdiv(4 * cus, p.ntiles))));
  }
  int64_t rps = cdiv(n, ns);
  rps = cdiv(rps, ks) * ks;
  const int64_t rps_max = std::max<int64_t>(ks, ((int64_t(1) << 31) / std::max<int64_t>(d, 1)) / ks * ks);
  rps = std::min(rps, rps_max);
  p.rows_per_split = rps;
  p.nsplit = cdiv(n, rps);
  p.ws_bytes = (size_t)p.nsplit * (size_t)p.ntiles * (size_t)p.bt * (size_t)p.bt * sizeof(float);
  return p;
}

hipError_t hessian_launch(const HessianPlan& p, float* H, int64_t d, const void* X, int64_t n,
                          int64_t ldx, void* ws, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  float* part = (float*)ws;
  const int64_t grid = p.ntiles * p.nsplit;
  if (p.dtype == 1) {
    const bool vec = (d % 8 == 0) && (ldx % 8 == 0) && (((uintptr_t)X & 15) == 0);
    if (vec)
      hipLaunchKernelGGL(syrk_f16_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         (const _Float16*)X, ldx, n, (int)d, p.ntiles, p.nsplit, p.rows_per_split, part);
    else
      hipLaunchKernelGGL(syrk_f16_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         (const _Float16*)X, ldx, n, (int)d, p.ntiles, p.nsplit, p.rows_per_split, part);
  } else {
    const bool vec = (d % 4 == 0) && (ldx % 4 == 0) && (((uintptr_t)X & 15) == 0);
    if (vec)
      hipLaunchKernelGGL(syrk_f32_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         (const float*)X, ldx, n, (int)d, p.ntiles, p.nsplit, p.rows_per_split, part);
    else
      hipLaunchKernelGGL(syrk_f32_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         (const float*)X, ldx, n, (int)d, p.ntiles, p.nsplit, p.rows_per_split, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nsub = p.bt / 64;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)(p.ntiles * nsub * nsub)), dim3(kThreads),
                     0, s, part, p.ntiles, p.nsplit, p.bt, (int)d, H);
  return hipGetLastError();
}

}  // namespace gptq
