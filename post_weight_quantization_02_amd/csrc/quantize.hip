// The lazy-batch quantization loop (itwiki "GPTQ": Algorithm 1, minimal
// implementation, practical variants / group quantization).
//
//   grid  per row from W0 (scale = max(max - min, 1e-8) / maxq, zero =
//         round(-min / scale)), or per group from the current weights when
//         the group's first column is reached;
//   panel for each column j of a block: c = clamp(round(w/scale) + zero, 0,
//         maxq); e = (w - scale (c - zero)) / U[j,j]; W[:, j:] -= e U[j, j:]
//         inside the block; E[:, j] = e;
//   GEMM  W[:, i+B:] -= E U[i:i+B, i+B:]  (gemm.hip; E is kept transposed);
//   error ||X dW^T||^2 = 1/2 ||E||^2 - lambda/2 ||dW||^2 (the damped objective
//         is 1/2 ||E||^2 by the OBS increment of the wiki's OBQ equation).
//
// Panel layout (gfx950): rows are independent (all rows share U, the wiki's
// change 1), so a wave holds 4 rows and each row is spread over a 16-lane DPP
// row, 8 consecutive block columns per lane (B = 128).  Per column the owner
// lane's scaled error reaches the other 15 lanes of its row with one DPP
// row_newbcast, and every lane applies the rank-1 update to its own columns
// with U[j, :] read from LDS (the block's diagonal part of U lives there),
// prefetched a few columns ahead so the serial column chain never waits on LDS.
// Per-group min/max is a 16-lane butterfly.  No block-wide barrier is needed
// after U is staged.
#include "gptq_internal.h"

#include <mutex>

namespace gptq {
namespace {

constexpr int kThreads = 256;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// lane (16 * (lane / 16) + K) of the caller's DPP row, broadcast to the row
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  // every lane is written (full row and bank masks), so no old value is kept
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + K, 0xF, 0xF, true));
}

__device__ __forceinline__ void grid_from_minmax(float mn, float mx, int maxq, float& s, float& z) {
  s = fmaxf(mx - mn, 1e-8f) / (float)maxq;
  z = rintf(-mn / s);
}

__global__ void zero_f64_kernel(double* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0;
}

// a column index from a caller's permutation, clamped into range
__device__ __forceinline__ int64_t perm_col(const int32_t* __restrict__ perm, int64_t c, int64_t d_col) {
  return perm ? min<int64_t>(max<int32_t>(perm[c], 0), d_col - 1) : c;
}

// fp32 working copy of W0 (column c of the copy is column perm[c] of W0 when a
// quantization order is given); with a per-row grid also that row's scale / zero
template <typename T>
__global__ __launch_bounds__(kThreads) void prep_kernel(const T* __restrict__ W0, int64_t ldw,
                                                        int64_t d_col, const int32_t* __restrict__ perm,
                                                        float* __restrict__ W,
                                                        int per_row, int maxq,
                                                        float* __restrict__ scales,
                                                        int32_t* __restrict__ zeros, int vec8) {
  __shared__ float smn[kThreads], smx[kThreads];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  float mn = INFINITY, mx = -INFINITY;
  // natural order with 16-byte (fp16) or 32-byte (fp32) aligned rows: 8 columns
  // per thread and step
  for (int64_t c = 8 * (int64_t)t; vec8 && c < d_col; c += 8 * kThreads) {
    f32x4 v0, v1;
    if constexpr (sizeof(T) == 2) {
      typedef _Float16 h8 __attribute__((ext_vector_type(8)));
      const h8 x = *(const h8*)(W0 + row * ldw + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[e] = (float)x[e];
        v1[e] = (float)x[e + 4];
      }
    } else {
      v0 = *(const f32x4*)(W0 + row * ldw + c);
      v1 = *(const f32x4*)(W0 + row * ldw + c + 4);
    }
    *(f32x4*)(W + row * d_col + c) = v0;
    *(f32x4*)(W + row * d_col + c + 4) = v1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mn = fminf(mn, fminf(v0[e], v1[e]));
      mx = fmaxf(mx, fmaxf(v0[e], v1[e]));
    }
  }
  for (int64_t c = t; !vec8 && c < d_col; c += kThreads) {
    const float v = (float)W0[row * ldw + perm_col(perm, c, d_col)];
    W[row * d_col + c] = v;
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  if (!per_row) return;
  smn[t] = mn;
  smx[t] = mx;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (t < o) {
      smn[t] = fminf(smn[t], smn[t + o]);
      smx[t] = fmaxf(smx[t], smx[t + o]);
    }
    __syncthreads();
  }
  if (t == 0) {
    float s, z;
    grid_from_minmax(smn[0], smx[0], maxq, s, z);
    scales[row] = s;
    zeros[row] = (int32_t)z;
  }
}

// group grid for groups wider than the block, at a block start: one wave per row
__global__ __launch_bounds__(kThreads) void group_grid_kernel(const float* __restrict__ W,
                                                              int64_t d_row, int64_t d_col,
                                                              int64_t g0, int64_t gw, int64_t gi,
                                                              int64_t ngroups, int maxq,
                                                              float* __restrict__ scales,
                                                              int32_t* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= d_row) return;
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t c = g0 + lane; c < g0 + gw; c += 64) {
    const float v = W[row * d_col + c];
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, 64));
    mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  }
  if (lane == 0) {
    float s, z;
    grid_from_minmax(mn, mx, maxq, s, z);
    scales[row * ngroups + gi] = s;
    zeros[row * ngroups + gi] = (int32_t)z;
  }
}

// One block of columns [i1, i1 + width) for 16 rows per work-group.
// GIN: group size when groups start inside the block (a multiple of 16 that
// divides B), else 0 (per-row grid, or groups wider than the block whose
// parameters group_grid_kernel wrote at the block start).  FULL: width == B.
// Both are compile-time so the fully unrolled column loop carries the group
// code only at the group starts.
// Blocks paired in the out-of-block correction: the previous block's share
// W[:, i1:i1+width] -= E_prev U[i1-B:i1, i1:i1+width] is applied by the
// work-group to its own rows before the column loop, with E_prev either read
// from memory (kEprevMem: Eprev, NULL when there is no share) or, when the same
// work-group has just quantized those rows through the previous block, taken
// from each lane's errors in registers (kEprevRegs: er on entry).
enum { kEprevMem = 0, kEprevRegs = 1 };

// LDS of one block: U's diagonal block, the per-wave strips of the share
// (blocks of 128), 1/U_jj, the error reduction
template <int CPL>
struct PanelLds {
  static constexpr int B = 16 * CPL;
  float Us[B * B];
  float dl[CPL == 8 ? 16 * B : 4];
  float rd[B];
  double red[kThreads / 64];
};

template <int CPL, int GIN, bool FULL, int EMODE, bool PRE = false>
__device__ __forceinline__ void panel_body(
    float* __restrict__ W, int d_row, int d_col, int i1, int width,
    const float* __restrict__ U, int maxq, int gwide, int ngroups,
    uint8_t* __restrict__ codes, float* __restrict__ scales, int32_t* __restrict__ zeros,
    float* __restrict__ E, double* __restrict__ part_e, const float* __restrict__ Eprev,
    float (&er)[CPL], PanelLds<CPL>& L, double& se, float (&ush)[2][CPL == 8 ? 32 : 1]) {
  constexpr int B = 16 * CPL;
  static_assert(GIN == 0 || (GIN % 16 == 0 && B % GIN == 0), "group inside block");
  static_assert(EMODE == kEprevMem || (FULL && CPL == 8), "shares from registers: full blocks of 128");
  float* Us = L.Us;
  float* rd = L.rd;
  const int t = threadIdx.x;
  const size_t ldu = (size_t)d_col;
  // stage U's diagonal block in LDS.  Full blocks of 64 or 128 columns: whole
  // rows by direct-to-LDS buffer loads in two parts, the first kRows0 rows
  // waited for before the column loop, the rest at column kRows0 - kPF (just
  // before the prefetch reaches them); entries left of the diagonal are read
  // too but only ever update columns already quantized.  Otherwise: the upper
  // part through registers, with zeros outside it.
  constexpr bool kDma = FULL && (B == 64 || B == 128);
  constexpr int kPF = 4;
  constexpr int kRowsPerLoad = 256 / B;                 // rows per 64-lane 16-byte load
  constexpr int kLoads = B / kRowsPerLoad;              // loads for the whole block
  constexpr int kRows0 = 32;                            // rows of the first part
  constexpr int kLoads0 = kRows0 / kRowsPerLoad;
  static_assert(!kDma || (kLoads0 % 4 == 0 && kLoads % 4 == 0), "loads per wave");
  // The previous block's share on full blocks of 128 runs on the matrix cores
  // (v_mfma_f32_16x16x4f32: 16 rows of the work-group x 32 columns per wave,
  // K = 128).  Its B operand, U[i1 - B + k][i1 + 32 wave + n], lane l holding
  // rows k = 4 kk + l / 16 and column n = 16 tt + l % 16, is loaded early: by
  // the previous block of the same launch right after its column loop (PRE),
  // else here, ahead of the diagonal block's staging.
  constexpr bool kShareMfma = FULL && CPL == 8;
  const bool share = EMODE == kEprevRegs || Eprev != nullptr;
  auto share_loads = [&](int ib) {
    const int l = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);
    const float* us = U + (size_t)(ib - B + (l >> 4)) * ldu + ib + 32 * wv + (l & 15);
#pragma unroll
    for (int kk = 0; kk < B / 4; ++kk)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) ush[tt][kk] = us[(size_t)(4 * kk) * ldu + 16 * tt];
  };
  static_assert(!PRE || kShareMfma, "operands of the next block's share: full blocks of 128");
  if constexpr (kShareMfma && EMODE == kEprevMem) {
    if (share) share_loads(i1);
  }
  const float udg = (t < width) ? U[(size_t)(i1 + t) * ldu + i1 + t] : 1.f;
  if constexpr (kDma) {
    const int w4 = __builtin_amdgcn_readfirstlane(t >> 6), l = t & 63;
    const float* ubase = U + (size_t)i1 * ldu + i1;
    const uint64_t ba = (uint64_t)(uintptr_t)ubase;
    const float* ubu = (const float*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(ba >> 32)) << 32) |
                                                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ba));
    const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc(
        (void*)ubu, (short)0, (int)((((int64_t)B - 1) * (int64_t)ldu + B) * 4), 0x00020000);
    constexpr int kLanesPerRow = B / 4;
    const uint32_t vo = (uint32_t)(((l / kLanesPerRow) * ldu + (l % kLanesPerRow) * 4) * 4);
#pragma unroll
    for (int i = 0; i < kLoads / 4; ++i) {
      const int q = w4 + 4 * i;  // load q fills rows q * kRowsPerLoad ..
      const int so = __builtin_amdgcn_readfirstlane((int)((uint32_t)(q * kRowsPerLoad) * (uint32_t)ldu * 4u));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ur, (void __attribute__((address_space(3)))*)(Us + q * kRowsPerLoad * B),
                                               16, vo, so, 0, 0);
    }
    if (t < B) rd[t] = (t < width) ? 1.0f / udg : 0.f;
    // this wave's first-part loads are its first kLoads0 / 4; the rest may still be in flight
    if constexpr (kLoads / 4 - kLoads0 / 4 == 12)
      asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
    else if constexpr (kLoads / 4 - kLoads0 / 4 == 2)
      asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    constexpr int kPer = B * B / kThreads;
    constexpr int kBatch = kPer < 32 ? kPer : 32;
#pragma unroll
    for (int u0 = 0; u0 < kPer; u0 += kBatch) {
      float ub[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int idx = t + (u0 + u) * kThreads;
        const int r = idx / B, c = idx % B;
        ub[u] = (r < width && c < width && c >= r) ? U[(size_t)(i1 + r) * ldu + i1 + c] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) Us[t + (u0 + u) * kThreads] = ub[u];
    }
    if (t < B) rd[t] = (t < width) ? 1.0f / udg : 0.f;
    __syncthreads();
  }

  const int lane = t & 63, p = lane & 15;
  const int row = blockIdx.x * 16 + (t >> 6) * 4 + (lane >> 4);
  const bool valid = row < d_row;
  const size_t rowc = (size_t)(valid ? row : d_row - 1);
  float w[CPL], cr[CPL];
#pragma unroll
  for (int r = 0; r < CPL; ++r) {
    const int col = p * CPL + r;
    w[r] = (FULL || col < width) ? W[rowc * d_col + i1 + col] : 0.f;
    cr[r] = 0.f;
  }
  if (share) {
    // E_prev is stored [k][row].
    if constexpr (kShareMfma) {
      // W[rows, block] -= E_prev U[i1 - B:i1, block]: E_prev staged in LDS as
      // [k][16 rows] (the A operand, from the registers of the work-group's own
      // previous block or from memory), U from the registers loaded above; the
      // 16 x 128 product returns to the column layout through the same LDS.
      // Words written by one lane and read by another are ordered by a
      // work-group barrier with LDS-only fences (the diagonal block's
      // direct-to-LDS loads may stay in flight across it).
      float* es = L.dl;  // 16 B floats: [k][16] for E_prev, then [16][B] for the product
      const int rl = (t >> 6) * 4 + (lane >> 4);
      if constexpr (EMODE == kEprevRegs) {
#pragma unroll
        for (int r = 0; r < CPL; ++r) es[(p * CPL + r) * 16 + rl] = er[r];
      } else {
#pragma unroll
        for (int q = 0; q < 16 * B / kThreads; ++q) {
          const int idx = q * kThreads + t;
          const int erow = std::min((int)blockIdx.x * 16 + (idx & 15), d_row - 1);
          es[idx] = Eprev[(size_t)(idx >> 4) * d_row + erow];
        }
      }
      auto lds_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      };
      lds_sync();
      // two independent chains per column tile (the even and odd k steps)
      f32x4 acc[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[h][0] = acc[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < B / 4; ++kk) {
        const float a = es[(4 * kk + (lane >> 4)) * 16 + (lane & 15)];
        acc[kk & 1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, ush[0][kk], acc[kk & 1][0], 0, 0, 0);
        acc[kk & 1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, ush[1][kk], acc[kk & 1][1], 0, 0, 0);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[0][tt] += acc[1][tt];
      lds_sync();  // every E word read
      // lane l holds rows 4 (l / 16) + i, column 32 wave + 16 tt + l % 16
      const int wv = t >> 6;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) es[(4 * (lane >> 4) + i) * B + 32 * wv + 16 * tt + (lane & 15)] = acc[0][tt][i];
      lds_sync();
      const f32x4 s0 = *(const f32x4*)&es[rl * B + p * CPL];
      const f32x4 s1 = *(const f32x4*)&es[rl * B + p * CPL + 4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        w[r] -= s0[r];
        w[4 + r] -= s1[r];
      }
    } else {
      const float* ep = Eprev + rowc;
      const float* up = U + (size_t)(i1 - B) * ldu + i1 + p * CPL;
      for (int k = 0; k < B; ++k) {
        const float e = ep[(size_t)k * d_row];
#pragma unroll
        for (int r = 0; r < CPL; ++r)
          if (FULL || p * CPL + r < width) w[r] = fmaf(-e, up[(size_t)k * ldu + r], w[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < CPL; ++r) er[r] = 0.f;
  float s = 1.f, z = 0.f;
  if (GIN == 0) {
    // per-row grid (one column of scales) or a group wider than the block
    const int gi = gwide ? i1 / gwide : 0;
    s = scales[rowc * ngroups + gi];
    z = (float)zeros[rowc * ngroups + gi];
  }
  float rs = 1.f / s;
  const float fmaxq = (float)maxq;
  // c - z = clamp(round(x / s), -z, maxq - z), exact on integer-valued floats
  float nz = -z, mz = fmaxq - z;
  // 1 / U[j][j] for this lane's own columns (only the owner's error is used)
  float rdl[CPL];
#pragma unroll
  for (int r = 0; r < CPL; ++r) rdl[r] = rd[p * CPL + r];
  // U rows of the block, this lane's CPL columns, prefetched kPF columns ahead
  constexpr int kQ = (CPL + 3) / 4;
  f32x4 ub[kPF][kQ];
  auto uload = [&](int j, f32x4* dst) {
    if constexpr (CPL >= 4) {
#pragma unroll
      for (int q = 0; q < kQ; ++q) dst[q] = *(const f32x4*)&Us[j * B + p * CPL + 4 * q];
    } else {
#pragma unroll
      for (int r = 0; r < CPL; ++r) dst[0][r] = Us[j * B + p * CPL + r];
    }
  };
#pragma unroll
  for (int j = 0; j < kPF; ++j) uload(j, ub[j]);

  // the grid of the group starting at column j, from the current weights
  auto group_start = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    // group [j, j + GIN): lanes j/CPL .. (j+GIN)/CPL - 1 of the row hold it
    constexpr int l0 = j / CPL, l1 = (j + GIN) / CPL;
    float mn = INFINITY, mx = -INFINITY;
    const bool mine = (p >= l0 && p < l1);
#pragma unroll
    for (int r = 0; r < CPL; ++r) {
      const bool in = mine && (FULL || p * CPL + r < width);
      mn = in ? fminf(mn, w[r]) : mn;
      mx = in ? fmaxf(mx, w[r]) : mx;
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      mn = fminf(mn, __shfl_xor(mn, o, 16));
      mx = fmaxf(mx, __shfl_xor(mx, o, 16));
    }
    grid_from_minmax(mn, mx, maxq, s, z);
    rs = 1.f / s;
    nz = -z;
    mz = fmaxq - z;
    if (p == 0 && valid) {
      const int gi = (i1 + j) / GIN;
      scales[rowc * ngroups + gi] = s;
      zeros[rowc * ngroups + gi] = (int32_t)z;
    }
  };
  // code and scaled error of the column in register jj (every lane computes
  // it on its own register; the owner lane's values are the column's)
  auto quant = [&](auto jc, float& e, float& c) {
    constexpr int jj = decltype(jc)::value;
    const float x = w[jj];
    const float cz = __builtin_amdgcn_fmed3f(rintf(x * rs), nz, mz);
    e = fmaf(-s, cz, x) * rdl[jj];
    c = cz + z;
  };

  // Column j's e and c are ready when step j starts: step j broadcasts e,
  // updates column j + 1 first and computes its e and c at once, so that chain
  // runs under the rest of step j's updates.  At a group start the next
  // column's chain waits for the group's grid, which needs every update.
  float ecur = 0.f, ccur = 0.f;
  if constexpr (GIN != 0) group_start(std::integral_constant<int, 0>{});
  quant(std::integral_constant<int, 0>{}, ecur, ccur);
  static_for<0, 16>([&](auto kc) {
    constexpr int kk = decltype(kc)::value;
    static_for<0, CPL>([&](auto jc) {
      constexpr int jj = decltype(jc)::value;
      constexpr int j = kk * CPL + jj;
      if (FULL || j < width) {
        if constexpr (kDma && kRows0 < B && j == kRows0 - kPF)
          asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        const float eb = row_bcast<kk>(ecur);
        const f32x4* u = ub[j % kPF];
        constexpr int jn = (jj + 1) % CPL;
        constexpr bool kNext = j + 1 < B;
        constexpr bool kNextGroup = kNext && GIN != 0 && (j + 1) % (GIN ? GIN : 1) == 0;
        w[jn] = fmaf(-eb, u[jn / 4][jn % 4], w[jn]);
        float enx = 0.f, cnx = 0.f;
        if constexpr (kNext && !kNextGroup) quant(std::integral_constant<int, jn>{}, enx, cnx);
#pragma unroll
        for (int r = 0; r < CPL; ++r)
          if (r != jn) w[r] = fmaf(-eb, u[r / 4][r % 4], w[r]);
        const bool own = (p == kk);
        cr[jj] = own ? ccur : cr[jj];
        er[jj] = own ? ecur : er[jj];
        // The owner's e and c are selected inside their own step: left free,
        // the compiler keeps every step's e and c live to the end of the block,
        // and the register pressure that causes sinks each U-row prefetch to one
        // step ahead of its use.  (A scheduling barrier per step as well cost 7%:
        // the next step's chain then cannot fill this step's gaps.)
        asm volatile("" : "+v"(cr[jj]), "+v"(er[jj]));
        if constexpr (j + kPF < B) uload(j + kPF, ub[j % kPF]);
        if constexpr (kNextGroup) {
          if (FULL || j + 1 < width) {
            group_start(std::integral_constant<int, j + 1>{});
            quant(std::integral_constant<int, jn>{}, enx, cnx);
          }
        }
        ecur = enx;
        ccur = cnx;
      }
    });
  });

  if constexpr (PRE) share_loads(i1 + B);
#pragma unroll
  for (int r = 0; r < CPL; ++r) {
    const int col = p * CPL + r;
    if (valid && (FULL || col < width)) {
      codes[(size_t)row * d_col + i1 + col] = (uint8_t)cr[r];
      E[(size_t)col * d_row + row] = er[r];   // E stored transposed: [B x d_row]
      se += (double)er[r] * (double)er[r];
    }
  }
  // the next block's diagonal staging (pair launches) overwrites the LDS this
  // block's waves read
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// the work-group's sum of its lanes' squared errors, added to its partial
__device__ __forceinline__ void panel_error_sum(double se, double* __restrict__ part_e, double* red) {
  const int t = threadIdx.x;
  for (int o = 32; o > 0; o >>= 1) se += __shfl_xor(se, o, 64);
  if ((t & 63) == 0) red[t >> 6] = se;
  __syncthreads();
  if (t == 0) part_e[blockIdx.x] += (red[0] + red[1]) + (red[2] + red[3]);
}

template <int CPL, int GIN, bool FULL>
__global__ __launch_bounds__(kThreads) void panel_kernel(
    float* __restrict__ W, int d_row, int d_col, int i1, int width,
    const float* __restrict__ U, int maxq, int gwide, int ngroups,
    uint8_t* __restrict__ codes, float* __restrict__ scales, int32_t* __restrict__ zeros,
    float* __restrict__ E, double* __restrict__ part_e, const float* __restrict__ Eprev) {
  __shared__ __attribute__((aligned(16))) PanelLds<CPL> L;
  float er[CPL];
  double se = 0.0;
  float ush[2][CPL == 8 ? 32 : 1];
  panel_body<CPL, GIN, FULL, kEprevMem>(W, d_row, d_col, i1, width, U, maxq, gwide, ngroups, codes, scales,
                                         zeros, E, part_e, Eprev, er, L, se, ush);
  panel_error_sum(se, part_e, L.red);
}

// Two full blocks of 128 columns, [i1, i1 + 128) and [i1 + 128, i1 + 256), for
// 16 rows per work-group: the second block's share of the first block's
// correction depends only on the work-group's own rows, so the same work-group
// applies it from the errors it has just computed and goes on (one launch per
// pair instead of two; E of the two blocks consecutive, E and E + 128 d_row).
template <int GIN>
__global__ __launch_bounds__(kThreads) void panel_pair_kernel(
    float* __restrict__ W, int d_row, int d_col, int i1, const float* __restrict__ U, int maxq, int gwide,
    int ngroups, uint8_t* __restrict__ codes, float* __restrict__ scales, int32_t* __restrict__ zeros,
    float* __restrict__ E, double* __restrict__ part_e) {
  __shared__ __attribute__((aligned(16))) PanelLds<8> L;
  float er[8];
  double se = 0.0;  // both blocks' squared errors, one sum per lane
  float ush[2][32];  // the odd block's share operands, loaded after the even block's loop
  panel_body<8, GIN, true, kEprevMem, true>(W, d_row, d_col, i1, 128, U, maxq, gwide, ngroups, codes, scales,
                                            zeros, E, part_e, nullptr, er, L, se, ush);
  panel_body<8, GIN, true, kEprevRegs>(W, d_row, d_col, i1 + 128, 128, U, maxq, gwide, ngroups, codes, scales,
                                       zeros, E + (size_t)128 * d_row, part_e, nullptr, er, L, se, ush);
  panel_error_sum(se, part_e, L.red);
}

hipError_t launch_panel_pair(int gin, dim3 grid, hipStream_t s, float* W, int d_row, int d_col, int i1,
                             const float* U, int maxq, int gwide, int ngroups, uint8_t* codes, float* scales,
                             int32_t* zeros, float* E, double* part_e) {
#define GPTQ_PAIR_CASE(G)                                                                                   \
  case G:                                                                                                  \
    hipLaunchKernelGGL(panel_pair_kernel<G>, grid, dim3(kThreads), 0, s, W, d_row, d_col, i1, U, maxq, gwide, \
                       ngroups, codes, scales, zeros, E, part_e);                                          \
    return hipGetLastError();
  switch (gin) {
    GPTQ_PAIR_CASE(0)
    GPTQ_PAIR_CASE(16)
    GPTQ_PAIR_CASE(32)
    GPTQ_PAIR_CASE(64)
    GPTQ_PAIR_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef GPTQ_PAIR_CASE
}

template <int CPL, int GIN>
hipError_t launch_panel_g(bool full, dim3 grid, hipStream_t s, float* W, int d_row, int d_col,
                          int i1, int width, const float* U, int maxq, int gwide, int ngroups,
                          uint8_t* codes, float* scales, int32_t* zeros, float* E, double* part_e,
                          const float* Eprev) {
  if (full)
    hipLaunchKernelGGL((panel_kernel<CPL, GIN, true>), grid, dim3(kThreads), 0, s, W, d_row, d_col,
                       i1, width, U, maxq, gwide, ngroups, codes, scales, zeros, E, part_e, Eprev);
  else
    hipLaunchKernelGGL((panel_kernel<CPL, GIN, false>), grid, dim3(kThreads), 0, s, W, d_row, d_col,
                       i1, width, U, maxq, gwide, ngroups, codes, scales, zeros, E, part_e, Eprev);
  return hipGetLastError();
}

template <int CPL>
hipError_t launch_panel(int gin, bool full, dim3 grid, hipStream_t s, float* W, int d_row,
                        int d_col, int i1, int width, const float* U, int maxq, int gwide,
                        int ngroups, uint8_t* codes, float* scales, int32_t* zeros, float* E,
                        double* part_e, const float* Eprev) {
#define GPTQ_PANEL_CASE(G)                                                                  \
  case G:                                                                                  \
    if constexpr (G <= 16 * CPL)                                                           \
      return launch_panel_g<CPL, G>(full, grid, s, W, d_row, d_col, i1, width, U, maxq,   \
                                    gwide, ngroups, codes, scales, zeros, E, part_e, Eprev);\
    return hipErrorInvalidValue;
  switch (gin) {
    GPTQ_PANEL_CASE(0)
    GPTQ_PANEL_CASE(16)
    GPTQ_PANEL_CASE(32)
    GPTQ_PANEL_CASE(64)
    GPTQ_PANEL_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef GPTQ_PANEL_CASE
}

// sum over rows of (W0 - scale (c - zero))^2, per work-group partials
template <typename T>
__global__ __launch_bounds__(kThreads) void err_delta_kernel(
    const T* __restrict__ W0, int64_t ldw, int64_t d_row, int64_t d_col,
    const uint8_t* __restrict__ cpos, const float* __restrict__ scales,
    const int32_t* __restrict__ zeros, int g, int64_t ngroups, const int32_t* __restrict__ perm,
    uint8_t* __restrict__ codes, double* __restrict__ part_d, int vec8) {
  __shared__ double red[kThreads];
  const int t = threadIdx.x;
  double acc = 0.0;
  // natural order with 8-column runs inside one group and 16-byte (fp16) or
  // 32-byte (fp32) aligned rows: 8 columns per thread and step
  for (int64_t row = blockIdx.x; vec8 && row < d_row; row += gridDim.x) {
    for (int64_t c = 8 * (int64_t)t; c < d_col; c += 8 * kThreads) {
      const int gi = (int)(c / g);
      const float s = scales[row * ngroups + gi];
      const float z = (float)zeros[row * ngroups + gi];
      const uint64_t cv = *(const uint64_t*)(cpos + row * d_col + c);
      float wv[8];
      if constexpr (sizeof(T) == 2) {
        typedef _Float16 h8 __attribute__((ext_vector_type(8)));
        const h8 x = *(const h8*)(W0 + row * ldw + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) wv[e] = (float)x[e];
      } else {
        const f32x4 x0 = *(const f32x4*)(W0 + row * ldw + c);
        const f32x4 x1 = *(const f32x4*)(W0 + row * ldw + c + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wv[e] = x0[e];
          wv[e + 4] = x1[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float wh = s * ((float)((cv >> (8 * e)) & 255u) - z);
        const double dlt = (double)wv[e] - (double)wh;
        acc += dlt * dlt;
      }
    }
  }
  for (int64_t row = blockIdx.x; !vec8 && row < d_row; row += gridDim.x) {
    for (int64_t c = t; c < d_col; c += kThreads) {
      // c: position in the quantization order (groups are runs of positions)
      const int gi = (int)c / g;
      const int64_t oc = perm_col(perm, c, d_col);
      const float s = scales[row * ngroups + gi];
      const float z = (float)zeros[row * ngroups + gi];
      const uint8_t cv = cpos[row * d_col + c];
      if (perm) codes[row * d_col + oc] = cv;  // back to the original column
      const float wh = s * ((float)cv - z);
      const double dlt = (double)(float)W0[row * ldw + oc] - (double)wh;
      acc += dlt * dlt;
    }
  }
  red[t] = acc;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  if (t == 0) part_d[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kThreads) void err_final_kernel(const double* __restrict__ part_e,
                                                             int64_t ne,
                                                             const double* __restrict__ part_d,
                                                             int64_t nd, const float* lambda,
                                                             double* out) {
  __shared__ double re[kThreads], rdd[kThreads];
  const int t = threadIdx.x;
  double a = 0.0, b = 0.0;
  for (int64_t i = t; i < ne; i += kThreads) a += part_e[i];
  for (int64_t i = t; i < nd; i += kThreads) b += part_d[i];
  re[t] = a;
  rdd[t] = b;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (t < o) {
      re[t] += re[t + o];
      rdd[t] += rdd[t + o];
    }
    __syncthreads();
  }
  if (t == 0) *out = 0.5 * re[0] - (lambda ? 0.5 * (double)*lambda * rdd[0] : 0.0);
}

// The same sum in the quantization order of a permutation, with the row of W0
// and the row's codes staged in LDS (dynamic: d_col floats, then d_col bytes):
// W0 is read and the codes are written back to their original columns with
// coalesced accesses, the gather and the scatter go through LDS.  Each element
// is taken by the same thread, in the same order, as in err_delta_kernel.
template <typename T>
__global__ __launch_bounds__(kThreads) void err_delta_perm_kernel(
    const T* __restrict__ W0, int64_t ldw, int64_t d_row, int64_t d_col,
    const uint8_t* __restrict__ cpos, const float* __restrict__ scales,
    const int32_t* __restrict__ zeros, int g, int64_t ngroups, const int32_t* __restrict__ perm,
    uint8_t* __restrict__ codes, double* __restrict__ part_d) {
  extern __shared__ __attribute__((aligned(16))) unsigned char err_lds[];
  float* wrow = (float*)err_lds;
  uint8_t* crow = err_lds + d_col * sizeof(float);
  __shared__ double red[kThreads];
  const int t = threadIdx.x;
  double acc = 0.0;
  for (int64_t row = blockIdx.x; row < d_row; row += gridDim.x) {
    for (int64_t c = t; c < d_col; c += kThreads) wrow[c] = (float)W0[row * ldw + c];
    __syncthreads();
    for (int64_t c = t; c < d_col; c += kThreads) {
      const int gi = (int)c / g;
      const int64_t oc = perm_col(perm, c, d_col);
      const float s = scales[row * ngroups + gi];
      const float z = (float)zeros[row * ngroups + gi];
      const uint8_t cv = cpos[row * d_col + c];
      crow[oc] = cv;
      const float wh = s * ((float)cv - z);
      const double dlt = (double)wrow[oc] - (double)wh;
      acc += dlt * dlt;
    }
    __syncthreads();
    for (int64_t c = t; c < d_col; c += kThreads) codes[row * d_col + c] = crow[c];
    __syncthreads();  // this row's LDS fully read before the next row's
  }
  red[t] = acc;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (t < o) red[t] += red[t + o];
    __syncthreads();
  }
  if (t == 0) part_d[blockIdx.x] = red[0];
}
// widths whose row fits the LDS of err_delta_perm_kernel
constexpr int64_t kErrPermMaxCols = 12288;  // d_col * 5 bytes + 2 KB within 64 KB of LDS

// group of each original column: g_idx[perm[c]] = c / g
__global__ __launch_bounds__(kThreads) void g_idx_kernel(const int32_t* __restrict__ perm, int64_t d_col,
                                                         int64_t g, int32_t* __restrict__ g_idx) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c < d_col) g_idx[perm_col(perm, c, d_col)] = (int32_t)(c / g);
}

constexpr int64_t kErrWGs = 1024;
#ifndef GPTQ_ROW_PANEL_MIN_ROWS
#define GPTQ_ROW_PANEL_MIN_ROWS 32768
#endif
constexpr int64_t kRowPanelMinRows = GPTQ_ROW_PANEL_MIN_ROWS;

}  // namespace

// The workspace of the no-allocation entry point: one array per device, loaded
// with the code object and held until the process ends.  Host code reaches it
// only through the address hipGetSymbolAddress returns for the current device
// (the array's name in host code is a host-side stand-in, not that address).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

QuantPlan quant_plan(int64_t d_row, int64_t d_col, int64_t B) {
  QuantPlan p{};
  p.d_row = d_row;
  p.d_col = d_col;
  p.B = B;
  p.nblk = cdiv(d_col, B);
  p.panel_wgs = cdiv(d_row, 16);
  // the panel has at most one work-group per CU up to 4096 rows: bound by its
  // column chain's latency, it absorbs the even block's share nearly for free;
  // past that the shares inside a group take thin launches
  p.pair = p.panel_wgs <= 256 ? 1 : 2;
  size_t off = 0;
  p.off_w = off;
  off = align_up(off + (size_t)d_row * d_col * sizeof(float), 256);
  p.off_e = off;  // E of the blocks of one group (up to four), consecutive
  off = align_up(off + (size_t)d_row * B * (p.pair == 1 ? 2 : 4) * sizeof(float), 256);
  p.off_part = off;
  off = align_up(off + (size_t)p.panel_wgs * sizeof(double), 256);
  p.off_err = off;
  off = align_up(off + (size_t)kErrWGs * sizeof(double), 256);
  p.off_cpos = off;  // codes in quantization order (used under a permutation)
  off = align_up(off + (size_t)d_row * d_col, 256);
  p.ws_bytes = off;
  return p;
}

hipError_t quant_launch(const QuantPlan& p, const void* W0, int w_dtype, int64_t ldw,
                        const float* U, const float* lambda, const int32_t* perm, int bits,
                        int64_t group, uint8_t* codes, float* scales, int32_t* zeros,
                        int32_t* g_idx, double* out_err, void* ws, hipStream_t s) {
  const int64_t d_row = p.d_row, d_col = p.d_col, B = p.B;
  char* base = (char*)ws;
  float* W = (float*)(base + p.off_w);
  float* E = (float*)(base + p.off_e);
  double* part_e = (double*)(base + p.off_part);
  double* part_d = (double*)(base + p.off_err);
  // codes by position of the quantization order: the caller's array in natural
  // order, a workspace copy under a permutation (scattered back at the end)
  uint8_t* cpos = perm ? (uint8_t*)(base + p.off_cpos) : codes;
  const int maxq = (1 << bits) - 1;
  const int64_t ngroups = group ? cdiv(d_col, group) : 1;
  hipError_t e;
  hipLaunchKernelGGL(zero_f64_kernel, dim3(64), dim3(kThreads), 0, s, part_e, p.panel_wgs);
  const int pvec8 = !perm && d_col % 8 == 0 && ldw % 8 == 0 && ((uintptr_t)W0 & (w_dtype == 1 ? 15 : 31)) == 0 &&
                    ((uintptr_t)W & 31) == 0;
  if (w_dtype == 1)
    hipLaunchKernelGGL(prep_kernel<_Float16>, dim3((unsigned)d_row), dim3(kThreads), 0, s,
                       (const _Float16*)W0, ldw, d_col, perm, W, group == 0, maxq, scales, zeros, pvec8);
  else
    hipLaunchKernelGGL(prep_kernel<float>, dim3((unsigned)d_row), dim3(kThreads), 0, s,
                       (const float*)W0, ldw, d_col, perm, W, group == 0, maxq, scales, zeros, pvec8);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // Grouped blocks: the out-of-block update of the columns after a group of nb
  // consecutive blocks runs once, after the group's last block, as one product of
  // depth nb B: W[:, i2:] -= [E_0; ..; E_nb-1] U[i0:i2, i2:], which reads and
  // writes W there 1/nb as often.  Inside the group each block's columns first
  // take the shares of the group's earlier blocks: for pairs in the odd block's
  // panel (nb = 2, at most 4096 rows) or by a thin launch after the even block;
  // for quads by thin launches after block 0 (E_0 on block 1), block 1
  // ([E_0; E_1] on blocks 2 and 3) and block 2 (E_2 on block 3).  The updates
  // are linear in E, so the result is the same up to rounding order.  A grid of
  // groups wider than B is fitted to fully updated columns, so such groups may
  // start only where the columns after them are up to date; the panel's vector
  // reads of U need 16-byte rows.
  const bool base_ok = p.pair && B % 64 == 0 && d_col % 4 == 0 && ((uintptr_t)U & 15) == 0;
  const bool fused = base_ok && p.pair == 1 && (group == 0 || group <= B || group % (2 * B) == 0);
  const bool quad = base_ok && p.pair == 2 && (group == 0 || group <= 2 * B || group % (4 * B) == 0);
  const bool pair2 = base_ok && p.pair == 2 && !quad && (group <= B || group % (2 * B) == 0);
  const int nb = quad ? 4 : (fused || pair2) ? 2 : 1;
  LaunchTimer* timer = launch_timer();
  // enough rows for one row per lane to fill the chip (and no in-panel share)
  const bool row_panel = B == 128 && d_row >= kRowPanelMinRows && d_col % 4 == 0 &&
                         ((uintptr_t)U & 15) == 0;
  // a fused pair of full blocks of 128 takes one launch (panel_pair_kernel)
  bool pair_launched = false;
  for (int64_t i1 = 0, blk = 0; i1 < d_col; i1 += B, ++blk) {
    const int width = (int)std::min<int64_t>(B, d_col - i1);
    const int r = (int)(blk % nb);  // position in the group
    float* Eb = E + (int64_t)r * B * d_row;
    const float* Ep = (fused && r == 1) ? E : nullptr;
    const bool pair_here = fused && r == 0 && B == 128 && i1 + 2 * B <= d_col && !row_panel;
    const bool skip_panel = fused && r == 1 && pair_launched;
    pair_launched = pair_here;
    if (group > B && i1 % group == 0) {
      const int64_t gw = std::min<int64_t>(group, d_col - i1);
      hipLaunchKernelGGL(group_grid_kernel, dim3((unsigned)cdiv(d_row, 4)), dim3(kThreads), 0, s, W,
                         d_row, d_col, i1, gw, i1 / group, ngroups, maxq, scales, zeros);
    }
    const dim3 pg((unsigned)p.panel_wgs);
    const bool full = (width == B);
    const int gin = (group > 0 && group <= B) ? (int)group : 0;
    const int gwide = (group > B) ? (int)group : 0;
    const int ng = (int)ngroups;
    if (!skip_panel && (e = timer_begin(timer, s)) != hipSuccess) return e;
    if (skip_panel) {
      e = hipSuccess;
    } else if (pair_here) {
      e = launch_panel_pair(gin, pg, s, W, (int)d_row, (int)d_col, (int)i1, U, maxq, gwide, ng, cpos, scales,
                            zeros, E, part_e);
    } else if (row_panel && !Ep && full && (gin == 0 || gin == B)) {
      // one row per lane: 64 to 256 rows per work-group, sized so that the
      // work-groups cover the CUs about once
      const int64_t waves = cdiv(d_row, 64);
      const int nw = (int)std::min<int64_t>(4, std::max<int64_t>(1, cdiv(waves, 256)));
      const dim3 rg((unsigned)cdiv(d_row, 64 * nw)), rb((unsigned)(64 * nw));
      e = (gin == B ? row_panel_launch_group : row_panel_launch_grid)(
          rg, rb, s, W, (int)d_row, (int)d_col, (int)i1, U, maxq, gwide, ng, cpos, scales, zeros, Eb, part_e);
    } else switch (B) {
      case 16: e = launch_panel<1>(gin, full, pg, s, W, (int)d_row, (int)d_col, (int)i1, width, U,
                                   maxq, gwide, ng, cpos, scales, zeros, Eb, part_e, Ep); break;
      case 32: e = launch_panel<2>(gin, full, pg, s, W, (int)d_row, (int)d_col, (int)i1, width, U,
                                   maxq, gwide, ng, cpos, scales, zeros, Eb, part_e, Ep); break;
      case 64: e = launch_panel<4>(gin, full, pg, s, W, (int)d_row, (int)d_col, (int)i1, width, U,
                                   maxq, gwide, ng, cpos, scales, zeros, Eb, part_e, Ep); break;
      default: e = launch_panel<8>(gin, full, pg, s, W, (int)d_row, (int)d_col, (int)i1, width, U,
                                   maxq, gwide, ng, cpos, scales, zeros, Eb, part_e, Ep); break;
    }
    if (e != hipSuccess) return e;
    if (timer && !skip_panel) {
      // algorithmic bytes of the launch's blocks: W block in, E and codes out, U's
      // diagonal block, the grid parameters of the groups that start there
      double bytes = 0.0;
      for (int64_t b1 = i1; b1 < i1 + (pair_here ? 2 * B : width); b1 += B) {
        const int64_t wb = std::min<int64_t>(B, d_col - b1);
        const int64_t gstarts = group ? (int64_t)(cdiv(b1 + wb, group) - cdiv(b1, group)) : 0;
        bytes += 9.0 * (double)d_row * wb + 4.0 * wb * wb + 8.0 * (double)d_row * gstarts;
      }
      if ((e = timer_end(timer, kTimePanel, bytes, s)) != hipSuccess) return e;
    }
    const int64_t i2 = i1 + width;
    if (i2 < d_col) {
      int64_t ncols = 0, krows = 0, urow = 0;
      const float* Et = E;
      if (r == nb - 1) {  // the group's last block: every block of the group on the rest
        ncols = d_col - i2;
        krows = (int64_t)r * B + width;
        urow = i1 - (int64_t)r * B;
      } else if (!fused && r == 1) {  // quads: [E_0; E_1] on blocks 2 and 3
        ncols = std::min<int64_t>(2 * B, d_col - i2);
        krows = B + width;
        urow = i1 - B;
      } else if (!fused) {  // E_r on the next block
        ncols = std::min<int64_t>(B, d_col - i2);
        krows = width;
        urow = i1;
        Et = Eb;
      }
      if (ncols > 0) {
        if ((e = timer_begin(timer, s)) != hipSuccess) return e;
        e = trail_update_launch(W + i2, d_col, (int)d_row, (int)ncols, (int)krows, Et, d_row,
                                U + urow * d_col + i2, d_col, s);
        if (e != hipSuccess) return e;
        if ((e = timer_end(timer, kTimeTrail, 2.0 * (double)d_row * ncols * krows, s)) != hipSuccess) return e;
      }
    }
  }
  const unsigned nerr = (unsigned)std::min<int64_t>(kErrWGs, d_row);
  const int64_t gsz = group ? group : d_col;
  const int vec8 = !perm && gsz % 8 == 0 && d_col % 8 == 0 && ldw % 8 == 0 && ((uintptr_t)cpos & 7) == 0 &&
                   ((uintptr_t)W0 & (w_dtype == 1 ? 15 : 31)) == 0;
  if (perm && d_col <= kErrPermMaxCols) {
    const size_t lds = (size_t)d_col * (sizeof(float) + 1);
    if (w_dtype == 1)
      hipLaunchKernelGGL(err_delta_perm_kernel<_Float16>, dim3(nerr), dim3(kThreads), lds, s,
                         (const _Float16*)W0, ldw, d_row, d_col, cpos, scales, zeros, gsz, ngroups, perm, codes,
                         part_d);
    else
      hipLaunchKernelGGL(err_delta_perm_kernel<float>, dim3(nerr), dim3(kThreads), lds, s, (const float*)W0, ldw,
                         d_row, d_col, cpos, scales, zeros, gsz, ngroups, perm, codes, part_d);
  } else if (w_dtype == 1) {
    hipLaunchKernelGGL(err_delta_kernel<_Float16>, dim3(nerr), dim3(kThreads), 0, s,
                       (const _Float16*)W0, ldw, d_row, d_col, cpos, scales, zeros, gsz, ngroups, perm, codes, part_d, vec8);
  } else {
    hipLaunchKernelGGL(err_delta_kernel<float>, dim3(nerr), dim3(kThreads), 0, s, (const float*)W0, ldw,
                       d_row, d_col, cpos, scales, zeros, gsz, ngroups, perm, codes, part_d, vec8);
  }
  hipLaunchKernelGGL(err_final_kernel, dim3(1), dim3(kThreads), 0, s, part_e, p.panel_wgs, part_d,
                     (int64_t)nerr, lambda, out_err);
  if (g_idx)
    hipLaunchKernelGGL(g_idx_kernel, dim3((unsigned)cdiv(d_col, kThreads)), dim3(kThreads), 0, s, perm, d_col,
                       gsz, g_idx);
  return hipGetLastError();
}

}  // namespace gptq
