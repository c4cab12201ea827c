// The one-row-per-lane panel of the lazy-batch loop (itwiki "GPTQ", Algorithm 1,
// the in-block column loop), as a template shared by the two sources that
// instantiate it (one grid per row / per wider group, and one group per block),
// so that the two large unrolled kernels compile in parallel.
#pragma once

#include "gptq_internal.h"

namespace gptq {
namespace rowpanel {

constexpr int kThreads = 256;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ void grid_from_minmax(float mn, float mx, int maxq, float& s, float& z) {
  s = fmaxf(mx - mn, 1e-8f) / (float)maxq;
  z = rintf(-mn / s);
}

// One full block of 128 columns with one weight row per lane, for layers with
// enough rows to fill the chip this way (each wave holds 64 rows).  The row's
// block columns live in the lane's registers; U's diagonal block is staged in
// LDS (with 1 / U[j][j] in place of its diagonal) and read at one address by
// the whole wave (a broadcast), 16 bytes at a time, so the column chain needs
// no cross-lane traffic and the in-block update does exactly the triangular
// work: at column j the lane updates only its columns after j.  Same
// arithmetic, in the same order per element, as panel_kernel.  The LDS data
// path bounds it: every U value reaches all 64 lanes of every wave.
//
// Scheduling: the quads of U (row j, columns 4q .. 4q + 3, q >= j / 4) are one
// stream over all steps, read kRing items ahead through a register ring, and a
// scheduling barrier closes every quad's updates, so reads are neither hoisted
// into registers wholesale nor left on a step's critical path (the next step's
// diagonal quad, which carries 1 / U[j][j], arrives during the current step).
// E is written column by column with buffer stores (64 consecutive rows per
// store; lanes past the last row get an out-of-range offset and their stores
// are dropped), the codes packed four to a register and written per row at the
// end.  Grids: one per row (or a group wider than the block, from
// group_grid_kernel), or one group spanning the whole block (GB).
constexpr int kB = 128;
constexpr int kRing = 8;

// stream items before step j (step i contributes kB / 4 - i / 4 quads)
constexpr int stream_start(int j) {
  int g = 0;
  for (int i = 0; i < j; ++i) g += kB / 4 - i / 4;
  return g;
}

// LDS float offset (row j * kB + 4 q) of every stream item
struct QuadStream {
  static constexpr int L = stream_start(kB);
  int off[L + kRing];
  constexpr QuadStream() : off() {
    int g = 0;
    for (int j = 0; j < kB; ++j)
      for (int q = j / 4; q < kB / 4; ++q) off[g++] = j * kB + 4 * q;
    for (; g < L + kRing; ++g) off[g] = 0;
  }
};
__device__ constexpr QuadStream kQuadStream{};

template <bool GB>
__global__ __launch_bounds__(kThreads) void panel_row_kernel(
    float* __restrict__ W, int d_row, int d_col, int i1,
    const float* __restrict__ U, int maxq, int gwide, int ngroups,
    uint8_t* __restrict__ codes, float* __restrict__ scales, int32_t* __restrict__ zeros,
    float* __restrict__ E, double* __restrict__ part_e) {
  __shared__ __attribute__((aligned(16))) float Us[kB * kB];
  __shared__ double red[kThreads / 64];
  const int t = threadIdx.x, nt = blockDim.x;
  const size_t ldu = (size_t)d_col;
  // stage U's diagonal block (16-byte rows: the caller checks d_col % 4 and
  // U's alignment), its diagonal replaced by the reciprocal
  for (int idx = 4 * t; idx < kB * kB; idx += 4 * nt) {
    const int r = idx / kB, c = idx % kB;
    f32x4 v = *(const f32x4*)(U + (size_t)(i1 + r) * ldu + i1 + c);
    if (r >= c && r < c + 4) v[r - c] = 1.0f / v[r - c];
    *(f32x4*)&Us[idx] = v;
  }
  __syncthreads();

  const int row = blockIdx.x * nt + t;
  const bool valid = row < d_row;
  const size_t rowc = (size_t)(valid ? row : d_row - 1);
  float w[kB];
  const float* wr = W + rowc * d_col + i1;
#pragma unroll
  for (int q = 0; q < kB / 4; ++q) {
    const f32x4 v = *(const f32x4*)(wr + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[4 * q + e] = v[e];
  }
  float s, z;
  if (GB) {
    float mn = w[0], mx = w[0];
#pragma unroll
    for (int c = 1; c < kB; ++c) {
      mn = fminf(mn, w[c]);
      mx = fmaxf(mx, w[c]);
    }
    grid_from_minmax(mn, mx, maxq, s, z);
    if (valid) {
      scales[rowc * ngroups + i1 / kB] = s;
      zeros[rowc * ngroups + i1 / kB] = (int32_t)z;
    }
  } else {
    const int gi = gwide ? i1 / gwide : 0;
    s = scales[rowc * ngroups + gi];
    z = (float)zeros[rowc * ngroups + gi];
  }
  const float rs = 1.f / s;
  const float nz = -z, mz = (float)maxq - z;
  // E through a buffer resource: [kB x d_row] floats; invalid lanes write out of range
  const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc(
      (void*)E, (short)0, (int)((int64_t)kB * d_row * 4), 0x00020000);
  const uint32_t eoff = valid ? (uint32_t)row * 4u : 0x80000000u;
  uint32_t cpk[kB / 4];
  double se = 0.0;
  float sef = 0.f;
  f32x4 ring[kRing];
#pragma unroll
  for (int k = 0; k < kRing; ++k) ring[k] = *(const f32x4*)&Us[kQuadStream.off[k]];
  static_for<0, kB>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int g0 = stream_start(j);
    constexpr int off = g0 % kRing;
    constexpr int q0 = j / 4, nq = kB / 4 - j / 4;
    // the diagonal quad of row j (item 0) carries 1 / U[j][j] at position j % 4
    const float rdj = ring[off][j % 4];
    const float x = w[j];
    const float cz = __builtin_amdgcn_fmed3f(rintf(x * rs), nz, mz);
    const float e = fmaf(-s, cz, x) * rdj;
    cpk[j / 4] = __builtin_amdgcn_cvt_pk_u8_f32(cz + z, j % 4, (j % 4) ? cpk[j / 4] : 0u);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, e), er, eoff,
                                          (int)((uint32_t)j * (uint32_t)d_row * 4u), 0);
    sef = fmaf(e, e, sef);
    if constexpr (j % 16 == 15) {
      se += (double)sef;
      sef = 0.f;
    }
    // the negated error as an operand of its own keeps the updates in the
    // 4-byte accumulate form
    float ne = -e;
    asm volatile("" : "+v"(ne));
#pragma unroll
    for (int k = 0; k < nq; ++k) {
      const int q = q0 + k;
      const f32x4 u = ring[(off + k) % kRing];
      if (g0 + k + kRing < QuadStream::L)
        ring[(off + k) % kRing] = *(const f32x4*)&Us[kQuadStream.off[g0 + k + kRing]];
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        if (4 * q + e4 > j) w[4 * q + e4] = fmaf(ne, u[e4], w[4 * q + e4]);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        if (4 * q + e4 > j) asm volatile("" : "+v"(w[4 * q + e4]));
      __builtin_amdgcn_sched_barrier(0);
    }
  });
  if (valid) {
    uint8_t* crow = codes + rowc * d_col + i1;
    if (d_col % 16 == 0) {
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int q = 0; q < kB / 16; ++q)
        *(u32x4*)(crow + 16 * q) = u32x4{cpk[4 * q], cpk[4 * q + 1], cpk[4 * q + 2], cpk[4 * q + 3]};
    } else {
#pragma unroll
      for (int c = 0; c < kB; ++c) crow[c] = (uint8_t)(cpk[c / 4] >> (8 * (c % 4)));
    }
  } else {
    se = 0.0;
  }
  se += valid ? (double)sef : 0.0;
  for (int o = 32; o > 0; o >>= 1) se += __shfl_xor(se, o, 64);
  if ((t & 63) == 0) red[t >> 6] = se;
  __syncthreads();
  if (t == 0) {
    double a = 0.0;
    for (int i = 0; i < nt / 64; ++i) a += red[i];
    part_e[blockIdx.x] += a;
  }
}

template <bool GB>
hipError_t launch(dim3 grid, dim3 block, hipStream_t s, float* W, int d_row, int d_col, int i1, const float* U,
                  int maxq, int gwide, int ngroups, uint8_t* codes, float* scales, int32_t* zeros, float* E,
                  double* part_e) {
  hipLaunchKernelGGL((panel_row_kernel<GB>), grid, block, 0, s, W, d_row, d_col, i1, U, maxq, gwide,
                     ngroups, codes, scales, zeros, E, part_e);
  return hipGetLastError();
}

}  // namespace rowpanel
}  // namespace gptq
