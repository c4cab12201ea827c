// Packed low-bit codes and the dequantizing product Y = X What^T: the consumer
// of the solver's codes (itwiki "GPTQ", section "결과": kernels that unpack the
// weights on the fly).
//
// Layout: each row is a little-endian bitstream of `bits`-bit fields in 32-bit
// words; position i of a row occupies bits [bits*i, bits*i + bits) of the
// stream, and rows are padded to whole chunks of 32 codes, so a chunk is
// exactly `bits` words and no chunk shares a word with another.  Position i
// holds column perm[i] when a quantization order is given (act-order), so the
// groups of positions stay contiguous; the product then gathers X in the same
// order.
//
// Product (MI355X): HBM-bound on the packed words.  Each work-group stages the
// m rows of X for a tile of columns in LDS (fp32, gathered through perm); each
// wave owns kRows output rows and each lane whole 32-code chunks: it unpacks
// the chunk's codes once per row, and per batch row adds
// s * (sum c x - z * sum x) for each 16-code half (a half never spans two
// groups, as group sizes are multiples of 16).  Lanes reduce by shuffles.
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t perm_idx(const int32_t* __restrict__ perm, int64_t c, int64_t d_col) {
  return perm ? min<int64_t>(max<int32_t>(perm[c], 0), d_col - 1) : c;
}

// one thread per (row, chunk): read the chunk's 32 codes (by position), write `BITS` words
template <int BITS>
__global__ __launch_bounds__(kThreads) void pack_kernel(const uint8_t* __restrict__ codes, int64_t d_row,
                                                        int64_t d_col, int64_t ld_codes,
                                                        const int32_t* __restrict__ perm,
                                                        uint32_t* __restrict__ packed, int64_t ld_packed,
                                                        int64_t nchunk) {
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= d_row * nchunk) return;
  const int64_t row = id / nchunk, ch = id % nchunk;
  uint32_t w[BITS];
#pragma unroll
  for (int k = 0; k < BITS; ++k) w[k] = 0u;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int64_t pos = ch * 32 + e;
    const uint32_t c = (pos < d_col) ? ((uint32_t)codes[row * ld_codes + perm_idx(perm, pos, d_col)] &
                                        ((1u << BITS) - 1u))
                                     : 0u;
    const int off = BITS * e, k = off >> 5, sh = off & 31;
    w[k] |= c << sh;
    if (sh + BITS > 32) w[k + 1] |= c >> (32 - sh);
  }
#pragma unroll
  for (int k = 0; k < BITS; ++k) packed[row * ld_packed + ch * BITS + k] = w[k];
}

// codes e of a chunk (32 x BITS bits in w[0 .. BITS-1]) as floats
template <int BITS>
__device__ __forceinline__ void unpack32(const uint32_t (&w)[BITS], float (&c)[32]) {
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int off = BITS * e, k = off >> 5, sh = off & 31;
    uint32_t v = w[k] >> sh;
    if (sh + BITS > 32) v |= w[k + 1] << (32 - sh);
    c[e] = (float)(v & ((1u << BITS) - 1u));
  }
}

// output rows per wave: fewer with more batch rows, to keep codes and sums in registers
template <int M>
constexpr int rows_per_wave() { return M == 1 ? 4 : (M == 2 ? 2 : 1); }
constexpr int kTileFloats = 8192; // X staged per tile (32 KB)

template <int BITS, int M, typename T>
__global__ __launch_bounds__(kThreads) void dequant_matmul_kernel(
    const uint32_t* __restrict__ packed, int64_t ld_packed, const float* __restrict__ scales,
    const int32_t* __restrict__ zeros, int64_t ngroups, int64_t G, const int32_t* __restrict__ perm,
    int64_t d_row, int64_t d_col, const T* __restrict__ X, int m, int64_t ld_x, float* __restrict__ Y,
    int64_t ld_y) {
  constexpr int CT = kTileFloats / M;  // columns per tile (a multiple of 32)
  constexpr int kRows = rows_per_wave<M>();
  __shared__ __attribute__((aligned(16))) float xs[M * CT];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t row0 = ((int64_t)blockIdx.x * (kThreads / 64) + w) * kRows;
  float y[M][kRows];
#pragma unroll
  for (int b = 0; b < M; ++b)
#pragma unroll
    for (int r = 0; r < kRows; ++r) y[b][r] = 0.f;
  for (int64_t c0 = 0; c0 < d_col; c0 += CT) {
    const int64_t ncols = min<int64_t>(CT, d_col - c0);
    __syncthreads();
    for (int i = t; i < M * CT; i += kThreads) {
      const int b = i / CT, c = i % CT;
      xs[i] = (b < m && c < ncols) ? (float)X[(int64_t)b * ld_x + perm_idx(perm, c0 + c, d_col)] : 0.f;
    }
    __syncthreads();
    const int nch = (int)((ncols + 31) / 32);
    for (int ch = lane; ch < nch; ch += 64) {
      const int64_t pos0 = c0 + (int64_t)ch * 32;
      // codes of this chunk for the wave's rows
      float cv[kRows][32];
      float sc[kRows][2], zc[kRows][2];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int64_t row = row0 + r;
        uint32_t wd[BITS];
#pragma unroll
        for (int k = 0; k < BITS; ++k)
          wd[k] = (row < d_row) ? packed[row * ld_packed + (pos0 / 32) * BITS + k] : 0u;
        unpack32<BITS>(wd, cv[r]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t g = min<int64_t>((pos0 + 16 * h) / G, ngroups - 1);
          sc[r][h] = (row < d_row) ? scales[row * ngroups + g] : 0.f;
          zc[r][h] = (row < d_row) ? (float)zeros[row * ngroups + g] : 0.f;
        }
      }
#pragma unroll
      for (int b = 0; b < M; ++b) {
        if (b >= m) break;
        float xv[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const f32x4 v = *(const f32x4*)&xs[b * CT + ch * 32 + 4 * q];
          xv[4 * q] = v[0]; xv[4 * q + 1] = v[1]; xv[4 * q + 2] = v[2]; xv[4 * q + 3] = v[3];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float xsum = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) xsum += xv[16 * h + e];
#pragma unroll
          for (int r = 0; r < kRows; ++r) {
            float a = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) a = fmaf(cv[r][16 * h + e], xv[16 * h + e], a);
            y[b][r] = fmaf(sc[r][h], fmaf(-zc[r][h], xsum, a), y[b][r]);
          }
        }
      }
    }
  }
  // wave reduction; lane 0 writes
#pragma unroll
  for (int b = 0; b < M; ++b)
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      float v = y[b][r];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      y[b][r] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int b = 0; b < M; ++b)
#pragma unroll
      for (int r = 0; r < kRows; ++r)
        if (b < m && row0 + r < d_row) Y[(int64_t)b * ld_y + row0 + r] = y[b][r];
  }
}

template <int BITS, typename T>
hipError_t dequant_launch_m(const uint32_t* packed, int64_t ld_packed, const float* scales,
                            const int32_t* zeros, int64_t ngroups, int64_t G, const int32_t* perm,
                            int64_t d_row, int64_t d_col, const T* X, int m, int64_t ld_x, float* Y,
                            int64_t ld_y, hipStream_t s) {
#define GPTQ_DQ(MM)                                                                                     \
  hipLaunchKernelGGL((dequant_matmul_kernel<BITS, MM, T>),                                              \
                     dim3((unsigned)cdiv(d_row, (kThreads / 64) * rows_per_wave<MM>())), dim3(kThreads), \
                     0, s, packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y)
  if (m <= 1) GPTQ_DQ(1);
  else if (m <= 2) GPTQ_DQ(2);
  else if (m <= 4) GPTQ_DQ(4);
  else GPTQ_DQ(8);
#undef GPTQ_DQ
  return hipGetLastError();
}

template <typename T>
hipError_t dequant_launch_t(int bits, const uint32_t* packed, int64_t ld_packed, const float* scales,
                            const int32_t* zeros, int64_t ngroups, int64_t G, const int32_t* perm,
                            int64_t d_row, int64_t d_col, const T* X, int m, int64_t ld_x, float* Y,
                            int64_t ld_y, hipStream_t s) {
  switch (bits) {
    case 2: return dequant_launch_m<2, T>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
    case 3: return dequant_launch_m<3, T>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
    case 4: return dequant_launch_m<4, T>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
    case 8: return dequant_launch_m<8, T>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t packed_words_per_row(int64_t d_col, int bits) { return cdiv(d_col, 32) * bits; }

hipError_t pack_launch(const uint8_t* codes, int64_t d_row, int64_t d_col, int64_t ld_codes, int bits,
                       const int32_t* perm, uint32_t* packed, int64_t ld_packed, hipStream_t s) {
  const int64_t nchunk = cdiv(d_col, 32);
  const dim3 grid((unsigned)cdiv(d_row * nchunk, kThreads)), blk(kThreads);
  switch (bits) {
    case 2: hipLaunchKernelGGL(pack_kernel<2>, grid, blk, 0, s, codes, d_row, d_col, ld_codes, perm, packed, ld_packed, nchunk); break;
    case 3: hipLaunchKernelGGL(pack_kernel<3>, grid, blk, 0, s, codes, d_row, d_col, ld_codes, perm, packed, ld_packed, nchunk); break;
    case 4: hipLaunchKernelGGL(pack_kernel<4>, grid, blk, 0, s, codes, d_row, d_col, ld_codes, perm, packed, ld_packed, nchunk); break;
    case 8: hipLaunchKernelGGL(pack_kernel<8>, grid, blk, 0, s, codes, d_row, d_col, ld_codes, perm, packed, ld_packed, nchunk); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t dequant_matmul_launch(const uint32_t* packed, int64_t ld_packed, int bits, const float* scales,
                                 const int32_t* zeros, int64_t group, const int32_t* perm, int64_t d_row,
                                 int64_t d_col, const void* X, int x_dtype, int m, int64_t ld_x, float* Y,
                                 int64_t ld_y, hipStream_t s) {
  const int64_t G = group ? group : cdiv(d_col, 32) * 32;   // one group: every position maps to 0
  const int64_t ngroups = group ? cdiv(d_col, group) : 1;
  if (x_dtype == 1)
    return dequant_launch_t<_Float16>(bits, packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col,
                                      (const _Float16*)X, m, ld_x, Y, ld_y, s);
  return dequant_launch_t<float>(bits, packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col,
                                 (const float*)X, m, ld_x, Y, ld_y, s);
}

}  // namespace gptq
