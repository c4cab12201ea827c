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
// Product (MI355X): HBM-bound on the packed words.  Four kernels:
//  - gemv1_f16_kernel: one row of fp16 X (the per-token product) whose width fits
//    one LDS tile, groups of whole 32-code chunks; a persistent grid, codes turned
//    into fp16 pairs and multiplied by v_dot2_f32_f16, loads one step ahead.
//  - gemm_mfma_f16_kernel: 2..8 rows of fp16 X (or one wider row), one group per
//    128 columns: the same pairs as the A operand of v_mfma_f32_16x16x32_f16.
//  - dequant_gemv_f16_kernel: the pair arithmetic with v_dot2 for groups of 32 or 64,
//    over column tiles of X staged in LDS.
//  - dequant_matmul_kernel: the general case (fp32 X, or groups of 16 that split a
//    chunk): codes unpacked to fp32, s * (sum c x - z * sum x) per 16-code half.
// Each wave owns whole output rows and each lane whole chunks; lanes reduce by
// shuffles, so every output is written once, with no atomics.
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

// ---------------------------------------------------------------------------
// fp16 X, groups of whole chunks: codes as fp16 pairs and v_dot2_f32_f16.
//
// A pair takes two fields of one 32-bit word, one in each 16-bit half, at bit
// offsets A and B (A, B <= 10 - bits).  OR-ing the masked word with an fp16
// exponent of 25 - A (low half) and 25 - B (high half) gives the halves
// 2^(10-A) + c_lo and 2^(10-B) + c_hi exactly, and one packed f16 subtraction
// leaves c_lo and c_hi, so two codes cost one v_and_or_b32 and one v_pk_add_f16;
// v_dot2_f32_f16 then multiplies them by the matching pair of X values (fp16 x
// fp16 products are exact in fp32) and accumulates in fp32.  Each bit width has
// its own order of the 16 pairs of a chunk (below); X is staged in LDS in that
// order.
// ---------------------------------------------------------------------------
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "s"(mask), "v"(magic));
  return r;
}

template <int BITS, int A, int B>
__device__ __forceinline__ h2 fpair(uint32_t v) {
  static_assert(A + BITS <= 10 && B + BITS <= 10, "field must lie in the fp16 mantissa");
  constexpr uint32_t m = (1u << BITS) - 1u;
  constexpr uint32_t mask = (m << A) | ((m << B) << 16);
  constexpr uint32_t magic = ((25u - A) << 10) | (((25u - B) << 10) << 16);
  const h2 off = {(_Float16)(float)(1 << (10 - A)), (_Float16)(float)(1 << (10 - B))};
  return __builtin_bit_cast(h2, and_or(v, mask, magic)) - off;
}

// chunk positions (lo, hi) of pair p, in the order unpack_pairs<BITS> returns them
template <int BITS>
__device__ __forceinline__ int2 pair_pos(int p) {
  if constexpr (BITS == 4) {          // word k: (8k+j, 8k+4+j), j = 0..3
    const int k = p >> 2, j = p & 3;
    return make_int2(8 * k + j, 8 * k + 4 + j);
  } else if constexpr (BITS == 2) {   // word k: (16k+j, 16k+8+j), j = 0..7
    const int k = p >> 3, j = p & 7;
    return make_int2(16 * k + j, 16 * k + 8 + j);
  } else if constexpr (BITS == 8) {   // word k: (4k+j, 4k+2+j), j = 0..1
    const int k = p >> 1, j = p & 1;
    return make_int2(4 * k + j, 4 * k + 2 + j);
  } else {                            // 3 bits: fields straddle words; see unpack_pairs<3>
    const uint8_t lo[16] = {0, 1, 2, 3, 4, 22, 23, 24, 25, 11, 12, 13, 14, 15, 5, 10};
    const uint8_t hi[16] = {16, 17, 18, 19, 20, 6, 7, 8, 9, 27, 28, 29, 30, 31, 21, 26};
    return make_int2(lo[p], hi[p]);
  }
}

template <int BITS>
__device__ __forceinline__ void unpack_pairs(const uint32_t (&w)[BITS], h2 (&c)[16]) {
  if constexpr (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t s = w[k] >> 8;
      c[4 * k + 0] = fpair<4, 0, 0>(w[k]);
      c[4 * k + 1] = fpair<4, 4, 4>(w[k]);
      c[4 * k + 2] = fpair<4, 0, 0>(s);
      c[4 * k + 3] = fpair<4, 4, 4>(s);
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t s = w[k] >> 10;
      c[8 * k + 0] = fpair<2, 0, 0>(w[k]);
      c[8 * k + 1] = fpair<2, 2, 2>(w[k]);
      c[8 * k + 2] = fpair<2, 4, 4>(w[k]);
      c[8 * k + 3] = fpair<2, 6, 6>(w[k]);
      c[8 * k + 4] = fpair<2, 8, 8>(w[k]);
      c[8 * k + 5] = fpair<2, 0, 0>(s);
      c[8 * k + 6] = fpair<2, 2, 2>(s);
      c[8 * k + 7] = fpair<2, 4, 4>(s);
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      c[2 * k + 0] = fpair<8, 0, 0>(w[k]);
      c[2 * k + 1] = fpair<8, 0, 0>(w[k] >> 8);
    }
  } else {
    // A chunk is 96 bits: code e at stream bits 3e.  Halves of two words whose
    // fields sit at equal offsets are merged with one byte permute; the two
    // codes that straddle word boundaries pair with the two that straddle
    // half-word boundaries.
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2];
    const uint32_t q1 = __builtin_amdgcn_perm(w1, w0, 0x07060100u);  // w0 bits 0-15 | w1 bits 16-31
    const uint32_t q2 = __builtin_amdgcn_perm(w0, w2, 0x07060100u);  // w2 bits 0-15 | w0 bits 16-31
    const uint32_t q3 = __builtin_amdgcn_perm(w2, w1, 0x07060100u);  // w1 bits 0-15 | w2 bits 16-31
    c[0] = fpair<3, 0, 0>(q1);          // codes 0, 16
    c[1] = fpair<3, 3, 3>(q1);          // 1, 17
    c[2] = fpair<3, 6, 6>(q1);          // 2, 18
    c[3] = fpair<3, 0, 0>(q1 >> 9);     // 3, 19
    c[4] = fpair<3, 3, 3>(q1 >> 9);     // 4, 20
    c[5] = fpair<3, 2, 2>(q2);          // 22, 6
    c[6] = fpair<3, 5, 5>(q2);          // 23, 7
    c[7] = fpair<3, 0, 0>(q2 >> 8);     // 24, 8
    c[8] = fpair<3, 3, 3>(q2 >> 8);     // 25, 9
    c[9] = fpair<3, 1, 1>(q3);          // 11, 27
    c[10] = fpair<3, 4, 4>(q3);         // 12, 28
    c[11] = fpair<3, 7, 7>(q3);         // 13, 29
    c[12] = fpair<3, 0, 0>(q3 >> 10);   // 14, 30
    c[13] = fpair<3, 3, 3>(q3 >> 10);   // 15, 31
    // code 5 at stream bits 15-17, code 21 at 63-65
    const uint32_t t = __builtin_amdgcn_alignbit(w2, w1, 31);
    c[14] = fpair<3, 0, 1>(__builtin_amdgcn_alignbit(t, w0, 15));
    // code 10 at stream bits 30-32, code 26 at 78-80
    const uint32_t v = __builtin_amdgcn_alignbit(w1, w0, 30);
    c[15] = fpair<3, 0, 6>(__builtin_amdgcn_perm(w2, v, 0x06050100u));
  }
}

constexpr int kPairTileHalves = 16384;   // X staged per tile as fp16 pairs (32 KB)

// Rows per wave: RG groups of R rows, R rows unpacked per chunk.  LDS: the X
// tile as uint4 = 4 pairs, xp4[(b * 4 + q) * nchT + ch] holding pairs 4q .. 4q+3
// of chunk ch (lane-consecutive 16-byte reads), and the fp32 sum of X over each
// chunk for the zero term.
template <int BITS, int M, int R, int RG>
__global__ __launch_bounds__(kThreads) void dequant_gemv_f16_kernel(
    const uint32_t* __restrict__ packed, int64_t ld_packed, const float* __restrict__ scales,
    const int32_t* __restrict__ zeros, int64_t ngroups, int64_t G, const int32_t* __restrict__ perm,
    int64_t d_row, int64_t d_col, const _Float16* __restrict__ X, int m, int64_t ld_x,
    float* __restrict__ Y, int64_t ld_y) {
  constexpr int CT = kPairTileHalves / M;   // columns per tile
  constexpr int NCT = CT / 32;              // chunks per tile
  __shared__ uint4 xp4[M * 4 * NCT];
  __shared__ float xsum[M * NCT];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index: uniform, so row bases are scalar
  const int64_t rbase = ((int64_t)blockIdx.x * (kThreads / 64) + w) * (RG * R);
  const int cpg = (int)(G >> 5);   // chunks per group
  float y[RG * R][M];
#pragma unroll
  for (int i = 0; i < RG * R; ++i)
#pragma unroll
    for (int b = 0; b < M; ++b) y[i][b] = 0.f;
  uint32_t* xp = reinterpret_cast<uint32_t*>(xp4);
  for (int64_t c0 = 0; c0 < d_col; c0 += CT) {
    const int64_t ncols = min<int64_t>(CT, d_col - c0);
    const int nch = (int)((ncols + 31) / 32);
    __syncthreads();
    for (int i = t; i < M * nch * 16; i += kThreads) {
      const int b = i / (nch * 16), rem = i % (nch * 16), ch = rem >> 4, p = rem & 15;
      const int2 pp = pair_pos<BITS>(p);
      const int64_t plo = c0 + ch * 32 + pp.x, phi = c0 + ch * 32 + pp.y;
      _Float16 xl = (_Float16)0.f, xh = (_Float16)0.f;
      if (b < m) {
        if (plo < d_col) xl = X[(int64_t)b * ld_x + perm_idx(perm, plo, d_col)];
        if (phi < d_col) xh = X[(int64_t)b * ld_x + perm_idx(perm, phi, d_col)];
      }
      const h2 v = {xl, xh};
      xp[((b * 4 + (p >> 2)) * NCT + ch) * 4 + (p & 3)] = __builtin_bit_cast(uint32_t, v);
    }
    __syncthreads();
    for (int i = t; i < M * nch; i += kThreads) {
      const int b = i / nch, ch = i % nch;
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = xp4[(b * 4 + q) * NCT + ch];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const h2 hv = __builtin_bit_cast(h2, u[e]);
          s += (float)hv[0] + (float)hv[1];
        }
      }
      xsum[b * NCT + ch] = s;
    }
    __syncthreads();
    const int cg0 = (int)(c0 >> 5);
    for (int ch = lane; ch < nch; ch += 64) {
      const int cg = cg0 + ch;                              // chunk index in the row
      const int gi = min(cg / cpg, (int)ngroups - 1);
      float xs[M];
#pragma unroll
      for (int b = 0; b < M; ++b) xs[b] = xsum[b * NCT + ch];
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        uint32_t wd[R][BITS];
        float sc[R], zc[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          // rows past the end read the last row; their sums are never written
          const int64_t row = min<int64_t>(rbase + g * R + i, d_row - 1);
          const uint32_t* pr = packed + row * ld_packed + (int64_t)cg * BITS;
#pragma unroll
          for (int k = 0; k < BITS; ++k) wd[i][k] = pr[k];
          sc[i] = scales[row * ngroups + gi];
          zc[i] = (float)zeros[row * ngroups + gi];
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
          h2 cp[16];
          unpack_pairs<BITS>(wd[i], cp);
#pragma unroll
          for (int b = 0; b < M; ++b) {
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint4 v = xp4[(b * 4 + q) * NCT + ch];
              acc = __builtin_amdgcn_fdot2(cp[4 * q + 0], __builtin_bit_cast(h2, v.x), acc, false);
              acc = __builtin_amdgcn_fdot2(cp[4 * q + 1], __builtin_bit_cast(h2, v.y), acc, false);
              acc = __builtin_amdgcn_fdot2(cp[4 * q + 2], __builtin_bit_cast(h2, v.z), acc, false);
              acc = __builtin_amdgcn_fdot2(cp[4 * q + 3], __builtin_bit_cast(h2, v.w), acc, false);
            }
            y[g * R + i][b] = fmaf(sc[i], fmaf(-zc[i], xs[b], acc), y[g * R + i][b]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RG * R; ++i)
#pragma unroll
    for (int b = 0; b < M; ++b) {
      float v = y[i][b];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      y[i][b] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < RG * R; ++i)
#pragma unroll
      for (int b = 0; b < M; ++b)
        if (b < m && rbase + i < d_row) Y[(int64_t)b * ld_y + rbase + i] = y[i][b];
  }
}

// chunk position of half `hi` (0 = low, 1 = high) of pair p, in the order
// unpack_pairs<BITS> returns the pairs (a compile-time constant once unrolled)
template <int BITS>
__device__ __forceinline__ constexpr int pair_code(int p, int hi) {
  if (BITS == 4) return 8 * (p >> 2) + (p & 3) + 4 * hi;
  if (BITS == 2) return 16 * (p >> 3) + (p & 7) + 8 * hi;
  if (BITS == 8) return 4 * (p >> 1) + (p & 1) + 2 * hi;
  const int lo3[16] = {0, 1, 2, 3, 4, 22, 23, 24, 25, 11, 12, 13, 14, 15, 5, 10};
  const int hi3[16] = {16, 17, 18, 19, 20, 6, 7, 8, 9, 27, 28, 29, 30, 31, 21, 26};
  return hi ? hi3[p] : lo3[p];
}

// the weight words are read once: loaded with the non-temporal hint (cache policy bit 1)
constexpr int kStreamOnce = 2;

template <int BITS>
__device__ __forceinline__ void buffer_words(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamOnce);
    w[0] = v[0]; w[1] = v[1];
  } else if constexpr (BITS == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, kStreamOnce);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2];
  } else {
#pragma unroll
    for (int h = 0; h < BITS / 4; ++h) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * h, soff, kStreamOnce);
      w[4 * h] = v[0]; w[4 * h + 1] = v[1]; w[4 * h + 2] = v[2]; w[4 * h + 3] = v[3];
    }
  }
}

// One row of X whose pairs fit one LDS tile (d_col <= kPairTileHalves): a
// persistent grid (as many work-groups as are resident at once) stages X once
// per work-group, then each wave takes groups of R rows in a grid-stride loop.
// A lane takes chunks lane, lane + 64, ...; the staged row is zero beyond d_col
// up to a multiple of 64 chunks (nch64), so lanes past the end read a clamped
// chunk and add nothing.  The words of the next (rows, chunk) step are loaded
// before the current step is computed, and the first step's before X is staged.
// Weights, scales and zeros come through buffer loads from a scalar base (the
// step's first row) with one lane offset and a scalar offset per row, so the
// loads cost no vector address arithmetic.  The group of chunk cg is
// floor((2 cg + 1) * (0.5 / cpg)), exact in fp32 for cg < 2^15 (the distance to
// the next integer, 1 / (2 cpg), exceeds the rounding error).
// Dynamic LDS: nch64 * 4 uint4 of pairs, then nch64 floats of chunk sums.
template <int BITS, int R>
__global__ __launch_bounds__(kThreads) void gemv1_f16_kernel(
    const uint32_t* __restrict__ packed, int64_t ld_packed, const float* __restrict__ scales,
    const int32_t* __restrict__ zeros, int64_t ngroups, float half_inv_cpg, const int32_t* __restrict__ perm,
    int64_t d_row, int64_t d_col, const _Float16* __restrict__ X, float* __restrict__ Y) {
  extern __shared__ uint4 lds_dyn[];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int nch = (int)((d_col + 31) / 32);
  const int nch64 = (nch + 63) & ~63;
  uint4* xp4 = lds_dyn;
  float* xsum = reinterpret_cast<float*>(lds_dyn + 4 * nch64);
  const int J = nch64 >> 6;                                   // chunk steps per row group
  const int64_t ngrp = (d_row + R - 1) / R;
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  int64_t q = (int64_t)blockIdx.x * (kThreads / 64) + w;
  const int ldb = (int)(ld_packed * 4), ngb = (int)(ngroups * 4);   // row strides in bytes

  // raw words only: converting a loaded value here would wait for the load
  struct Step { uint32_t wd[R][BITS]; uint32_t sc[R], zc[R]; };
  auto load = [&](int64_t qq, int jj, Step& st) {
    const int cg = min(lane + 64 * jj, nch - 1);
    const int gi = min((int)((float)(2 * cg + 1) * half_inv_cpg), (int)ngroups - 1);
    const int64_t row0 = qq * R;
    const int last = (int)min<int64_t>(R - 1, d_row - 1 - row0);   // rows past the end read the last row
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc((void*)(packed + row0 * ld_packed), (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(scales + row0 * ngroups), (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc((void*)(zeros + row0 * ngroups), (short)0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int ri = min(i, last);
      buffer_words<BITS>(rp, cg * BITS * 4, ri * ldb, st.wd[i]);
      st.sc[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, gi * 4, ri * ngb, 0);
      st.zc[i] = __builtin_amdgcn_raw_buffer_load_b32(rz, gi * 4, ri * ngb, 0);
    }
  };
  Step cur, nxt;
  int j = 0;
  if (q < ngrp) load(q, j, cur);

  // stage X by whole chunks: 32 values, their 16 pairs, and the chunk's sum
  const bool vec = perm == nullptr && (reinterpret_cast<uintptr_t>(X) & 15) == 0;
  const h2 ones = {(_Float16)1.f, (_Float16)1.f};
  for (int ch = t; ch < nch64; ch += kThreads) {
    const int64_t c0 = (int64_t)ch * 32;
    _Float16 xv[32];
    if (vec && c0 + 32 <= d_col) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint4 u = *reinterpret_cast<const uint4*>(X + c0 + 8 * v);
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const h2 hv = __builtin_bit_cast(h2, uu[e]);
          xv[8 * v + 2 * e] = hv[0];
          xv[8 * v + 2 * e + 1] = hv[1];
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) xv[e] = c0 + e < d_col ? X[perm_idx(perm, c0 + e, d_col)] : (_Float16)0.f;
    }
    uint32_t pr[16];
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const h2 v = {xv[pair_code<BITS>(p, 0)], xv[pair_code<BITS>(p, 1)]};
      pr[p] = __builtin_bit_cast(uint32_t, v);
      s = __builtin_amdgcn_fdot2(v, ones, s, false);
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) xp4[qq * nch64 + ch] = make_uint4(pr[4 * qq], pr[4 * qq + 1], pr[4 * qq + 2], pr[4 * qq + 3]);
    xsum[ch] = s;
  }
  __syncthreads();
  if (q >= ngrp) return;

  float y[R];
#pragma unroll
  for (int i = 0; i < R; ++i) y[i] = 0.f;
  // one (rows, chunk) step on st: the dot products, then at the last chunk the
  // lane reduction and the store
  auto compute = [&](const Step& st, int64_t qq, int jj) {
    const int ch = lane + 64 * jj;
    uint4 xv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) xv[k] = xp4[k * nch64 + ch];
    const float xs = xsum[ch];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      h2 cp[16];
      unpack_pairs<BITS>(st.wd[i], cp);
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc = __builtin_amdgcn_fdot2(cp[4 * k + 0], __builtin_bit_cast(h2, xv[k].x), acc, false);
        acc = __builtin_amdgcn_fdot2(cp[4 * k + 1], __builtin_bit_cast(h2, xv[k].y), acc, false);
        acc = __builtin_amdgcn_fdot2(cp[4 * k + 2], __builtin_bit_cast(h2, xv[k].z), acc, false);
        acc = __builtin_amdgcn_fdot2(cp[4 * k + 3], __builtin_bit_cast(h2, xv[k].w), acc, false);
      }
      const float sc = __builtin_bit_cast(float, st.sc[i]), zc = (float)(int32_t)st.zc[i];
      y[i] = fmaf(sc, fmaf(-zc, xs, acc), y[i]);
    }
    if (jj == J - 1) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float v = y[i];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0 && qq * R + i < d_row) Y[qq * R + i] = v;
        y[i] = 0.f;
      }
    }
  };
  // two step buffers in turn: the loads of one are in flight while the other is
  // computed, with no register copies between them.  The prefetch is issued on
  // every step (the last one re-reads its own step) so that the wait before
  // each compute counts exactly the newer loads.
  while (true) {
    int64_t qn = q;
    int jn = j + 1;
    if (jn == J) { jn = 0; qn += nwaves; }
    bool more = qn < ngrp;
    load(more ? qn : q, more ? jn : j, nxt);
    compute(cur, q, j);
    if (!more) break;
    q = qn;
    j = jn;
    qn = q;
    jn = j + 1;
    if (jn == J) { jn = 0; qn += nwaves; }
    more = qn < ngrp;
    load(more ? qn : q, more ? jn : j, cur);
    compute(nxt, q, j);
    if (!more) break;
    q = qn;
    j = jn;
  }
}

// ---------------------------------------------------------------------------
// 2..16 rows of fp16 X: the product on the matrix cores.
//
// v_mfma_f32_16x16x32_f16 with A = 16 weight rows and B = up to 16 rows of X.
// Lane l = (i = l % 16, kb = l / 16) holds eight k-slots of A's row i and the same
// eight k-slots of B's column i; the k-slots of lane group kb are codes of chunk
// 4s + kb in the pair order of unpack_pairs (A) and the X values of the same
// columns (B, built from X in L2 with one byte permute per pair), so the four
// lane groups cover 128 columns per step and four instructions per row block.
// A fifth set with A = ones gives every column's sum of X over the step, for the
// zero term; one group covers the whole step (group 0 or a multiple of 128), so
// scale and zero are applied once per step to the fp32 accumulators.  A
// work-group takes 32 rows (two 16-row blocks, B built once for both) and its four
// waves split the row's steps; their partial sums meet in LDS and are added in a
// fixed order.  The D layout puts rows 4 kb + r (r = 0..3) of batch row i in lane
// l.  Loads run one step ahead as in gemv1_f16_kernel.  Rows past the end, batch
// rows past m and chunks past the row compute on clamped data and are never
// stored (X is zero past d_col).
// ---------------------------------------------------------------------------
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

template <int BITS, bool GATHER>
__global__ __launch_bounds__(kThreads) void gemm_mfma_f16_kernel(
    const uint32_t* __restrict__ packed, int64_t ld_packed, const float* __restrict__ scales,
    const int32_t* __restrict__ zeros, int64_t ngroups, int64_t G, const int32_t* __restrict__ perm,
    int64_t d_row, int64_t d_col, const _Float16* __restrict__ X, int m, int64_t ld_x,
    float* __restrict__ Y, int64_t ld_y) {
  __shared__ float red[kThreads / 64][8][64];               // partial sums of the four waves
  const int t = threadIdx.x, lane = t & 63, li = lane & 15, kb = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int dc = (int)d_col;                                  // widths and offsets fit 32 bits (checked at launch)
  const int nch = (dc + 31) / 32;
  const int NS = (nch + 3) / 4;                               // 128-column steps per row
  const int NSW = (NS + 3) / 4;                               // steps per wave
  const int s_lo = min(w * NSW, NS), s_hi = min(s_lo + NSW, NS);
  const int64_t nbp = (d_row + 31) / 32;                      // pairs of 16-row blocks
  const int jx = min(li, m - 1);                              // batch row whose X this lane loads
  const int xoff = jx * (int)ld_x;
  const int gstep = G >= d_col ? 0 : (int)(G / 128);          // steps per group (G a multiple of 128)
  const int ldb = (int)(ld_packed * 4), ngb = (int)(ngroups * 4);
  const h2 one2 = {(_Float16)1.f, (_Float16)1.f};
  const h8 ones = {one2[0], one2[1], one2[0], one2[1], one2[0], one2[1], one2[0], one2[1]};
  // X's exact extent: a 16-byte read past its end returns zeros
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, (int)(((int64_t)(m - 1) * ld_x + d_col) * 2), 0x00020000);

  struct Step { uint32_t wd[2][BITS]; uint32_t xr[16]; uint32_t sc[2][4], zc[2][4]; };
  for (int64_t bp = blockIdx.x; bp < nbp; bp += gridDim.x) {
    const int64_t r0 = bp * 32;
    const int last = (int)min<int64_t>(31, d_row - 1 - r0);   // rows past the end read the last row
    const __amdgpu_buffer_rsrc_t rp =
        __builtin_amdgcn_make_buffer_rsrc((void*)(packed + r0 * ld_packed), (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(scales + r0 * ngroups), (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc((void*)(zeros + r0 * ngroups), (short)0, 0x7FFFFFFF, 0x00020000);
    int vw[2], vs[2][4];                                      // this lane's row offsets, in bytes
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      vw[rb] = min(16 * rb + li, last) * ldb;
#pragma unroll
      for (int r = 0; r < 4; ++r) vs[rb][r] = min(16 * rb + 4 * kb + r, last) * ngb;
    }
    auto load = [&](int s, Step& st) {
      const int chunk = 4 * s + kb;
      const int cl = min(chunk, nch - 1);
      const int g = gstep == 0 ? 0 : min(s / gstep, (int)ngroups - 1);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        buffer_words<BITS>(rp, vw[rb] + cl * BITS * 4, 0, st.wd[rb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          st.sc[rb][r] = __builtin_amdgcn_raw_buffer_load_b32(rs, vs[rb][r] + g * 4, 0, 0);
          st.zc[rb][r] = __builtin_amdgcn_raw_buffer_load_b32(rz, vs[rb][r] + g * 4, 0, 0);
        }
      }
      const int c0 = chunk * 32;
      if constexpr (!GATHER) {
        const int vo = (xoff + c0) * 2;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const auto u = __builtin_amdgcn_raw_buffer_load_b128(rx, vo + 16 * v, 0, 0);
          st.xr[4 * v] = u[0]; st.xr[4 * v + 1] = u[1]; st.xr[4 * v + 2] = u[2]; st.xr[4 * v + 3] = u[3];
        }
      } else {
        // element by element, through the quantization order if any; zero past d_col
        const _Float16* xrow = X + xoff;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int p0 = c0 + 2 * e, p1 = p0 + 1;
          const int q0 = perm ? min(max(perm[min(p0, dc - 1)], 0), dc - 1) : min(p0, dc - 1);
          const int q1 = perm ? min(max(perm[min(p1, dc - 1)], 0), dc - 1) : min(p1, dc - 1);
          const _Float16 a = p0 < dc ? xrow[q0] : (_Float16)0.f;
          const _Float16 bb = p1 < dc ? xrow[q1] : (_Float16)0.f;
          const h2 v = {a, bb};
          st.xr[e] = __builtin_bit_cast(uint32_t, v);
        }
      }
    };
    f4v y[2];
    y[0] = (f4v){0.f, 0.f, 0.f, 0.f};
    y[1] = y[0];
    auto compute = [&](const Step& st, int s) {
      uint32_t xr[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) xr[e] = st.xr[e];
      if constexpr (!GATHER) {
        // the row's last chunk: zero the values past d_col (they belong to the next row)
        const int valid = dc - (4 * s + kb) * 32;
        if (valid < 32) {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            xr[e] &= (2 * e + 1 < valid ? 0xFFFFFFFFu : 0u) | (2 * e < valid ? 0x0000FFFFu : 0u);
        }
      }
      // B: the step's X values in pair order
      uint32_t xp[16];
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int lo = pair_code<BITS>(p, 0), hi = pair_code<BITS>(p, 1);
        const uint32_t sel = (uint32_t)(2 * (lo & 1)) | ((uint32_t)(2 * (lo & 1) + 1) << 8) |
                             ((uint32_t)(4 + 2 * (hi & 1)) << 16) | ((uint32_t)(4 + 2 * (hi & 1) + 1) << 24);
        xp[p] = __builtin_amdgcn_perm(xr[hi >> 1], xr[lo >> 1], sel);
      }
      h8 bq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const h2 a0 = __builtin_bit_cast(h2, xp[4 * q]), a1 = __builtin_bit_cast(h2, xp[4 * q + 1]);
        const h2 a2 = __builtin_bit_cast(h2, xp[4 * q + 2]), a3 = __builtin_bit_cast(h2, xp[4 * q + 3]);
        bq[q] = (h8){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      }
      f4v dx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) dx = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, bq[q], dx, 0, 0, 0);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        h2 cp[16];
        unpack_pairs<BITS>(st.wd[rb], cp);
        f4v d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const h8 aq = {cp[4 * q][0], cp[4 * q][1], cp[4 * q + 1][0], cp[4 * q + 1][1],
                         cp[4 * q + 2][0], cp[4 * q + 2][1], cp[4 * q + 3][0], cp[4 * q + 3][1]};
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq, bq[q], d, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sc = __builtin_bit_cast(float, st.sc[rb][r]), zc = (float)(int32_t)st.zc[rb][r];
          y[rb][r] = fmaf(sc, fmaf(-zc, dx[r], d[r]), y[rb][r]);
        }
      }
    };
    // this wave's steps, two step buffers in turn (the prefetch is issued on every
    // step, the last one re-reading its own step, so each wait counts exactly)
    if (s_lo < s_hi) {
      Step cur, nxt;
      int s = s_lo;
      load(s, cur);
      while (true) {
        bool more = s + 1 < s_hi;
        load(more ? s + 1 : s, nxt);
        compute(cur, s);
        if (!more) break;
        ++s;
        more = s + 1 < s_hi;
        load(more ? s + 1 : s, cur);
        compute(nxt, s);
        if (!more) break;
        ++s;
      }
    }
    // the four waves' partial sums, added in a fixed order
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[w][4 * rb + r][lane] = y[rb][r];
    __syncthreads();
    if (w == 0 && li < m) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = ((red[0][4 * rb + r][lane] + red[1][4 * rb + r][lane]) + red[2][4 * rb + r][lane]) +
                          red[3][4 * rb + r][lane];
          const int64_t row = r0 + 16 * rb + 4 * kb + r;
          if (row < d_row) Y[(int64_t)li * ld_y + row] = v;
        }
    }
    __syncthreads();
  }
}

template <int BITS>
hipError_t gemm_mfma_f16_launch(const uint32_t* packed, int64_t ld_packed, const float* scales,
                                const int32_t* zeros, int64_t ngroups, int64_t G, const int32_t* perm,
                                int64_t d_row, int64_t d_col, const _Float16* X, int m, int64_t ld_x, float* Y,
                                int64_t ld_y, hipStream_t s) {
  const bool gather = perm != nullptr || (reinterpret_cast<uintptr_t>(X) & 15) != 0 || (ld_x & 7) != 0;
  const auto kern = gather ? gemm_mfma_f16_kernel<BITS, true> : gemm_mfma_f16_kernel<BITS, false>;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, 0);
  if (e != hipSuccess) return e;
  const int64_t wgs = std::max<int64_t>(1, std::min<int64_t>((int64_t)std::max(per_cu, 1) * cus, cdiv(d_row, 32)));
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kThreads), 0, s, packed, ld_packed, scales, zeros, ngroups,
                     G, perm, d_row, d_col, X, m, ld_x, Y, ld_y);
  return hipGetLastError();
}

// rows unpacked together per chunk and the widest row-group count per wave
template <int M>
constexpr int gemv_rows() { return M <= 4 ? 4 : 2; }
template <int M>
constexpr int gemv_groups_max() { return M == 1 ? 4 : (M == 2 ? 2 : 1); }

template <int BITS, int M, int RG>
void gemv_f16_launch_rg(const uint32_t* packed, int64_t ld_packed, const float* scales, const int32_t* zeros,
                        int64_t ngroups, int64_t G, const int32_t* perm, int64_t d_row, int64_t d_col,
                        const _Float16* X, int m, int64_t ld_x, float* Y, int64_t ld_y, hipStream_t s) {
  constexpr int R = gemv_rows<M>();
  hipLaunchKernelGGL((dequant_gemv_f16_kernel<BITS, M, R, RG>),
                     dim3((unsigned)cdiv(d_row, (kThreads / 64) * R * RG)), dim3(kThreads), 0, s, packed,
                     ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y);
}

// the most rows per wave (up to RGM groups of R) that still gives at least 1024 work-groups
template <int BITS, int M>
void gemv_f16_launch_m(const uint32_t* packed, int64_t ld_packed, const float* scales, const int32_t* zeros,
                       int64_t ngroups, int64_t G, const int32_t* perm, int64_t d_row, int64_t d_col,
                       const _Float16* X, int m, int64_t ld_x, float* Y, int64_t ld_y, hipStream_t s) {
  constexpr int R = gemv_rows<M>(), RGM = gemv_groups_max<M>();
  int rg = RGM;
  while (rg > 1 && cdiv(d_row, (kThreads / 64) * R * rg) < 1024) rg >>= 1;
  if constexpr (RGM >= 4) {
    if (rg == 4) {
      gemv_f16_launch_rg<BITS, M, 4>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
      return;
    }
  }
  if constexpr (RGM >= 2) {
    if (rg == 2) {
      gemv_f16_launch_rg<BITS, M, 2>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
      return;
    }
  }
  gemv_f16_launch_rg<BITS, M, 1>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
}

constexpr int kGemv1Rows = 4;

// the persistent one-row kernel: as many work-groups as are resident at once
// (occupancy from its registers and this launch's LDS), at most one per group
// of rows per wave
template <int BITS>
hipError_t gemv1_f16_launch(const uint32_t* packed, int64_t ld_packed, const float* scales, const int32_t* zeros,
                            int64_t ngroups, int64_t G, const int32_t* perm, int64_t d_row, int64_t d_col,
                            const _Float16* X, float* Y, hipStream_t s) {
  const auto kern = gemv1_f16_kernel<BITS, kGemv1Rows>;
  const int64_t nch64 = cdiv(cdiv(d_col, 32), 64) * 64;
  const size_t lds = (size_t)nch64 * (4 * sizeof(uint4) + sizeof(float));
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, lds);
  if (e != hipSuccess) return e;
  const int64_t groups = cdiv(d_row, kGemv1Rows);
  const int64_t wgs = std::max<int64_t>(1, std::min<int64_t>((int64_t)std::max(per_cu, 1) * cus,
                                                              cdiv(groups, kThreads / 64)));
  const float half_inv_cpg = 0.5f / (float)(G >> 5);
  hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kThreads), lds, s, packed, ld_packed, scales, zeros,
                     ngroups, half_inv_cpg, perm, d_row, d_col, X, Y);
  return hipGetLastError();
}

template <int BITS>
hipError_t gemv_f16_launch(const uint32_t* packed, int64_t ld_packed, const float* scales, const int32_t* zeros,
                           int64_t ngroups, int64_t G, const int32_t* perm, int64_t d_row, int64_t d_col,
                           const _Float16* X, int m, int64_t ld_x, float* Y, int64_t ld_y, hipStream_t s) {
  if (m == 1 && d_col <= kPairTileHalves)
    return gemv1_f16_launch<BITS>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, Y, s);
  // the matrix-core kernel: one group per 128-column step, and 32-bit buffer offsets
  const bool one_group_per_step = G % 128 == 0 || G >= d_col;
  const bool offsets_fit = ((int64_t)(m - 1) * ld_x + d_col) * 2 < (int64_t(1) << 31) &&
                           (32 * ld_packed + BITS) * 4 < (int64_t(1) << 31) && 32 * ngroups * 4 < (int64_t(1) << 31);
  if (one_group_per_step && offsets_fit)
    return gemm_mfma_f16_launch<BITS>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x,
                                      Y, ld_y, s);
  if (m <= 1) gemv_f16_launch_m<BITS, 1>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
  else if (m <= 2) gemv_f16_launch_m<BITS, 2>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
  else if (m <= 4) gemv_f16_launch_m<BITS, 4>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
  else gemv_f16_launch_m<BITS, 8>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, X, m, ld_x, Y, ld_y, s);
  return hipGetLastError();
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

namespace {
// What = scale * (code - zero), one thread per weight; the group of column j is
// g_idx[j] (clamped) when given, else j / group (0 for one group per row)
template <typename T>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint8_t* __restrict__ codes, int64_t d_row,
                                                              int64_t d_col, int64_t ld_codes,
                                                              const float* __restrict__ scales,
                                                              const int32_t* __restrict__ zeros, int64_t group,
                                                              int64_t ngroups, const int32_t* __restrict__ g_idx,
                                                              T* __restrict__ out, int64_t ld_out) {
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= d_row * d_col) return;
  const int64_t r = id / d_col, j = id % d_col;
  const int64_t g = g_idx ? min<int64_t>(max<int32_t>(g_idx[j], 0), ngroups - 1) : (group ? j / group : 0);
  const float s = scales[r * ngroups + g];
  const float z = (float)zeros[r * ngroups + g];
  out[r * ld_out + j] = (T)(s * ((float)codes[r * ld_codes + j] - z));
}
}  // namespace

hipError_t dequantize_launch(const uint8_t* codes, int64_t d_row, int64_t d_col, int64_t ld_codes,
                             const float* scales, const int32_t* zeros, int64_t group, const int32_t* g_idx,
                             void* out, int out_dtype, int64_t ld_out, hipStream_t s) {
  const int64_t ngroups = group ? cdiv(d_col, group) : 1;
  const dim3 grid((unsigned)cdiv(d_row * d_col, kThreads)), blk(kThreads);
  if (out_dtype == 1)
    hipLaunchKernelGGL(dequantize_kernel<_Float16>, grid, blk, 0, s, codes, d_row, d_col, ld_codes, scales, zeros,
                       group, ngroups, g_idx, (_Float16*)out, ld_out);
  else
    hipLaunchKernelGGL(dequantize_kernel<float>, grid, blk, 0, s, codes, d_row, d_col, ld_codes, scales, zeros,
                       group, ngroups, g_idx, (float*)out, ld_out);
  return hipGetLastError();
}

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
  if (x_dtype == 1 && G % 32 == 0) {   // every chunk inside one group: the fp16-pair kernel
    const _Float16* Xh = (const _Float16*)X;
    switch (bits) {
      case 2: return gemv_f16_launch<2>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, Xh, m, ld_x, Y, ld_y, s);
      case 3: return gemv_f16_launch<3>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, Xh, m, ld_x, Y, ld_y, s);
      case 4: return gemv_f16_launch<4>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, Xh, m, ld_x, Y, ld_y, s);
      case 8: return gemv_f16_launch<8>(packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col, Xh, m, ld_x, Y, ld_y, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (x_dtype == 1)
    return dequant_launch_t<_Float16>(bits, packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col,
                                      (const _Float16*)X, m, ld_x, Y, ld_y, s);
  return dequant_launch_t<float>(bits, packed, ld_packed, scales, zeros, ngroups, G, perm, d_row, d_col,
                                 (const float*)X, m, ld_x, Y, ld_y, s);
}

}  // namespace gptq
