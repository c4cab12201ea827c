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
// fp16 X: v_mfma_f32_32x32x16_f16, 256x256 tiles, X streamed into LDS by
// direct-to-LDS buffer loads and read back transposed (details below).
// fp32 X: v_mfma_f32_32x32x2f32 reads one row value per lane, so the natural
// [row][feature] LDS layout needs no transpose; 128x128 tiles.
#include "gptq_internal.h"

#include <numeric>
#include <vector>

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
// passes over them.  Work-groups are dispatched round-robin over the 8 XCDs,
// so with the tile count a multiple of 8, XCD x takes tiles
// ord[x * ntiles / 8 .. (x + 1) * ntiles / 8) of every split: the plan groups
// tiles that share column blocks there, so each XCD's L2 serves few blocks.
__device__ __forceinline__ void wg_map(int64_t ntiles, const TileOrder& ord,
                                       int64_t& tile, int64_t& split) {
  const int64_t bid = blockIdx.x;
  if ((ntiles & 7) == 0) {
    const int64_t per = ntiles >> 3;
    const int64_t j = bid >> 3;
    split = j / per;
    const int64_t k = (bid & 7) * per + j % per;
    tile = ord.n ? (int64_t)ord.id[k] : k;
  } else {
    split = bid / ntiles;
    tile = bid % ntiles;
  }
}

// ------------------------------------------------------------------ fp16
// 256x256 tile per work-group (four waves, 128x128 each, v_mfma_f32_32x32x16_f16),
// 32 calibration rows per stage, four LDS stage buffers.
//
// X stays row-major in LDS: stage buffer = [A rows 0..31][256 features] then
// the same for B, 512 bytes per row, with the 16-byte chunk c of row k stored
// at chunk c ^ (4 (k & 3)).  Global memory reaches LDS by buffer loads that
// write LDS directly (16 bytes per lane; one instruction fills two rows), so
// no registers, transposes or LDS stores sit between memory and LDS.  The MFMA
// wants 8 consecutive rows of one feature per lane; ds_read_b64_tr_b16 gives a
// lane 4 consecutive rows of one feature out of a 4-row x 16-feature block
// spread over 16 lanes, so two of them make one operand.  The swizzle spreads
// each half-wave's 4 rows x 4 chunks over all 16 bank groups, and the loads
// write whole rows, so neither side has bank conflicts.
//
// Pipeline (stage s in buffer s % 4, prefetch 3.5 stages deep):
//   MFMAs of k-step 0 of stage s | reads of k-step 1 fragments of stage s (all
//                                   issued under the first half of the MFMAs)
//   wait: own reads done, own loads of stage s+1 landed; barrier
//   loads of stage s+4 into buffer s % 4 (free: every wave is past its reads)
//   MFMAs of k-step 1 of stage s | reads of k-step 0 fragments of stage s+1
// The four buffers are separate LDS objects and the loop is unrolled by four,
// so the compiler can tell the buffer being read from the ones being filled
// and adds no waits of its own.  Waits and barriers are written out with a
// memory clobber so that no LDS access moves across them.
constexpr int kBT16 = 256, kKS16 = 32;
constexpr int kOpHalfs = kKS16 * kBT16;  // one operand of one stage (16 KB)
constexpr int kStageHalfs = 2 * kOpHalfs;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
#define GPTQ_LDS __attribute__((address_space(3)))

// byte offset of (row k, feature m) in one operand block; m a multiple of 4
__device__ __forceinline__ uint32_t swz16(int k, int m) {
  return (uint32_t)(k * 512 + ((((m >> 3) ^ ((k & 3) << 2))) << 4) + ((m & 7) << 1));
}

#define GPTQ_SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
constexpr int kSgMFMA = 0x008, kSgVMEMR = 0x020, kSgDSR = 0x100;

template <bool VEC>
__global__ __launch_bounds__(kThreads) void syrk_f16_kernel(
    const _Float16* __restrict__ X, int64_t ldx, int64_t n, int d, int64_t ntiles,
    int64_t nsplit, int64_t rps, float* __restrict__ part, const TileOrder ord) {
  __shared__ __attribute__((aligned(16))) _Float16 L0[kStageHalfs];
  __shared__ __attribute__((aligned(16))) _Float16 L1[kStageHalfs];
  __shared__ __attribute__((aligned(16))) _Float16 L2[kStageHalfs];
  __shared__ __attribute__((aligned(16))) _Float16 L3[kStageHalfs];
  int64_t tile, split;
  wg_map(ntiles, ord, tile, split);
  int ti, tj;
  tile_of(tile, ti, tj);
  const int I0 = ti * kBT16, J0 = tj * kBT16;
  const int64_t r0 = split * rps;
  const int64_t r1 = min(n, r0 + rps);
  const int nrows = (int)(r1 - r0);
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w & 1, wn = w >> 1;
  const bool full_cols = VEC && (I0 + kBT16 <= d) && (J0 + kBT16 <= d);
  const _Float16* __restrict__ Xs = X + r0 * ldx;  // this split's first row

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // fragment addresses: lane l reads rows 8 (l / 32) + (l % 16) / 4 (+ 4, + 16 per
  // k-step) of feature block wm * 128 + f * 32 + 16 ((l / 16) % 2) + 4 (l % 4)
  const int kl = 8 * (lane >> 5) + ((lane & 15) >> 2);
  uint32_t fadA[4], fadB[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int mo = f * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    fadA[f] = swz16(kl, wm * 128 + mo);
    fadB[f] = swz16(kl, wn * 128 + mo) + kOpHalfs * 2;
  }
  half8 fa[2][4], fb[2][4];
  auto frags = [&](const _Float16* L, int kk, half8* xa, half8* xb) {
    const char GPTQ_LDS* base = (const char GPTQ_LDS*)L;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const v4s a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s GPTQ_LDS*)(base + fadA[f] + kk * 16 * 512));
      const v4s a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s GPTQ_LDS*)(base + fadA[f] + kk * 16 * 512 + 4 * 512));
      const v4s b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s GPTQ_LDS*)(base + fadB[f] + kk * 16 * 512));
      const v4s b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s GPTQ_LDS*)(base + fadB[f] + kk * 16 * 512 + 4 * 512));
      xa[f] = __builtin_shufflevector(__builtin_bit_cast(half4, a0), __builtin_bit_cast(half4, a1), 0, 1, 2, 3, 4, 5, 6, 7);
      xb[f] = __builtin_shufflevector(__builtin_bit_cast(half4, b0), __builtin_bit_cast(half4, b1), 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto mfmas = [&](const half8* xa, const half8* xb) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa[fm], xb[fn], acc[fm][fn], 0, 0, 0);
  };

  const int nfull = full_cols ? nrows / kKS16 : 0;
  const int nq = nfull >> 2;  // pipelined stages come in fours
  if (nq > 0) {
    // buffer loads with a uniform base that moves with each group of four stages
    // and a per-stage offset inside the group, so the 32-bit offsets span at most
    // five stages of rows at any row width (the launch checks that bound)
    auto rsrc_at = [&](int st) {
      const uint64_t xb = (uint64_t)(uintptr_t)(Xs + (int64_t)(st & ~3) * kKS16 * ldx);
      const uint64_t xu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(xb >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)xb);
      return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)xu, (short)0, 0x7FFFFFFF, 0x00020000);
    };
    const uint32_t ldb = (uint32_t)ldx * 2u;
    // load j (0..3) of this wave fills rows 8 w + 2 j, + 1 of the operand; lane l
    // brings chunk l % 32 of row 8 w + 2 j + l / 32 (its logical chunk unswizzled)
    uint32_t voA[4], voB[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kr = 8 * w + 2 * j + (lane >> 5);
      const int c = (lane & 31) ^ ((kr & 3) << 2);
      voA[j] = (uint32_t)kr * ldb + (uint32_t)(I0 + 8 * c) * 2u;
      voB[j] = (uint32_t)kr * ldb + (uint32_t)(J0 + 8 * c) * 2u;
    }
    const int last = 4 * nq - 1;
    auto dma = [&](_Float16* L, int st) {
      const int sc = min(st, last);
      const __amdgpu_buffer_rsrc_t rsrc = rsrc_at(sc);
      const int so = __builtin_amdgcn_readfirstlane((int)((uint32_t)((sc & 3) * kKS16) * ldb));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void GPTQ_LDS*)(L + (8 * w + 2 * j) * kBT16), 16,
                                                 voA[j], so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void GPTQ_LDS*)(L + kOpHalfs + (8 * w + 2 * j) * kBT16),
                                                 16, voB[j], so, 0, 0);
      }
    };
    dma(L0, 0);
    dma(L1, 1);
    dma(L2, 2);
    dma(L3, 3);
    asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
    frags(L0, 0, fa[0], fb[0]);
    auto step = [&](_Float16* Lc, _Float16* Ln, int s) {
      frags(Lc, 1, fa[1], fb[1]);
      mfmas(fa[0], fb[0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) { GPTQ_SGB(kSgMFMA, 1); GPTQ_SGB(kSgDSR, 2); }
      GPTQ_SGB(kSgMFMA, 8);
      asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      dma(Lc, s + 4);
      frags(Ln, 0, fa[0], fb[0]);
      mfmas(fa[1], fb[1]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        GPTQ_SGB(kSgMFMA, 1);
        if (i < 8) GPTQ_SGB(kSgDSR, 2);
        else GPTQ_SGB(kSgVMEMR, 1);
      }
    };
    for (int q = 0; q < nq; ++q) {
      step(L0, L1, 4 * q + 0);
      step(L1, L2, 4 * q + 1);
      step(L2, L3, 4 * q + 2);
      step(L3, L0, 4 * q + 3);
    }
    // the surplus loads of the last steps must land before L0 is reused
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  // remaining stages (a split's last < 4 full stages, its partial stage, or a
  // partial column tile): masked register loads into L0, not pipelined
  const int nst = (nrows + kKS16 - 1) / kKS16;
  for (int s = 4 * nq; s < nst; ++s) {
    const int k0 = s * kKS16;
    half8 va[4], vb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = t + kThreads * u, k = q >> 5, c = q & 31;
      const int row = k0 + k;
      const bool rok = row < nrows;
      const int64_t rowc = rok ? row : 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ca = I0 + 8 * c + e, cb = J0 + 8 * c + e;
        const _Float16 xa = Xs[rowc * ldx + (ca < d ? ca : 0)];
        const _Float16 xbv = Xs[rowc * ldx + (cb < d ? cb : 0)];
        va[u][e] = (rok && ca < d) ? xa : (_Float16)0.f;
        vb[u][e] = (rok && cb < d) ? xbv : (_Float16)0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = t + kThreads * u, k = q >> 5, c = q & 31;
      *(half8*)((char*)L0 + swz16(k, 8 * c)) = va[u];
      *(half8*)((char*)L0 + kOpHalfs * 2 + swz16(k, 8 * c)) = vb[u];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      frags(L0, kk, fa[0], fb[0]);
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
    int64_t rps, float* __restrict__ part, const TileOrder ord) {
  __shared__ __attribute__((aligned(16))) float lds[2][kKS32 * kP32];
  int64_t tile, split;
  wg_map(ntiles, ord, tile, split);
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
  // 16 rows per thread; four splits' loads in flight per round trip, added in
  // split order
  const float* p0 = part + tile * tsz + (int64_t)(sa * 64 + (t >> 6)) * bt + sc * 64 + col;
  const int64_t sstride = ntiles * tsz;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  int64_t sp = 0;
  for (; sp + 4 <= nsplit; sp += 4) {
    float x[4][16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) x[j][i] = p0[(sp + j) * sstride + (int64_t)(4 * i) * bt];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = (((acc[i] + x[0][i]) + x[1][i]) + x[2][i]) + x[3][i];
  }
  for (; sp < nsplit; ++sp) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = p0[sp * sstride + (int64_t)(4 * i) * bt];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += x[i];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = (t >> 6) + 4 * i;
    const float s = 2.f * acc[i];
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

// Per-XCD tile sets, greedily: each XCD in turn takes ntiles / 8 tiles, always
// one that adds the fewest new column blocks to the blocks it already reads
// (ties: the farthest tile first).  Fewer blocks per XCD = fewer L2 misses.
// Depends on the tile count only; the last result is kept per host thread.
void tile_order(int64_t T, int64_t ntiles, TileOrder& out) {
  thread_local int64_t cached_T = -1;
  thread_local TileOrder cached;
  if (cached_T == T) {
    out = cached;
    return;
  }
  out.n = 0;
  if (ntiles % 8 == 0 && ntiles <= TileOrder::kMax && ntiles > 8) {
    const int64_t per = ntiles / 8;
    std::vector<int> ti(ntiles), tj(ntiles);
    for (int64_t j = 0, t = 0; j < T; ++j)
      for (int64_t i = 0; i <= j; ++i, ++t) {
        ti[t] = (int)i;
        tj[t] = (int)j;
      }
    std::vector<char> used(ntiles, 0);
    int64_t k = 0;
    for (int x = 0; x < 8; ++x) {
      std::vector<char> have(T, 0);
      for (int64_t q = 0; q < per; ++q) {
        int64_t best = -1;
        int bkey = 1 << 30;
        for (int64_t t = 0; t < ntiles; ++t) {
          if (used[t]) continue;
          const int add = !have[ti[t]] + (ti[t] != tj[t] && !have[tj[t]]);
          const int key = add * (1 << 20) - tj[t] * 1024 - ti[t];
          if (key < bkey) {
            bkey = key;
            best = t;
          }
        }
        used[best] = 1;
        have[ti[best]] = have[tj[best]] = 1;
        out.id[k++] = (uint16_t)best;
      }
    }
    out.n = (int)ntiles;
  }
  cached_T = T;
  cached = out;
}

}  // namespace

HessianPlan hessian_plan(int64_t d, int64_t n, int dtype) {
  HessianPlan p{};
  p.dtype = dtype;
  p.bt = (dtype == 1) ? kBT16 : kBT32;
  // fp16 splits are whole multiples of the four-stage pipelined unit
  const int ks = (dtype == 1) ? 4 * kKS16 : kKS32;
  p.tiles_side = cdiv(d, p.bt);
  p.ntiles = p.tiles_side * (p.tiles_side + 1) / 2;
  if (n <= 0) {
    p.nsplit = 0;
    p.rows_per_split = 0;
    p.ws_bytes = 0;
    return p;
  }
  // Splits: at least cdiv(n, 32768) (fp32 accumulation chains of at most 32768
  // rows), at least 4 work-group rounds over the 256 CUs when n allows 1024-row
  // splits, and the first count from there whose work-groups fill their last
  // round to >= 97% (tiles x splits just below a multiple of 256).  Fewer
  // splits means fewer partial tiles to write and reduce.
  const int64_t cus = 256;
  int64_t ns = cdiv(n, 32768);
  const int64_t ns_cap = std::max<int64_t>(1, cdiv(n, 1024));
  ns = std::max(ns, std::min(ns_cap, cdiv(4 * cus, p.ntiles)));
  for (int64_t c = ns; c <= std::min<int64_t>(ns_cap, ns + 64); ++c) {
    const int64_t wg = p.ntiles * c, rounds = cdiv(wg, cus);
    if (wg * 100 >= rounds * cus * 97) {
      ns = c;
      break;
    }
  }
  int64_t rps = cdiv(n, ns);
  rps = cdiv(rps, ks) * ks;
  p.rows_per_split = rps;
  p.nsplit = cdiv(n, rps);
  p.ws_bytes = (size_t)p.nsplit * (size_t)p.ntiles * (size_t)p.bt * (size_t)p.bt * sizeof(float);
  tile_order(p.tiles_side, p.ntiles, p.order);
  return p;
}

hipError_t hessian_launch(const HessianPlan& p, float* H, int64_t d, const void* X, int64_t n,
                          int64_t ldx, void* ws, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  float* part = (float*)ws;
  const int64_t grid = p.ntiles * p.nsplit;
  if (p.dtype == 1) {
    // the fast path addresses five stages of rows with 32-bit byte offsets
    const bool fits = (int64_t)(5 * kKS16) * ldx * 2 + 2 * d < (int64_t(1) << 31);
    const bool vec = fits && (d % 8 == 0) && (ldx % 8 == 0) && (((uintptr_t)X & 15) == 0);
    if (vec)
      hipLaunchKernelGGL(syrk_f16_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         (const _Float16*)X, ldx, n, (int)d, p.ntiles, p.nsplit, p.rows_per_split, part, p.order);
    else
      hipLaunchKernelGGL(syrk_f16_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         (const _Float16*)X, ldx, n, (int)d, p.ntiles, p.nsplit, p.rows_per_split, part, p.order);
  } else {
    const bool vec = (d % 4 == 0) && (ldx % 4 == 0) && (((uintptr_t)X & 15) == 0);
    if (vec)
      hipLaunchKernelGGL(syrk_f32_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         (const float*)X, ldx, n, (int)d, p.ntiles, p.nsplit, p.rows_per_split, part, p.order);
    else
      hipLaunchKernelGGL(syrk_f32_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                         (const float*)X, ldx, n, (int)d, p.ntiles, p.nsplit, p.rows_per_split, part, p.order);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nsub = p.bt / 64;
  hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)(p.ntiles * nsub * nsub)), dim3(kThreads),
                     0, s, part, p.ntiles, p.nsplit, p.bt, (int)d, H);
  return hipGetLastError();
}

}  // namespace gptq
