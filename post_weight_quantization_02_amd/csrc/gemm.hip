// Out-of-block correction of the lazy batch on fp32 matrix cores:
//   W[:, i+B:] -= E U[i:i+B, i+B:]
// (itwiki "GPTQ", three-changes table, change 2, and the last line of
// Algorithm 1).  K = B <= 128 (or the rows of up to four blocks, up to 512, when
// the caller groups blocks), M = d_row, N = the columns after the block.
//
// E arrives transposed (Et [B x d_row], written that way by the panel kernel)
// so that both operands stage with 16-byte loads along the M or N direction
// and land in LDS as [k][m] / [k][n]: the v_mfma_f32_32x32x2f32 operands are
// then one LDS word per lane with 32 consecutive lanes on consecutive words.
// 128x128 output tile per work-group (4 waves, 64x64 each), K in two 64-deep
// phases (67 KB LDS, two work-groups per CU); the C tile is read into
// registers at the start (its traffic hides under the MFMAs) and written once.  Tiles are mapped so that each XCD runs a contiguous range.
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kT = 128, kKP = 64, kP = kT + 4, kThreads = 256;
#define GPTQ_LDS __attribute__((address_space(3)))

__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t total) {
  const int64_t q = total / 8, r = total % 8;
  const int64_t x = bid % 8, i = bid / 8;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void trail_kernel(float* __restrict__ C, int64_t ldc,
                                                         int M, int N, int K,
                                                         const float* __restrict__ Et, int64_t lde,
                                                         const float* __restrict__ Ub, int64_t ldu,
                                                         int64_t tiles_m, int64_t tiles_n) {
  __shared__ __attribute__((aligned(16))) float SA[kKP * kP];
  __shared__ __attribute__((aligned(16))) float SB[kKP * kP];
  const int64_t lid = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int m0 = (int)(lid / tiles_n) * kT, n0 = (int)(lid % tiles_n) * kT;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, wm = w & 1, wn = w >> 1;

  // staging: thread t covers k rows t/32 + 8 i (i < 8) and 4 columns at (t % 32) * 4
  const int sk = t >> 5, sc = (t & 31) * 4;
  auto load4 = [&](const float* __restrict__ base, int64_t ld, int k, int x0, int lim) {
    f32x4 v;
    const int x = x0 + sc;
    if (VEC && k < K && x + 3 < lim) {
      v = *(const f32x4*)(base + (int64_t)k * ld + x);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (k < K && x + e < lim) ? base[(int64_t)k * ld + x + e] : 0.f;
    }
    return v;
  };
  f32x4 ra[8], rb[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + sk + 8 * i;
      ra[i] = load4(Et, lde, k, m0, M);
      rb[i] = load4(Ub, ldu, k, n0, N);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *(f32x4*)&SA[(sk + 8 * i) * kP + sc] = ra[i];
      *(f32x4*)&SB[(sk + 8 * i) * kP + sc] = rb[i];
    }
  };

  // C tile in the MFMA output layout, read at the start of the last K phase
  // (the staging registers are free by then; its latency hides under the MFMAs)
  float c[2][2][16];
  auto cload = [&]() {
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 2; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * 64 + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = n0 + wn * 64 + fn * 32 + (lane & 31);
          c[fm][fn][r] = (row < M && col < N) ? C[(int64_t)row * ldc + col] : 0.f;
        }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  auto mfma_phase = [&](int kn) {
#pragma unroll 4
    for (int kk = 0; kk < kKP / 2; ++kk) {
      if (2 * kk >= kn) break;
      const int k = 2 * kk + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        a[f] = SA[k * kP + wm * 64 + f * 32 + (lane & 31)];
        b[f] = SB[k * kP + wn * 64 + f * 32 + (lane & 31)];
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
  };
  // K <= 128: one or two straight-line phases of 64
  gload(0);
  lstore();
  __syncthreads();
  if (K > kKP) {
    gload(kKP);
    mfma_phase(kKP);
    __syncthreads();
    lstore();
    __syncthreads();
    cload();
    mfma_phase(K - kKP);
  } else {
    cload();
    mfma_phase(K);
  }
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = n0 + wn * 64 + fn * 32 + (lane & 31);
        if (row < M && col < N) C[(int64_t)row * ldc + col] = c[fm][fn][r] - acc[fm][fn][r];
      }
}


// ---------------------------------------------------------------------------
// Aligned operands (the usual case): the same 128x128 tile, with Et and U rows
// streamed by buffer loads straight into LDS (their row-major [k][m] / [k][n]
// layout is already what the 32x32x2 MFMA reads), K in up to sixteen sub-phases
// of 32 rows double-buffered, and the C tile read under the first sub-phase's
// MFMAs in a coalesced per-wave layout.  Each wave finishes its own 64x64 quadrant through a
// private LDS array: accumulators in, row-major out, C - acc, store.
// Rows past K and columns past N read zeros or neighbouring data that only
// reaches discarded outputs; the buffer extents keep every read inside Et and U.
constexpr int kKS = 32;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int NSUB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void trail_dma_kernel(float* __restrict__ C, int64_t ldc,
                                                             int M, int N, int K,
                                                             const float* __restrict__ Et, int64_t lde,
                                                             const float* __restrict__ Ub, int64_t ldu,
                                                             int64_t tiles_m, int64_t tiles_n) {
  __shared__ __attribute__((aligned(16))) float E0[kKS * kT];
  __shared__ __attribute__((aligned(16))) float U0[kKS * kT];
  __shared__ __attribute__((aligned(16))) float E1[kKS * kT];
  __shared__ __attribute__((aligned(16))) float U1[kKS * kT];
  const int64_t lid = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int m0 = (int)(lid / tiles_n) * kT, n0 = (int)(lid % tiles_n) * kT;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w & 1, wn = w >> 1;

  auto uniform_ptr = [](const float* p) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    return (const float*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32) |
                                     (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b));
  };
  // buffer extents: K rows of Et from column m0, K rows of U from column n0
  const float* eb = uniform_ptr(Et + m0);
  const float* ub = uniform_ptr(Ub + n0);
  const uint32_t ebytes = (uint32_t)(((int64_t)(K - 1) * lde + (M - m0)) * 4);
  const uint32_t ubytes = (uint32_t)(((int64_t)(K - 1) * ldu + (N - n0)) * 4);
  const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc((void*)eb, (short)0, (int)ebytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t ur = __builtin_amdgcn_make_buffer_rsrc((void*)ub, (short)0, (int)ubytes, 0x00020000);
  // load j of this wave fills rows 8 w + 2 j, + 1 (lane / 32) of a 32-row sub-phase
  uint32_t voE[4], voU[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kr = 8 * w + 2 * j + (lane >> 5);
    voE[j] = (uint32_t)(kr * lde + (lane & 31) * 4) * 4u;
    voU[j] = (uint32_t)(kr * ldu + (lane & 31) * 4) * 4u;
  }
  auto dma = [&](float* LE, float* LU, int sub) {
    const int soE = __builtin_amdgcn_readfirstlane((int)((uint32_t)(sub * kKS) * (uint32_t)lde * 4u));
    const int soU = __builtin_amdgcn_readfirstlane((int)((uint32_t)(sub * kKS) * (uint32_t)ldu * 4u));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(er, (void GPTQ_LDS*)(LE + (8 * w + 2 * j) * kT), 16, voE[j], soE, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ur, (void GPTQ_LDS*)(LU + (8 * w + 2 * j) * kT), 16, voU[j], soU, 0, 0);
    }
  };
  // C quadrant of this wave, coalesced: rows lane / 16 + 4 i, columns 4 (lane % 16) .. + 3.
  // Exactly 16 loads per wave, always issued (the waits below count them): a lane
  // outside M x N reads an in-bounds vector instead, whose value is never stored.
  const int qr0 = m0 + wm * 64 + (lane >> 4), qc = n0 + wn * 64 + (lane & 15) * 4;
  const int qcl = std::min(qc, (N - 4) & ~3);
  f32x4 cq[16];
  auto cload = [&]() {
    asm volatile("" ::: "memory");  // keep the C loads after the sub-phase loads
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = std::min(qr0 + 4 * i, M - 1);
      cq[i] = *(const f32x4*)(C + (int64_t)row * ldc + qcl);
    }
    asm volatile("" ::: "memory");
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  auto compute = [&](const float* LE, const float* LU, int sub) {
    const int kv = K - sub * kKS;  // valid rows in this sub-phase
#pragma unroll
    for (int kk = 0; kk < kKS / 2; ++kk) {
      const int k = 2 * kk + (lane >> 5);
      float a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        a[f] = LE[k * kT + wm * 64 + f * 32 + (lane & 31)];
        b[f] = LU[k * kT + wn * 64 + f * 32 + (lane & 31)];
        if (kv < kKS) a[f] = (k < kv) ? a[f] : 0.f;
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
    }
  };

  // sub-phase s lives in buffer s % 2; the loads of s + 1 run under the MFMAs of
  // s.  C is read right after the first two sub-phases' loads, so its HBM
  // traffic spreads over all the tile's MFMAs.  Each wait for sub-phase s allows
  // exactly the loads issued after it to stay in flight (8 per sub-phase, 16 for
  // C), so it never waits for C or a later sub-phase.
  dma(E0, U0, 0);
  if constexpr (NSUB > 1) {
    dma(E1, U1, 1);
    cload();
    asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
  } else {
    cload();
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  }
  compute(E0, U0, 0);
  // sub-phase S: once every wave is past S - 1 (whose buffer S + 1 reuses), the
  // loads of S + 1 go out; the wait for S then lets exactly C (if S == 1) and
  // S + 1 stay in flight
  static_for<1, NSUB>([&](auto SS) {
    constexpr int S = decltype(SS)::value;
    if constexpr (S + 1 < NSUB) {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if constexpr ((S + 1) % 2 == 0) dma(E0, U0, S + 1);
      else dma(E1, U1, S + 1);
      if constexpr (S == 1) asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    } else {
      if constexpr (S == 1) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if constexpr (S % 2 == 0) compute(E0, U0, S);
    else compute(E1, U1, S);
  });
  // epilogue: every wave is done with the operand buffers after this barrier
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  float* Q = (w == 0) ? E0 : (w == 1) ? U0 : (w == 2) ? E1 : U1;  // 64x64 private quadrant
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = fm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = fn * 32 + (lane & 31);
        Q[row * 64 + col] = acc[fm][fn][r];
      }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): own writes done before own reads
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int lr = (lane >> 4) + 4 * i;
    const f32x4 a = *(const f32x4*)&Q[lr * 64 + (lane & 15) * 4];
    const int row = qr0 + 4 * i;
    const f32x4 v = cq[i] - a;
    if (row < M && qc + 3 < N) {
      *(f32x4*)(C + (int64_t)row * ldc + qc) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (row < M && qc + e < N) C[(int64_t)row * ldc + qc + e] = v[e];
    }
  }
}

}  // namespace

// the instantiation with nsub sub-phases of 32 rows (1 .. 16)
template <int NS>
void launch_dma(int nsub, dim3 g, dim3 b, hipStream_t s, float* C, int64_t ldc, int M, int N, int K,
                const float* Et, int64_t lde, const float* Ub, int64_t ldu, int64_t tm, int64_t tn) {
  if constexpr (NS < 16) {
    if (nsub != NS) return launch_dma<NS + 1>(nsub, g, b, s, C, ldc, M, N, K, Et, lde, Ub, ldu, tm, tn);
  }
  hipLaunchKernelGGL(trail_dma_kernel<NS>, g, b, 0, s, C, ldc, M, N, K, Et, lde, Ub, ldu, tm, tn);
}

hipError_t trail_update_launch(float* C, int64_t ldc, int M, int N, int K, const float* Et,
                               int64_t lde, const float* Ub, int64_t ldu, hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  const int64_t tm = cdiv(M, kT), tn = cdiv(N, kT);
  const bool vec = (lde % 4 == 0) && (ldu % 4 == 0) && (((uintptr_t)Et & 15) == 0) &&
                   (((uintptr_t)Ub & 15) == 0);
  // buffer loads need 32-bit byte extents and 16-byte rows
  const bool dma = vec && (ldc % 4 == 0) && (((uintptr_t)C & 15) == 0) && K <= 16 * kKS && N >= 4 &&
                   (int64_t)K * std::max(lde, ldu) * 4 < (int64_t(1) << 31);
  if (dma) {
    const dim3 g((unsigned)(tm * tn)), b(kThreads);
    launch_dma<1>((K + kKS - 1) / kKS, g, b, s, C, ldc, M, N, K, Et, lde, Ub, ldu, tm, tn);
  } else {
    // the register-staged kernel takes K <= 2 kKP per launch
    for (int k0 = 0; k0 < K; k0 += 2 * kKP) {
      const int kc = std::min(2 * kKP, K - k0);
      if (vec)
        hipLaunchKernelGGL(trail_kernel<true>, dim3((unsigned)(tm * tn)), dim3(kThreads), 0, s, C, ldc,
                           M, N, kc, Et + (int64_t)k0 * lde, lde, Ub + (int64_t)k0 * ldu, ldu, tm, tn);
      else
        hipLaunchKernelGGL(trail_kernel<false>, dim3((unsigned)(tm * tn)), dim3(kThreads), 0, s, C, ldc,
                           M, N, kc, Et + (int64_t)k0 * lde, lde, Ub + (int64_t)k0 * ldu, ldu, tm, tn);
    }
  }
  return hipGetLastError();
}

}  // namespace gptq
