// Internal declarations shared by the gfx950 kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

namespace gptq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- Hessian
// Tile visiting order for the Hessian work-groups (upper-triangle tile ids),
// passed by value as a kernel argument.
struct TileOrder {
  static constexpr int kMax = 1024;
  int n;                  // 0: natural order
  uint16_t id[kMax];
};

struct HessianPlan {
  int dtype;              // 0 = f32, 1 = f16
  int bt;                 // square tile edge
  int64_t tiles_side;     // ceil(d / bt)
  int64_t ntiles;         // upper-triangle tiles
  int64_t nsplit;         // row ranges reduced in a fixed order
  int64_t rows_per_split;
  size_t ws_bytes;        // partial tiles
  TileOrder order;        // tiles grouped per XCD to share column blocks in its L2
};
HessianPlan hessian_plan(int64_t d, int64_t n, int dtype);
hipError_t hessian_launch(const HessianPlan& p, float* H, int64_t d, const void* X, int64_t n,
                          int64_t ldx, void* ws, hipStream_t s);

// ---------------------------------------------------------------- factor
struct FactorPlan {
  int64_t d;
  int nb;                 // Cholesky block
  int64_t nblk;
  size_t part_slot;       // doubles per half of the deferred-product double buffer
  size_t off_a64, off_part, off_tw, off_tmp, ws_bytes;
};
FactorPlan factor_plan(int64_t d);
// perm: NULL, or the order in which the columns are factored (H[perm][:, perm])
hipError_t factor_launch(const FactorPlan& p, const float* H, const int32_t* perm, float percdamp,
                         float* U, float* lambda_out, int32_t* info, void* ws, hipStream_t s);
// act-order: perm[i] = the column taken at position i (descending diag(H), stable)
hipError_t act_order_launch(const float* H, int64_t d, int32_t* perm, hipStream_t s);

// ---------------------------------------------------------------- packed codes
int64_t packed_words_per_row(int64_t d_col, int bits);
hipError_t pack_launch(const uint8_t* codes, int64_t d_row, int64_t d_col, int64_t ld_codes, int bits,
                       const int32_t* perm, uint32_t* packed, int64_t ld_packed, hipStream_t s);
hipError_t dequantize_launch(const uint8_t* codes, int64_t d_row, int64_t d_col, int64_t ld_codes,
                             const float* scales, const int32_t* zeros, int64_t group, const int32_t* g_idx,
                             void* out, int out_dtype, int64_t ld_out, hipStream_t s);
hipError_t dequant_matmul_launch(const uint32_t* packed, int64_t ld_packed, int bits, const float* scales,
                                 const int32_t* zeros, int64_t group, const int32_t* perm, int64_t d_row,
                                 int64_t d_col, const void* X, int x_dtype, int m, int64_t ld_x, float* Y,
                                 int64_t ld_y, hipStream_t s);

// ---------------------------------------------------------------- two-sided rounding
struct Plan2D {
  int64_t m, n, Mb, Nb;   // matrix and 32-tile counts
  int64_t nchunk_a;       // correction chunks per tile (8 tile-rows each)
  size_t off_m, off_e, off_cpart, off_err, off_part, off_grid, ws_bytes;
};
Plan2D plan2d(int64_t m, int64_t n);
hipError_t quantize2d_launch(const Plan2D& p, const void* X, int x_dtype, int64_t ldx, const float* UQ,
                             const float* UP, int bits, uint8_t* codes, int64_t ldc, float* scale, int32_t* zero,
                             double* out_err, void* ws, hipStream_t s);

// ---------------------------------------------------------------- quantize
struct QuantPlan {
  int64_t d_row, d_col, B, nblk;
  int64_t panel_wgs;      // work-groups of the panel kernel
  int pair;               // blocks grouped in the out-of-block update: pairs whose odd
                          // block's panel takes the even block's share (1), or groups of
                          // up to four blocks with thin launches inside the group (2)
  size_t off_w, off_e, off_part, off_err, off_cpos, ws_bytes;
};
QuantPlan quant_plan(int64_t d_row, int64_t d_col, int64_t B);
// perm: NULL (natural order) or the quantization order (position c takes column
// perm[c] of W0; codes land in the original columns; groups are runs of
// positions); g_idx: NULL or the group of every original column
hipError_t quant_launch(const QuantPlan& p, const void* W0, int w_dtype, int64_t ldw,
                        const float* U, const float* lambda, const int32_t* perm, int bits,
                        int64_t group, uint8_t* codes, float* scales, int32_t* zeros,
                        int32_t* g_idx, double* out_err, void* ws, hipStream_t s);

// ---------------------------------------------------------------- per-launch timing
// A measurement aid, off by default: when switched on for the calling host
// thread, the loop brackets each in-block panel launch (kind 0) and each
// out-of-block product launch (kind 1) with a pair of HIP events recorded on
// the call's stream, and notes the launch's algorithmic work (bytes for the
// panel, flop for the product).
enum { kTimePanel = 0, kTimeTrail = 1, kTimeKinds = 2 };
struct LaunchTimer;
LaunchTimer* launch_timer();   // the calling thread's timer, or nullptr when off
hipError_t timer_begin(LaunchTimer* t, hipStream_t s);
hipError_t timer_end(LaunchTimer* t, int kind, double work, hipStream_t s);

// The no-allocation entry point's workspace: a device array of this many bytes
// (one per device), and its address on the current device (looked up once per
// device, then kept).
constexpr size_t kNoAllocScratchBytes = size_t(96) << 20;
hipError_t noalloc_scratch(void** out);

// The one-row-per-lane panel for full blocks of 128 columns (layers with many
// rows): one grid per row (or per group wider than the block), or one group per
// block.  grid.x * block.x >= d_row, block.x a multiple of 64 up to 256.
hipError_t row_panel_launch_grid(dim3 grid, dim3 block, hipStream_t s, float* W, int d_row, int d_col, int i1,
                                 const float* U, int maxq, int gwide, int ngroups, uint8_t* codes,
                                 float* scales, int32_t* zeros, float* E, double* part_e);
hipError_t row_panel_launch_group(dim3 grid, dim3 block, hipStream_t s, float* W, int d_row, int d_col, int i1,
                                  const float* U, int maxq, int gwide, int ngroups, uint8_t* codes,
                                  float* scales, int32_t* zeros, float* E, double* part_e);

// W[:, i+B:] -= E U[i:i+B, i+B:] with E given transposed: C [M x N] (ldc) -=
// Et^T [M x K] * Ub [K x N]; Et is [K x M] (lde), Ub [K x N] (ldu); K <= 128.
hipError_t trail_update_launch(float* C, int64_t ldc, int M, int N, int K, const float* Et,
                               int64_t lde, const float* Ub, int64_t ldu, hipStream_t s);

}  // namespace gptq
