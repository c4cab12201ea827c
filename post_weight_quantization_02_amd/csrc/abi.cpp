// C ABI of the GPTQ layer solver: argument validation (host, before anything is
// enqueued), workspace queries and stream-ordered launches.  Declarations and
// the contract of every entry point are in include/gptq.h.
#include "gptq.h"

#include <cmath>
#include <vector>

#include "gptq_internal.h"

static_assert(gptq::kNoAllocScratchBytes == GPTQ_NOALLOC_SCRATCH_BYTES, "scratch size");

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 20;        // d_col and d_row limits
constexpr int64_t kMaxElems = int64_t(1) << 40;

bool block_ok(int64_t b) { return b == 16 || b == 32 || b == 64 || b == 128; }

gptq_status ws_check(const void* ws, size_t have, size_t need) {
  if (need == 0) return GPTQ_OK;
  if (ws == nullptr || have < need) return GPTQ_ERR_WORKSPACE;
  return GPTQ_OK;
}

gptq_status from_hip(hipError_t e) { return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_LAUNCH; }

}  // namespace

// ---------------------------------------------------------------- per-launch timing
namespace gptq {

struct LaunchTimer {
  struct Rec {
    int kind;
    double work;
    hipEvent_t a, b;
  };
  bool on = false;
  hipEvent_t open = nullptr;          // begin event of the launch being bracketed
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;       // events of earlier reads, reused

  hipError_t take(hipEvent_t* e) {
    if (!pool.empty()) {
      *e = pool.back();
      pool.pop_back();
      return hipSuccess;
    }
    return hipEventCreate(e);
  }
  ~LaunchTimer() {
    for (auto& r : recs) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    for (auto e : pool) (void)hipEventDestroy(e);
    if (open) (void)hipEventDestroy(open);
  }
};

static LaunchTimer& thread_timer() {
  thread_local LaunchTimer t;
  return t;
}

LaunchTimer* launch_timer() {
  LaunchTimer& t = thread_timer();
  return t.on ? &t : nullptr;
}

hipError_t timer_begin(LaunchTimer* t, hipStream_t s) {
  if (!t) return hipSuccess;
  hipError_t e = t->open ? hipSuccess : t->take(&t->open);
  return e == hipSuccess ? hipEventRecord(t->open, s) : e;
}

hipError_t timer_end(LaunchTimer* t, int kind, double work, hipStream_t s) {
  if (!t || !t->open) return hipSuccess;
  hipEvent_t b = nullptr;
  hipError_t e = t->take(&b);
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  t->recs.push_back({kind, work, t->open, b});
  t->open = nullptr;
  return hipSuccess;
}

}  // namespace gptq

extern "C" {

size_t gptq_hessian_accumulate_workspace_size(int64_t d_col, int64_t n_rows, int32_t x_dtype) {
  if (d_col <= 0 || d_col > kMaxDim || n_rows <= 0 || (x_dtype != GPTQ_F32 && x_dtype != GPTQ_F16))
    return 0;
  return gptq::hessian_plan(d_col, n_rows, x_dtype).ws_bytes;
}

gptq_status gptq_hessian_accumulate(float* H, int64_t d_col, const void* X, int32_t x_dtype,
                                    int64_t n_rows, int64_t ld_x, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (d_col <= 0 || n_rows < 0) return GPTQ_ERR_BAD_SIZE;
  if (d_col > kMaxDim || n_rows > kMaxElems / d_col) return GPTQ_ERR_TOO_LARGE;
  if (x_dtype != GPTQ_F32 && x_dtype != GPTQ_F16) return GPTQ_ERR_BAD_DTYPE;
  if (H == nullptr) return GPTQ_ERR_NULL_POINTER;
  if (n_rows == 0) return GPTQ_OK;
  if (X == nullptr) return GPTQ_ERR_NULL_POINTER;
  if (ld_x < d_col) return GPTQ_ERR_BAD_LEADING_DIM;
  const gptq::HessianPlan plan = gptq::hessian_plan(d_col, n_rows, x_dtype);
  if (gptq_status st = ws_check(ws, ws_bytes, plan.ws_bytes)) return st;
  return from_hip(gptq::hessian_launch(plan, H, d_col, X, n_rows, ld_x, ws, (hipStream_t)stream));
}

size_t gptq_prepare_hinv_workspace_size(int64_t d_col) {
  if (d_col <= 0 || d_col > kMaxDim) return 0;
  return gptq::factor_plan(d_col).ws_bytes;
}

static gptq_status prepare_hinv(const float* H, int64_t d_col, const int32_t* perm, float percdamp,
                                float* U, float* lambda_out, int32_t* info, void* ws, size_t ws_bytes,
                                void* stream) {
  if (d_col <= 0) return GPTQ_ERR_BAD_SIZE;
  if (d_col > kMaxDim) return GPTQ_ERR_TOO_LARGE;
  if (H == nullptr || U == nullptr || lambda_out == nullptr || info == nullptr)
    return GPTQ_ERR_NULL_POINTER;
  if (!std::isfinite(percdamp) || percdamp < 0.f) return GPTQ_ERR_BAD_DAMP;
  const gptq::FactorPlan plan = gptq::factor_plan(d_col);
  if (gptq_status st = ws_check(ws, ws_bytes, plan.ws_bytes)) return st;
  return from_hip(gptq::factor_launch(plan, H, perm, percdamp, U, lambda_out, info, ws, (hipStream_t)stream));
}

gptq_status gptq_prepare_hinv(const float* H, int64_t d_col, float percdamp, float* U,
                              float* lambda_out, int32_t* info, void* ws, size_t ws_bytes,
                              void* stream) {
  return prepare_hinv(H, d_col, nullptr, percdamp, U, lambda_out, info, ws, ws_bytes, stream);
}

gptq_status gptq_act_order_perm(const float* H, int64_t d_col, int32_t* perm, void* stream) {
  if (d_col <= 0) return GPTQ_ERR_BAD_SIZE;
  if (d_col > kMaxDim) return GPTQ_ERR_TOO_LARGE;
  if (H == nullptr || perm == nullptr) return GPTQ_ERR_NULL_POINTER;
  return from_hip(gptq::act_order_launch(H, d_col, perm, (hipStream_t)stream));
}

gptq_status gptq_prepare_hinv_perm(const float* H, int64_t d_col, const int32_t* perm, float percdamp,
                                   float* U, float* lambda_out, int32_t* info, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (perm == nullptr && d_col > 0 && d_col <= kMaxDim) return GPTQ_ERR_NULL_POINTER;
  return prepare_hinv(H, d_col, perm, percdamp, U, lambda_out, info, ws, ws_bytes, stream);
}

size_t gptq_quantize_layer_workspace_size(int64_t d_row, int64_t d_col, int64_t block_size) {
  if (d_row <= 0 || d_col <= 0 || d_row > kMaxDim || d_col > kMaxDim || !block_ok(block_size))
    return 0;
  return gptq::quant_plan(d_row, d_col, block_size).ws_bytes;
}

static gptq_status check_quantize_args(const void* W0, int32_t w_dtype, int64_t d_row, int64_t d_col,
                                       int64_t ld_w, const float* U, int32_t bits, int64_t group_size,
                                       int64_t block_size, const uint8_t* codes, const float* scales,
                                       const int32_t* zeros, const double* out_err) {
  if (d_row <= 0 || d_col <= 0) return GPTQ_ERR_BAD_SIZE;
  if (d_row > kMaxDim || d_col > kMaxDim) return GPTQ_ERR_TOO_LARGE;
  if (w_dtype != GPTQ_F32 && w_dtype != GPTQ_F16) return GPTQ_ERR_BAD_DTYPE;
  if (W0 == nullptr || U == nullptr || codes == nullptr || scales == nullptr || zeros == nullptr ||
      out_err == nullptr)
    return GPTQ_ERR_NULL_POINTER;
  if (ld_w < d_col) return GPTQ_ERR_BAD_LEADING_DIM;
  if (bits < 2 || bits > 8) return GPTQ_ERR_BAD_BITS;
  if (!block_ok(block_size)) return GPTQ_ERR_BAD_BLOCK;
  if (group_size < 0 || (group_size > 0 && (group_size % 16 != 0 ||
                                            (group_size % block_size != 0 &&
                                             block_size % group_size != 0))))
    return GPTQ_ERR_BAD_GROUP;
  return GPTQ_OK;
}

static gptq_status quantize_layer(const void* W0, int32_t w_dtype, int64_t d_row, int64_t d_col,
                                  int64_t ld_w, const float* U, const float* lambda,
                                  const int32_t* perm, int32_t bits, int64_t group_size,
                                  int64_t block_size, uint8_t* codes, float* scales, int32_t* zeros,
                                  int32_t* g_idx, double* out_err, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (gptq_status st = check_quantize_args(W0, w_dtype, d_row, d_col, ld_w, U, bits, group_size,
                                           block_size, codes, scales, zeros, out_err))
    return st;
  const gptq::QuantPlan plan = gptq::quant_plan(d_row, d_col, block_size);
  if (gptq_status st = ws_check(ws, ws_bytes, plan.ws_bytes)) return st;
  return from_hip(gptq::quant_launch(plan, W0, w_dtype, ld_w, U, lambda, perm, bits, group_size, codes,
                                     scales, zeros, g_idx, out_err, ws, (hipStream_t)stream));
}

gptq_status gptq_quantize_layer(const void* W0, int32_t w_dtype, int64_t d_row, int64_t d_col,
                                int64_t ld_w, const float* U, const float* lambda, int32_t bits,
                                int64_t group_size, int64_t block_size, uint8_t* codes,
                                float* scales, int32_t* zeros, double* out_err, void* ws,
                                size_t ws_bytes, void* stream) {
  return quantize_layer(W0, w_dtype, d_row, d_col, ld_w, U, lambda, nullptr, bits, group_size,
                        block_size, codes, scales, zeros, nullptr, out_err, ws, ws_bytes, stream);
}

gptq_status gptq_quantize_layer_noalloc(const void* W0, int32_t w_dtype, int64_t d_row, int64_t d_col,
                                        int64_t ld_w, const float* U, const float* lambda, int32_t bits,
                                        int64_t group_size, int64_t block_size, uint8_t* codes,
                                        float* scales, int32_t* zeros, double* out_err, void* stream) {
  if (gptq_status st = check_quantize_args(W0, w_dtype, d_row, d_col, ld_w, U, bits, group_size,
                                           block_size, codes, scales, zeros, out_err))
    return st;
  const gptq::QuantPlan plan = gptq::quant_plan(d_row, d_col, block_size);
  if (plan.ws_bytes > gptq::kNoAllocScratchBytes) return GPTQ_ERR_SCRATCH;
  void* scratch = nullptr;
  if (gptq::noalloc_scratch(&scratch) != hipSuccess) return GPTQ_ERR_LAUNCH;
  return from_hip(gptq::quant_launch(plan, W0, w_dtype, ld_w, U, lambda, nullptr, bits, group_size, codes,
                                     scales, zeros, nullptr, out_err, scratch, (hipStream_t)stream));
}

gptq_status gptq_quantize_layer_perm(const void* W0, int32_t w_dtype, int64_t d_row, int64_t d_col,
                                     int64_t ld_w, const float* U, const float* lambda,
                                     const int32_t* perm, int32_t bits, int64_t group_size,
                                     int64_t block_size, uint8_t* codes, float* scales,
                                     int32_t* zeros, int32_t* g_idx, double* out_err, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (perm == nullptr || g_idx == nullptr) return GPTQ_ERR_NULL_POINTER;
  return quantize_layer(W0, w_dtype, d_row, d_col, ld_w, U, lambda, perm, bits, group_size,
                        block_size, codes, scales, zeros, g_idx, out_err, ws, ws_bytes, stream);
}

static bool pack_bits_ok(int32_t b) { return b == 2 || b == 3 || b == 4 || b == 8; }

int64_t gptq_packed_words_per_row(int64_t d_col, int32_t bits) {
  if (d_col <= 0 || d_col > kMaxDim || !pack_bits_ok(bits)) return 0;
  return gptq::packed_words_per_row(d_col, bits);
}

gptq_status gptq_pack_codes(const uint8_t* codes, int64_t d_row, int64_t d_col, int64_t ld_codes,
                            int32_t bits, const int32_t* perm, uint32_t* packed, int64_t ld_packed,
                            void* stream) {
  if (d_row <= 0 || d_col <= 0) return GPTQ_ERR_BAD_SIZE;
  if (d_row > kMaxDim || d_col > kMaxDim) return GPTQ_ERR_TOO_LARGE;
  if (codes == nullptr || packed == nullptr) return GPTQ_ERR_NULL_POINTER;
  if (!pack_bits_ok(bits)) return GPTQ_ERR_BAD_BITS;
  if (ld_codes < d_col || ld_packed < gptq::packed_words_per_row(d_col, bits)) return GPTQ_ERR_BAD_LEADING_DIM;
  return from_hip(gptq::pack_launch(codes, d_row, d_col, ld_codes, bits, perm, packed, ld_packed,
                                    (hipStream_t)stream));
}

size_t gptq2d_quantize_workspace_size(int64_t m, int64_t n) {
  if (m <= 0 || n <= 0 || m > kMaxDim || n > kMaxDim) return 0;
  return gptq::plan2d(m, n).ws_bytes;
}

gptq_status gptq2d_quantize(const void* X, int32_t x_dtype, int64_t m, int64_t n, int64_t ldx, const float* U_Q,
                            const float* U_P, int32_t bits, uint8_t* codes, int64_t ld_codes, float* scale,
                            int32_t* zero, double* out_err, void* ws, size_t ws_bytes, void* stream) {
  if (m <= 0 || n <= 0) return GPTQ_ERR_BAD_SIZE;
  if (m > kMaxDim || n > kMaxDim) return GPTQ_ERR_TOO_LARGE;
  if (X == nullptr || U_Q == nullptr || U_P == nullptr || codes == nullptr || scale == nullptr ||
      zero == nullptr || out_err == nullptr)
    return GPTQ_ERR_NULL_POINTER;
  if (x_dtype != GPTQ_F32 && x_dtype != GPTQ_F16) return GPTQ_ERR_BAD_DTYPE;
  if (bits < 2 || bits > 8) return GPTQ_ERR_BAD_BITS;
  if (ldx < n || ld_codes < n) return GPTQ_ERR_BAD_LEADING_DIM;
  const gptq::Plan2D p = gptq::plan2d(m, n);
  if (ws == nullptr || ws_bytes < p.ws_bytes) return GPTQ_ERR_WORKSPACE;
  return from_hip(gptq::quantize2d_launch(p, X, x_dtype == GPTQ_F16 ? 1 : 0, ldx, U_Q, U_P, bits, codes, ld_codes,
                                          scale, zero, out_err, ws, (hipStream_t)stream));
}

gptq_status gptq_dequantize(const uint8_t* codes, int64_t d_row, int64_t d_col, int64_t ld_codes,
                            const float* scales, const int32_t* zeros, int64_t group_size, const int32_t* g_idx,
                            void* out, int32_t out_dtype, int64_t ld_out, void* stream) {
  if (d_row <= 0 || d_col <= 0) return GPTQ_ERR_BAD_SIZE;
  if (d_row > kMaxDim || d_col > kMaxDim) return GPTQ_ERR_TOO_LARGE;
  if (codes == nullptr || scales == nullptr || zeros == nullptr || out == nullptr) return GPTQ_ERR_NULL_POINTER;
  if (out_dtype != GPTQ_F32 && out_dtype != GPTQ_F16) return GPTQ_ERR_BAD_DTYPE;
  if (group_size < 0) return GPTQ_ERR_BAD_GROUP;
  if (ld_codes < d_col || ld_out < d_col) return GPTQ_ERR_BAD_LEADING_DIM;
  return from_hip(gptq::dequantize_launch(codes, d_row, d_col, ld_codes, scales, zeros, group_size, g_idx, out,
                                          out_dtype == GPTQ_F16 ? 1 : 0, ld_out, (hipStream_t)stream));
}

gptq_status gptq_dequant_matmul(const uint32_t* packed, int64_t ld_packed, int32_t bits,
                                const float* scales, const int32_t* zeros, int64_t group_size,
                                const int32_t* perm, int64_t d_row, int64_t d_col, const void* X,
                                int32_t x_dtype, int64_t m, int64_t ld_x, float* Y, int64_t ld_y,
                                void* stream) {
  if (d_row <= 0 || d_col <= 0 || m <= 0) return GPTQ_ERR_BAD_SIZE;
  if (d_row > kMaxDim || d_col > kMaxDim || m > 8) return GPTQ_ERR_TOO_LARGE;
  if (packed == nullptr || scales == nullptr || zeros == nullptr || X == nullptr || Y == nullptr)
    return GPTQ_ERR_NULL_POINTER;
  if (!pack_bits_ok(bits)) return GPTQ_ERR_BAD_BITS;
  if (x_dtype != GPTQ_F32 && x_dtype != GPTQ_F16) return GPTQ_ERR_BAD_DTYPE;
  if (group_size < 0 || (group_size > 0 && group_size % 16 != 0)) return GPTQ_ERR_BAD_GROUP;
  if (ld_packed < gptq::packed_words_per_row(d_col, bits) || ld_x < d_col || ld_y < d_row)
    return GPTQ_ERR_BAD_LEADING_DIM;
  return from_hip(gptq::dequant_matmul_launch(packed, ld_packed, bits, scales, zeros, group_size, perm,
                                              d_row, d_col, X, x_dtype, (int)m, ld_x, Y, ld_y,
                                              (hipStream_t)stream));
}

gptq_status gptq_launch_timing(int32_t enable) {
  gptq::thread_timer().on = enable != 0;
  return GPTQ_OK;
}

gptq_status gptq_launch_timing_read(int32_t kind, double* ms, int64_t* launches, double* work) {
  if (ms == nullptr || launches == nullptr || work == nullptr) return GPTQ_ERR_NULL_POINTER;
  if (kind < 0 || kind >= gptq::kTimeKinds) return GPTQ_ERR_BAD_SIZE;
  gptq::LaunchTimer& t = gptq::thread_timer();
  *ms = 0.0;
  *launches = 0;
  *work = 0.0;
  std::vector<gptq::LaunchTimer::Rec> keep;
  for (auto& r : t.recs) {
    if (r.kind != kind) {
      keep.push_back(r);
      continue;
    }
    float dt = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&dt, r.a, r.b) != hipSuccess)
      return GPTQ_ERR_LAUNCH;
    *ms += dt;
    *launches += 1;
    *work += r.work;
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.recs.swap(keep);
  return GPTQ_OK;
}

const char* gptq_status_string(int32_t status) {
  switch (status) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_NULL_POINTER: return "a required pointer is NULL";
    case GPTQ_ERR_BAD_SIZE: return "a size is zero or negative";
    case GPTQ_ERR_BAD_LEADING_DIM: return "leading dimension smaller than the row width";
    case GPTQ_ERR_BAD_DTYPE: return "unsupported element type";
    case GPTQ_ERR_BAD_BITS: return "bits must be in [2, 8] (2, 3, 4 or 8 for packed codes)";
    case GPTQ_ERR_BAD_BLOCK: return "block_size must be 16, 32, 64 or 128";
    case GPTQ_ERR_BAD_GROUP: return "group_size must be 0, or a multiple of 16 that divides or is divided by block_size";
    case GPTQ_ERR_WORKSPACE: return "workspace missing or smaller than the query";
    case GPTQ_ERR_BAD_DAMP: return "percdamp must be finite and >= 0";
    case GPTQ_ERR_LAUNCH: return "a HIP launch or runtime call failed";
    case GPTQ_ERR_TOO_LARGE: return "a size exceeds the library limits";
    case GPTQ_ERR_SCRATCH:
      return "the shape needs more workspace than the no-allocation entry point holds "
             "(gptq_quantize_layer_workspace_size > GPTQ_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

const char* gptq_version(void) { return "gptq-gfx950 0.1.0"; }

}  // extern "C"
