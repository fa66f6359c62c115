// tq_api.cpp -- the C ABI declared in include/tq.h: argument validation on the
// host, then kernel launches on the caller's stream.  Nothing here allocates,
// frees or synchronizes.
#include <hip/hip_runtime.h>

#include "../../include/tq.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxRows = int64_t(1) << 26;
constexpr int64_t kMaxCols = int64_t(1) << 20;
constexpr int64_t kMaxWeights = int64_t(1) << 36;
constexpr int64_t kMaxTokens = int64_t(1) << 20;
constexpr int64_t kMaxPtq1Cols = 32768;  // the ptq1_0 tables of one workgroup (1792 B per 1024 cols and token) stay within its LDS budget

bool fmt_ok(int f) { return f == TQ_FMT_PQ2_0 || f == TQ_FMT_PTQ1_0; }

int shape_status(int f, int64_t rows, int64_t cols, int64_t tokens) {
  if (!fmt_ok(f)) return TQ_ERR_FORMAT;
  if (rows < 1 || rows > kMaxRows || cols < 256 || cols > kMaxCols || cols % 256 != 0) return TQ_ERR_SHAPE;
  if (rows * cols > kMaxWeights) return TQ_ERR_SHAPE;
  if (tokens < 1 || tokens > kMaxTokens || tokens * cols > kMaxWeights) return TQ_ERR_SHAPE;
  if (f == TQ_FMT_PTQ1_0 && cols > kMaxPtq1Cols) return TQ_ERR_SHAPE;
  return TQ_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return TQ_OK;
  g_last_hip_error = (int)e;
  return TQ_ERR_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Shared checks of the product entry points.
int product_args(int fmt, const void* w, int64_t rows, int64_t cols, int64_t tokens, const int8_t* q, const float* d,
                 const int16_t* bsums, const void* out, bool need_d) {
  const int st = shape_status(fmt, rows, cols, tokens);
  if (st != TQ_OK) return st;
  if (!w || !q || !out || (need_d && !d)) return TQ_ERR_NULL;
  if (fmt == TQ_FMT_PTQ1_0 && !bsums) return TQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(out, 4) || (d && !aligned(d, 4)) || (bsums && !aligned(bsums, 2)))
    return TQ_ERR_ALIGN;
  return TQ_OK;
}

}  // namespace

extern "C" {

int tq_check_shape(int fmt, int64_t rows, int64_t cols, int64_t tokens) { return shape_status(fmt, rows, cols, tokens); }

int64_t tq_canonical_bytes(int fmt, int64_t rows, int64_t cols) {
  if (shape_status(fmt, rows, cols, 1) != TQ_OK) return 0;
  return rows * (cols / 128) * (fmt == TQ_FMT_PQ2_0 ? 34 : 28);
}

int64_t tq_repacked_bytes(int fmt, int64_t rows, int64_t cols) {
  if (shape_status(fmt, rows, cols, 1) != TQ_OK) return 0;
  const tq::Dims dm = tq::dims(rows, cols);
  return fmt == TQ_FMT_PQ2_0 ? tq::pq2_code_bytes(dm) + tq::pq2_scale_bytes(dm) : tq::ptq1_code_bytes(dm) + tq::ptq1_scale_bytes(dm);
}

int tq_repack(int fmt, const void* src, void* dst, int64_t rows, int64_t cols, int32_t* bad_flag, void* stream) {
  const int st = shape_status(fmt, rows, cols, 1);
  if (st != TQ_OK) return st;
  if (!src || !dst) return TQ_ERR_NULL;
  if (!aligned(dst, 16) || (bad_flag && !aligned(bad_flag, 4))) return TQ_ERR_ALIGN;
  const tq::Dims dm = tq::dims(rows, cols);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  uint8_t* o = static_cast<uint8_t*>(dst);
  if (fmt == TQ_FMT_PQ2_0) return hip_status(tq::launch_repack_pq2(s, o, dm, bad_flag, as_stream(stream)));
  return hip_status(tq::launch_repack_ptq1(s, o, dm, as_stream(stream)));
}

int tq_unrepack(int fmt, const void* src_repacked, void* dst, int64_t rows, int64_t cols, void* stream) {
  const int st = shape_status(fmt, rows, cols, 1);
  if (st != TQ_OK) return st;
  if (!src_repacked || !dst) return TQ_ERR_NULL;
  if (!aligned(src_repacked, 16)) return TQ_ERR_ALIGN;
  const tq::Dims dm = tq::dims(rows, cols);
  const uint8_t* s = static_cast<const uint8_t*>(src_repacked);
  uint8_t* o = static_cast<uint8_t*>(dst);
  if (fmt == TQ_FMT_PQ2_0) return hip_status(tq::launch_unrepack_pq2(s, o, dm, as_stream(stream)));
  return hip_status(tq::launch_unrepack_ptq1(s, o, dm, as_stream(stream)));
}

int tq_quantize_q8k(const float* x, int64_t tokens, int64_t cols, int8_t* q, float* d, int16_t* bsums, void* stream) {
  const int st = shape_status(TQ_FMT_PQ2_0, 1, cols, tokens);
  if (st != TQ_OK) return st;
  if (!x || !q || !d || !bsums) return TQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(bsums, 2)) return TQ_ERR_ALIGN;
  return hip_status(tq::launch_quantize_q8k(x, tokens * cols / 256, q, d, bsums, as_stream(stream)));
}

int64_t tq_workspace_bytes(int fmt, int64_t rows, int64_t cols, int64_t tokens) {
  if (shape_status(fmt, rows, cols, tokens) != TQ_OK) return 0;
  return tq::workspace_bytes(tq::dims(rows, cols));
}

int tq_workspace_clear(void* workspace, int64_t bytes, void* stream) {
  if (bytes < 0) return TQ_ERR_SHAPE;
  if (bytes == 0) return TQ_OK;
  if (!workspace) return TQ_ERR_NULL;
  if (!aligned(workspace, 16)) return TQ_ERR_ALIGN;
  return hip_status(tq::launch_clear(workspace, bytes, as_stream(stream)));
}

int tq_gemv(int fmt, const void* w, int64_t rows, int64_t cols, const int8_t* q, const float* d, const int16_t* bsums,
            float* y, void* workspace, void* stream) {
  const int st = product_args(fmt, w, rows, cols, 1, q, d, bsums, y, true);
  if (st != TQ_OK) return st;
  if (workspace && !aligned(workspace, 16)) return TQ_ERR_ALIGN;
  const tq::Dims dm = tq::dims(rows, cols);
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  if (fmt == TQ_FMT_PQ2_0) return hip_status(tq::launch_gemv_pq2(wb, dm, q, d, y, nullptr, workspace, as_stream(stream)));
  return hip_status(tq::launch_gemv_ptq1(wb, dm, q, d, bsums, y, nullptr, workspace, as_stream(stream)));
}

int tq_gemv_f32(int fmt, const void* w, int64_t rows, int64_t cols, const float* x, float* y, void* workspace,
                void* stream) {
  // shape, then what this entry supports (a property of the shape alone), then the pointers
  const int st = shape_status(fmt, rows, cols, 1);
  if (st != TQ_OK) return st;
  const tq::Dims dm = tq::dims(rows, cols);
  if (fmt != TQ_FMT_PQ2_0 || !tq::gemv_pq2_fused_fits(dm, workspace != nullptr)) return TQ_ERR_UNSUPPORTED;
  if (!w || !x || !y) return TQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4) || (workspace && !aligned(workspace, 16))) return TQ_ERR_ALIGN;
  return hip_status(tq::launch_gemv_pq2_fused(static_cast<const uint8_t*>(w), dm, x, y, workspace, as_stream(stream)));
}

int tq_gemv_f32_scratch(int fmt, const void* w, int64_t rows, int64_t cols, const float* x, float* y, void* stream) {
  const int st = shape_status(fmt, rows, cols, 1);
  if (st != TQ_OK) return st;
  const tq::Dims dm = tq::dims(rows, cols);
  if (fmt != TQ_FMT_PQ2_0 || !tq::gemv_pq2_fused_fits(dm, true)) return TQ_ERR_UNSUPPORTED;
  // the split's workspace must fit the static scratch (always, for the current plan)
  const tq::GemvPlan p = tq::plan_gemv_pq2(dm, true);
  if (p.slices > 1 && tq::workspace_bytes(dm) > tq::scratch_bytes()) return TQ_ERR_UNSUPPORTED;
  if (!w || !x || !y) return TQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return TQ_ERR_ALIGN;
  void* ws = nullptr;
  const hipError_t e = tq::scratch_ptr(as_stream(stream), &ws);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(tq::launch_gemv_pq2_fused(static_cast<const uint8_t*>(w), dm, x, y, ws, as_stream(stream)));
}

int tq_gemv_f32_batch(int fmt, int n, const void* const* w, const int64_t* rows, int64_t cols, const float* const* x,
                      float* const* y, void* workspace, void* stream) {
  if (!fmt_ok(fmt)) return TQ_ERR_FORMAT;
  if (n < 1 || n > tq::kMaxBatch) return TQ_ERR_SHAPE;
  if (!w || !rows || !x || !y) return TQ_ERR_NULL;
  int64_t tiles = 0;
  for (int m = 0; m < n; ++m) {
    const int st = shape_status(fmt, rows[m], cols, 1);
    if (st != TQ_OK) return st;
    tiles += (rows[m] + 63) / 64;
  }
  if (shape_status(fmt, tiles * 64, cols, 1) != TQ_OK) return TQ_ERR_SHAPE;
  const tq::Dims dm = tq::dims(tiles * 64, cols);
  if (fmt != TQ_FMT_PQ2_0 || !tq::gemv_pq2_fused_fits(dm, workspace != nullptr)) return TQ_ERR_UNSUPPORTED;
  tq::GemvBatch b{};
  b.n = n;
  b.tile0[0] = 0;
  for (int m = 0; m < n; ++m) {
    if (!w[m] || !x[m] || !y[m]) return TQ_ERR_NULL;
    if (!aligned(w[m], 16) || !aligned(x[m], 16) || !aligned(y[m], 4)) return TQ_ERR_ALIGN;
    const tq::Dims dmm = tq::dims(rows[m], cols);
    const uint8_t* wb = static_cast<const uint8_t*>(w[m]);
    b.codes[m] = reinterpret_cast<const uint4*>(wb);
    b.scales[m] = reinterpret_cast<const uint32_t*>(wb + tq::kPq2ScaleOffset);
    b.x[m] = reinterpret_cast<const float4*>(x[m]);
    b.y[m] = y[m];
    b.rows[m] = (int)rows[m];
    b.tile0[m + 1] = b.tile0[m] + (int)dmm.ntiles;
  }
  for (int m = n; m < tq::kMaxBatch; ++m) b.tile0[m + 1] = b.tile0[n];
  if (workspace && !aligned(workspace, 16)) return TQ_ERR_ALIGN;
  return hip_status(tq::launch_gemv_pq2_fused_batch(b, dm, workspace, as_stream(stream)));
}

int tq_gemm(int fmt, const void* w, int64_t rows, int64_t cols, int64_t tokens, const int8_t* q, const float* d,
            const int16_t* bsums, float* y, void* workspace, void* stream) {
  const int st = product_args(fmt, w, rows, cols, tokens, q, d, bsums, y, true);
  if (st != TQ_OK) return st;
  if (workspace && !aligned(workspace, 16)) return TQ_ERR_ALIGN;
  // A single token takes the matrix-vector kernel (page 1, "the leftovers").
  if (tokens == 1) return tq_gemv(fmt, w, rows, cols, q, d, bsums, y, workspace, stream);
  const tq::Dims dm = tq::dims(rows, cols);
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  if (fmt == TQ_FMT_PTQ1_0)
    return hip_status(tq::launch_gemm_ptq1(wb, dm, tokens, q, d, bsums, y, nullptr, as_stream(stream)));
  return hip_status(tq::launch_gemm_pq2(wb, dm, tokens, q, d, y, nullptr, as_stream(stream)));
}

int tq_group_dots(int fmt, const void* w, int64_t rows, int64_t cols, int64_t tokens, const int8_t* q,
                  const int16_t* bsums, int32_t* idots, void* stream) {
  const int st = product_args(fmt, w, rows, cols, tokens, q, nullptr, bsums, idots, false);
  if (st != TQ_OK) return st;
  const tq::Dims dm = tq::dims(rows, cols);
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  if (tokens == 1) {
    if (fmt == TQ_FMT_PQ2_0)
      return hip_status(tq::launch_gemv_pq2(wb, dm, q, nullptr, nullptr, idots, nullptr, as_stream(stream)));
    return hip_status(tq::launch_gemv_ptq1(wb, dm, q, nullptr, bsums, nullptr, idots, nullptr, as_stream(stream)));
  }
  if (fmt == TQ_FMT_PTQ1_0)
    return hip_status(tq::launch_gemm_ptq1(wb, dm, tokens, q, nullptr, bsums, nullptr, idots, as_stream(stream)));
  return hip_status(tq::launch_gemm_pq2(wb, dm, tokens, q, nullptr, nullptr, idots, as_stream(stream)));
}

const char* tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_NULL: return "a required pointer is NULL";
    case TQ_ERR_SHAPE: return "unsupported shape (rows >= 1, cols a multiple of 256, tokens >= 1, size limits)";
    case TQ_ERR_ALIGN: return "misaligned pointer (weights and q: 16 bytes; x, d, y, idots: 4; bsums: 2)";
    case TQ_ERR_FORMAT: return "unknown weight format";
    case TQ_ERR_UNSUPPORTED: return "operation not provided for this format";
    case TQ_ERR_HIP: return "HIP runtime error (see tq_last_hip_error)";
    default: return "unknown status";
  }
}

int tq_last_hip_error(void) { return g_last_hip_error; }

int tq_version(void) { return 100; }

}  // extern "C"
