// api.hip -- the extern "C" entry points of libbrq (declared in
// include/brq.h): argument checks on the host, workspace carving, and the
// kernel launches on the caller's stream.  No device memory is allocated
// here; nothing synchronises.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "internal.hpp"

using namespace brq;

namespace {

thread_local int g_last_hip = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return BRQ_OK;
  g_last_hip = (int)e;
  return BRQ_E_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool fp_dtype(int d) { return d == BRQ_F32 || d == BRQ_BF16; }
int vec_elems(int d) { return d == BRQ_BF16 ? 8 : 4; }
hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// Fixed scratch block at the end of several workspaces: sum, max, s, r.
constexpr size_t kScalars = 256;

size_t quant_ws(int64_t rows, int64_t cols, const brq_tune* t) {
  return flat_reduce_ws(rows * cols, flat_chunk_log2(t)) + kScalars;
}

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// rotated input-gradient GEMM: q_h^T [K][N], q_g [M][N], scalars, then the
// larger of the two rotation stages' scratch, then the GEMM's
size_t dx_wht_stage_ws(int64_t M, int64_t N, int64_t K, int block) {
  size_t a = wht_x_ws(N, K, block), b = wht_rows_ws(M, N);
  return a > b ? a : b;
}
size_t dx_wht_ws(int64_t M, int64_t N, int64_t K, int block, const brq_tune* t) {
  return align256((size_t)(K * N)) + align256((size_t)(M * N)) + kScalars +
         dx_wht_stage_ws(M, N, K, block) + gemm_ws(M, K, N, t);
}

int check_dx_wht_shape(int64_t M, int64_t N, int64_t K, int block) {
  if (M < 0 || N < 0 || K < 0) return BRQ_E_SHAPE;
  if (!pow2(block) || block > 128) return BRQ_E_UNSUPPORTED;
  if (N == 0 || M % 16 || N % 64 || N % block || K % 64) return BRQ_E_UNSUPPORTED;
  if (N > BRQ_MAX_CONTRACTION) return BRQ_E_RANGE;
  return BRQ_OK;
}

size_t quant_exact_ws(int64_t rows, int64_t cols) {
  return exact_reduce_ws(rows * cols) + kScalars;
}

size_t dw_stage_ws(int64_t M, int64_t N, int64_t K, int block, const brq_tune* t) {
  size_t a = wht_x_ws(M, K, block), b = wht_dy_ws(M, N, block, flat_chunk_log2(t));
  return a > b ? a : b;
}

size_t dw_ws(int64_t M, int64_t N, int64_t K, int block, const brq_tune* t) {
  return align256((size_t)(K * M)) + align256((size_t)(N * M)) + kScalars +
         dw_stage_ws(M, N, K, block, t) + gemm_ws(N, K, M, t);
}

size_t dy_bwd_ws(int64_t M, int64_t N, int block, const brq_tune* t) {
  const int c = flat_chunk_log2(t);
  size_t a = dy_fused_ws(M, N, c), b = quant_ws(M, N, t), d = wht_dy_ws(M, N, block, c);
  return std::max(a, std::max(b, d));
}

int check_dw_shape(int64_t M, int64_t N, int64_t K, int block) {
  if (M < 0 || N < 0 || K < 0) return BRQ_E_SHAPE;
  if (!pow2(block) || block > 128) return BRQ_E_UNSUPPORTED;
  if (M % block || M % 64 || K % 64 || N % 64) return BRQ_E_UNSUPPORTED;
  if (M > BRQ_MAX_CONTRACTION) return BRQ_E_RANGE;
  return BRQ_OK;
}

}  // namespace

extern "C" {

int brq_spec_version(void) { return BRQ_SPEC_VERSION; }
int brq_last_hip_error(void) { return g_last_hip; }

const char* brq_status_string(int s) {
  switch (s) {
    case BRQ_OK: return "ok";
    case BRQ_E_NULL: return "required pointer is NULL";
    case BRQ_E_DTYPE: return "unsupported dtype";
    case BRQ_E_SHAPE: return "invalid shape";
    case BRQ_E_ALIGN: return "pointer not 16-byte aligned";
    case BRQ_E_UNSUPPORTED: return "shape outside the supported set";
    case BRQ_E_RANGE: return "contraction too long for exact int32 accumulation";
    case BRQ_E_WORKSPACE: return "workspace missing or too small";
    case BRQ_E_HIP: return "HIP launch error";
    case BRQ_E_ARG: return "invalid argument";
    case BRQ_E_SCRATCH: return "input too large for the library's static scratch buffer";
    default: return "unknown status";
  }
}

size_t brq_workspace_size(int op, int64_t a, int64_t b, int64_t c, int block, const brq_tune* t) {
  if (a < 0 || b < 0 || c < 0) return 0;
  switch (op) {
    case BRQ_OP_QUANTIZE: return quant_ws(a, b, t);
    case BRQ_OP_QUANTIZE_EXACT: return quant_exact_ws(a, b);
    case BRQ_OP_DX_WHT: return dx_wht_ws(a, b, c, block > 0 ? block : 1, t);
    case BRQ_OP_DY_ROWS_WHT: return wht_rows_ws(a, b) + kScalars;
    case BRQ_OP_QGEMM: return gemm_ws(a, b, c, t);
    case BRQ_OP_DW_WHT: return dw_ws(a, b, c, block > 0 ? block : 1, t);
    case BRQ_OP_RMSNORM_BWD: {
      size_t x = rmsnorm_bwd_ws(a, b, BRQ_BF16, t), y = rmsnorm_bwd_ws(a, b, BRQ_F32, t);
      return x > y ? x : y;
    }
    case BRQ_OP_GRAD_NORM: return kScalars + flat_reduce_ws(a, flat_chunk_log2(t));
    case BRQ_OP_DY_BWD: return dy_bwd_ws(a, b, block > 0 ? block : 1, t);
    case BRQ_OP_QUANTIZE_X_WHT:
      return quant_x_wht_ws(a, b, block > 0 ? block : 1, flat_chunk_log2(t));
    default: return 0;
  }
}

}  // extern "C"

namespace {

int quantize_common(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                    const float* col_mul, bool exact, int8_t* q, int8_t* q_t, float* scale,
                    float* amax, void* ws, size_t ws_bytes, int32_t* dflags,
                    const brq_tune* tune, void* stream) {
  if (!fp_dtype(x_dtype)) return BRQ_E_DTYPE;
  if (rows < 0 || cols < 0) return BRQ_E_SHAPE;
  if (gran != BRQ_PER_TENSOR && gran != BRQ_PER_ROW) return BRQ_E_ARG;
  const int64_t n = rows * cols;
  if (!scale || (n > 0 && (!x || !q))) return BRQ_E_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(q_t) || !aligned16(col_mul)) return BRQ_E_ALIGN;
  if (cols % vec_elems(x_dtype)) return BRQ_E_UNSUPPORTED;
  if (q_t && (rows % 16 || cols % 16)) return BRQ_E_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  hipError_t e;
  if (gran == BRQ_PER_ROW) {
    if (col_mul) return BRQ_E_UNSUPPORTED;
    if (cols > 16384 || cols == 0) return BRQ_E_UNSUPPORTED;
    if (rows == 0) return BRQ_OK;
    e = exact ? quant_rows_exact(x, x_dtype, rows, cols, q, scale, amax, dflags, s)
              : quant_rows(x, x_dtype, rows, cols, q, scale, amax, dflags, s);
    if (e != hipSuccess) return hip_status(e);
  } else {
    const size_t need = exact ? quant_exact_ws(rows, cols) : quant_ws(rows, cols, tune);
    if (!ws || ws_bytes < need) return BRQ_E_WORKSPACE;
    float* sc = (float*)((char*)ws + need - kScalars);  // [0]sum [1]max [2]s [3]r
    // an empty group has step size 0 (no mean is taken)
    const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;
    if (exact) {
      e = exact_reduce(x, x_dtype, col_mul, n, cols > 0 ? cols : 1, sc, ws, dflags, s);
      if (e != hipSuccess) return hip_status(e);
      if ((e = lsq_finalize(sc, inv_n, sc + 2, scale, amax, s)) != hipSuccess) return hip_status(e);
    } else {
      // the step size is computed by the reduction's final work-group
      const int leaf = col_mul ? LEAF_ABS_COLMUL : LEAF_ABS;
      const FlatFin fin{FIN_LSQ, inv_n, sc + 2, scale, amax, nullptr, nullptr};
      e = flat_reduce(x, x_dtype, leaf, col_mul, n, cols > 0 ? cols : 1, sc, ws,
                      flat_chunk_log2(tune), dflags, s, 0, &fin);
      if (e != hipSuccess) return hip_status(e);
    }
    if (n > 0 && (e = quant_flat(x, x_dtype, col_mul, n, cols, sc + 2, q, s)) != hipSuccess)
      return hip_status(e);
  }
  if (q_t && n > 0 && (e = transpose_i8(q, rows, cols, q_t, s)) != hipSuccess) return hip_status(e);
  return BRQ_OK;
}

}  // namespace

extern "C" {

int brq_quantize_lsq(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                     const float* col_mul, int8_t* q, int8_t* q_t, float* scale, float* amax,
                     void* ws, size_t ws_bytes, int32_t* dflags, const brq_tune* tune,
                     void* stream) {
  return quantize_common(x, x_dtype, rows, cols, gran, col_mul, false, q, q_t, scale, amax, ws,
                         ws_bytes, dflags, tune, stream);
}

int brq_quantize_lsq_rows_multi(const brq_rows_job* jobs, int count, int32_t* dflags,
                                void* stream) {
  if (count < 0 || count > BRQ_ROWS_MULTI_MAX) return BRQ_E_ARG;
  if (count == 0) return BRQ_OK;
  if (!jobs) return BRQ_E_NULL;
  // every job is checked before anything is launched (the per-row rules
  // of quantize_common)
  for (int c = 0; c < count; ++c) {
    const brq_rows_job& j = jobs[c];
    if (!fp_dtype(j.x_dtype)) return BRQ_E_DTYPE;
    if (j.rows < 0 || j.cols < 0) return BRQ_E_SHAPE;
    if ((j.rows > 0 && !j.scale) || (j.rows * j.cols > 0 && (!j.x || !j.q))) return BRQ_E_NULL;
    if (!aligned16(j.x) || !aligned16(j.q) || !aligned16(j.q_t)) return BRQ_E_ALIGN;
    if (j.cols % vec_elems(j.x_dtype)) return BRQ_E_UNSUPPORTED;
    if (j.q_t && (j.rows % 16 || j.cols % 16)) return BRQ_E_UNSUPPORTED;
    if (j.cols > 16384 || j.cols == 0) return BRQ_E_UNSUPPORTED;
  }
  return hip_status(quant_rows_multi(jobs, count, dflags, as_stream(stream)));
}

}  // extern "C"

// ---- the allocation-free variant's scratch ---------------------------------------
// One static device array per GPU the library runs on (it stays until the
// process ends).  In host code `scratch` names a host-side stand-in, not a
// device address: the device address comes from hipGetSymbolAddress, looked
// up once per device with that device current, and only that address is
// ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[BRQ_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first
// call on that device).
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return BRQ_E_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return BRQ_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BRQ_OK;
}

}  // namespace

extern "C" {

int brq_quantize_lsq_static(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                            const float* col_mul, int8_t* q, int8_t* q_t, float* scale,
                            float* amax, int32_t* dflags, const brq_tune* tune, void* stream) {
  // size check first: nothing is looked up or launched for an input the
  // scratch cannot hold
  if (rows < 0 || cols < 0) return BRQ_E_SHAPE;
  if (gran == BRQ_PER_TENSOR &&
      quant_ws(rows, cols, tune) > (size_t)BRQ_STATIC_SCRATCH_BYTES)
    return BRQ_E_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_of_current_device(&ws);
  if (st != BRQ_OK) return st;
  return quantize_common(x, x_dtype, rows, cols, gran, col_mul, false, q, q_t, scale, amax, ws,
                         BRQ_STATIC_SCRATCH_BYTES, dflags, tune, stream);
}

int brq_quantize_lsq_exact(const void* x, int x_dtype, int64_t rows, int64_t cols, int gran,
                           const float* col_mul, int8_t* q, int8_t* q_t, float* scale,
                           float* amax, void* ws, size_t ws_bytes, int32_t* dflags,
                           const brq_tune* tune, void* stream) {
  return quantize_common(x, x_dtype, rows, cols, gran, col_mul, true, q, q_t, scale, amax, ws,
                         ws_bytes, dflags, tune, stream);
}

static int gemm_common(const int8_t* A, const int8_t* B, int64_t I, int64_t J, int64_t Kc,
                       float* C, const EpiArgs& epi, void* ws, size_t ws_bytes,
                       const brq_tune* tune, void* stream) {
  if (I < 0 || J < 0 || Kc < 0) return BRQ_E_SHAPE;
  if (Kc % 16) return BRQ_E_UNSUPPORTED;
  if (Kc > BRQ_MAX_CONTRACTION) return BRQ_E_RANGE;
  if (I > 0 && J > 0 && (!C || (Kc > 0 && (!A || !B)))) return BRQ_E_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return BRQ_E_ALIGN;
  if (ws_bytes < gemm_ws(I, J, Kc, tune) || (gemm_ws(I, J, Kc, tune) && !ws))
    return BRQ_E_WORKSPACE;
  return hip_status(gemm_i8(A, B, I, J, Kc, C, epi, ws, ws_bytes, tune, as_stream(stream)));
}

int brq_qgemm_fwd(const int8_t* q_x, const float* s_x, const int8_t* q_w, const float* s_w,
                  int w_per_row, int64_t M, int64_t N, int64_t K, float* y, void* ws,
                  size_t ws_bytes, const brq_tune* tune, void* stream) {
  if (!s_x || !s_w) return BRQ_E_NULL;
  EpiArgs epi{EPI_FWD, s_x, s_w, nullptr, w_per_row ? 1 : 0, 1.0f};
  return gemm_common(q_x, q_w, M, N, K, y, epi, ws, ws_bytes, tune, stream);
}

int brq_qgemm_bwd_dx(const int8_t* q_g, const float* s_g, const int8_t* q_wt, int64_t M,
                     int64_t N, int64_t K, float* dx, void* ws, size_t ws_bytes,
                     const brq_tune* tune, void* stream) {
  if (!s_g) return BRQ_E_NULL;
  EpiArgs epi{EPI_SCALAR, s_g, nullptr, nullptr, 0, 1.0f};
  return gemm_common(q_g, q_wt, M, K, N, dx, epi, ws, ws_bytes, tune, stream);
}

int brq_qgemm_fwd_ex(const int8_t* q_x, const float* s_x, const int8_t* q_w, const float* s_w,
                     int w_per_row, int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                     void* ws, size_t ws_bytes, const brq_tune* tune, void* stream) {
  if (!s_x || !s_w) return BRQ_E_NULL;
  if (!fp_dtype(y_dtype)) return BRQ_E_DTYPE;
  EpiArgs epi{EPI_FWD, s_x, s_w, nullptr, w_per_row ? 1 : 0, 1.0f, y_dtype == BRQ_BF16};
  return gemm_common(q_x, q_w, M, N, K, (float*)y, epi, ws, ws_bytes, tune, stream);
}

int brq_qgemm_bwd_dx_ex(const int8_t* q_g, const float* s_g, const int8_t* q_wt, int64_t M,
                        int64_t N, int64_t K, void* dx, int dx_dtype, void* ws, size_t ws_bytes,
                        const brq_tune* tune, void* stream) {
  if (!s_g) return BRQ_E_NULL;
  if (!fp_dtype(dx_dtype)) return BRQ_E_DTYPE;
  EpiArgs epi{EPI_SCALAR, s_g, nullptr, nullptr, 0, 1.0f, dx_dtype == BRQ_BF16};
  return gemm_common(q_g, q_wt, M, K, N, (float*)dx, epi, ws, ws_bytes, tune, stream);
}

int brq_qgemm_dw(const int8_t* q_vt, const int8_t* q_ut, const float* s_x, const float* s_u,
                 const float* s_v, int64_t M, int64_t N, int64_t K, int block, float* dw,
                 void* ws, size_t ws_bytes, const brq_tune* tune, void* stream) {
  if (!s_x || !s_u || !s_v) return BRQ_E_NULL;
  if (!pow2(block) || block > 128) return BRQ_E_UNSUPPORTED;
  int lb = 0;
  while ((1 << lb) < block) ++lb;
  EpiArgs epi{EPI_DW, s_x, s_u, s_v, 0, ldexpf(1.0f, -lb)};
  return gemm_common(q_vt, q_ut, N, K, M, dw, epi, ws, ws_bytes, tune, stream);
}

int brq_wht_quant_x(const int8_t* q_x, int64_t M, int64_t K, int block, int8_t* q_ut, float* s_u,
                    void* ws, size_t ws_bytes, const brq_tune* tune, void* stream) {
  (void)tune;
  int st = check_dw_shape(M, 64, K, block);
  if (st != BRQ_OK) return st;
  if (!s_u || (M * K > 0 && (!q_x || !q_ut))) return BRQ_E_NULL;
  if (!aligned16(q_x) || !aligned16(q_ut)) return BRQ_E_ALIGN;
  if (!ws || ws_bytes < wht_x_ws(M, K, block)) return BRQ_E_WORKSPACE;
  return hip_status(wht_quant_x(q_x, M, K, block, q_ut, s_u, ws, as_stream(stream)));
}

int brq_quantize_x_wht(const void* x, int x_dtype, int64_t M, int64_t K, int block, int8_t* q_x,
                       float* s_x, float* amax_x, int8_t* q_ut, float* s_u, void* ws,
                       size_t ws_bytes, int32_t* dflags, const brq_tune* tune, void* stream) {
  if (!fp_dtype(x_dtype)) return BRQ_E_DTYPE;
  int st = check_dw_shape(M, 64, K, block);
  if (st != BRQ_OK) return st;
  if (!s_x || !s_u || (M * K > 0 && (!x || !q_x || !q_ut))) return BRQ_E_NULL;
  if (!aligned16(x) || !aligned16(q_x) || !aligned16(q_ut)) return BRQ_E_ALIGN;
  const int c = flat_chunk_log2(tune);
  if (!ws || ws_bytes < quant_x_wht_ws(M, K, block, c)) return BRQ_E_WORKSPACE;
  return hip_status(quantize_x_wht(x, x_dtype, M, K, block, q_x, s_x, amax_x, q_ut, s_u, ws, c,
                                   dflags, as_stream(stream)));
}

int brq_wht_quant_dy(const void* dy, int dy_dtype, int64_t M, int64_t N, int block, int8_t* q_vt,
                     float* s_v, void* ws, size_t ws_bytes, int32_t* dflags,
                     const brq_tune* tune, void* stream) {
  if (!fp_dtype(dy_dtype)) return BRQ_E_DTYPE;
  int st = check_dw_shape(M, N, 64, block);
  if (st != BRQ_OK) return st;
  if (!s_v || (M * N > 0 && (!dy || !q_vt))) return BRQ_E_NULL;
  if (!aligned16(dy) || !aligned16(q_vt)) return BRQ_E_ALIGN;
  const int c = flat_chunk_log2(tune);
  if (!ws || ws_bytes < wht_dy_ws(M, N, block, c)) return BRQ_E_WORKSPACE;
  return hip_status(wht_quant_dy(dy, dy_dtype, M, N, block, q_vt, s_v, ws, c, dflags,
                                 as_stream(stream)));
}

int brq_qgemm_bwd_dw_wht(const int8_t* q_x, const float* s_x, const void* dy, int dy_dtype,
                         int64_t M, int64_t N, int64_t K, int block, float* dw, float* s_u_out,
                         float* s_v_out, void* ws, size_t ws_bytes, int32_t* dflags,
                         const brq_tune* tune, void* stream) {
  if (!fp_dtype(dy_dtype)) return BRQ_E_DTYPE;
  int st = check_dw_shape(M, N, K, block);
  if (st != BRQ_OK) return st;
  if (!s_x) return BRQ_E_NULL;
  const size_t need = dw_ws(M, N, K, block, tune);
  if (!ws || ws_bytes < need) return BRQ_E_WORKSPACE;
  char* w = (char*)ws;
  int8_t* q_ut = (int8_t*)w;
  w += align256((size_t)(K * M));
  int8_t* q_vt = (int8_t*)w;
  w += align256((size_t)(N * M));
  float* scal = (float*)w;
  w += kScalars;
  void* stage = w;
  w += dw_stage_ws(M, N, K, block, tune);
  void* gws = w;
  float* s_u = s_u_out ? s_u_out : scal;
  float* s_v = s_v_out ? s_v_out : scal + 1;
  const size_t stage_bytes = dw_stage_ws(M, N, K, block, tune);
  int r = brq_wht_quant_x(q_x, M, K, block, q_ut, s_u, stage, stage_bytes, tune, stream);
  if (r != BRQ_OK) return r;
  r = brq_wht_quant_dy(dy, dy_dtype, M, N, block, q_vt, s_v, stage, stage_bytes, dflags, tune,
                       stream);
  if (r != BRQ_OK) return r;
  return brq_qgemm_dw(q_vt, q_ut, s_x, s_u, s_v, M, N, K, block, dw, gws, gemm_ws(N, K, M, tune),
                      tune, stream);
}

int brq_attn_fwd(const void* q, const void* k, const void* v, int64_t Hq, int64_t Hkv, int64_t T,
                 int64_t d, int64_t window, float* o, int32_t* dflags, const brq_tune* tune,
                 void* stream) {
  (void)tune;
  if (Hq < 0 || Hkv <= 0 || T < 0 || window < 1) return BRQ_E_SHAPE;
  if (Hq % Hkv || T % 64 || (d != 64 && d != 128)) return BRQ_E_UNSUPPORTED;
  if (Hq * T > 0 && (!q || !k || !v || !o)) return BRQ_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return BRQ_E_ALIGN;
  if (Hq == 0 || T == 0) return BRQ_OK;
  if (T / 64 > 65535) return BRQ_E_UNSUPPORTED;
  return hip_status(attn_fwd((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, Hq, Hkv,
                             T, d, window, o, dflags, as_stream(stream)));
}

int brq_wht_quant_dy_rows(const void* dy, int dy_dtype, int64_t M, int64_t N, const float* s_w,
                          int block, int8_t* q_g, float* s_g, void* ws, size_t ws_bytes,
                          int32_t* dflags, const brq_tune* tune, void* stream) {
  (void)tune;
  if (!fp_dtype(dy_dtype)) return BRQ_E_DTYPE;
  int st = check_dx_wht_shape(M, N, 64, block);
  if (st != BRQ_OK) return st;
  if (!s_g || (M * N > 0 && (!dy || !s_w || !q_g))) return BRQ_E_NULL;
  if (!aligned16(dy) || !aligned16(q_g) || !aligned16(s_w)) return BRQ_E_ALIGN;
  const size_t need = wht_rows_ws(M, N) + kScalars;
  if (!ws || ws_bytes < need) return BRQ_E_WORKSPACE;
  float* sr = (float*)((char*)ws + wht_rows_ws(M, N));
  return hip_status(wht_rows_quant(dy, dy_dtype, M, N, s_w, block, q_g, s_g, sr, ws, dflags,
                                   as_stream(stream)));
}

int brq_qgemm_bwd_dx_wht(const void* dy, int dy_dtype, const float* s_w, const int8_t* q_w,
                         int64_t M, int64_t N, int64_t K, int block, float* dx, float* s_g_out,
                         float* s_h_out, void* ws, size_t ws_bytes, int32_t* dflags,
                         const brq_tune* tune, void* stream) {
  if (!fp_dtype(dy_dtype)) return BRQ_E_DTYPE;
  int st = check_dx_wht_shape(M, N, K, block);
  if (st != BRQ_OK) return st;
  if (M * N > 0 && (!dy || !s_w)) return BRQ_E_NULL;
  if (N * K > 0 && !q_w) return BRQ_E_NULL;
  if (M * K > 0 && !dx) return BRQ_E_NULL;
  if (!aligned16(dy) || !aligned16(q_w) || !aligned16(dx) || !aligned16(s_w)) return BRQ_E_ALIGN;
  if (M == 0 || K == 0) return BRQ_OK;  // dx is empty: nothing is computed
  const size_t need = dx_wht_ws(M, N, K, block, tune);
  if (!ws || ws_bytes < need) return BRQ_E_WORKSPACE;
  char* w = (char*)ws;
  int8_t* q_ht = (int8_t*)w;
  w += align256((size_t)(K * N));
  int8_t* q_g = (int8_t*)w;
  w += align256((size_t)(M * N));
  float* scal = (float*)w;  // [0] s_g [1] r_g [2] 1 [3] s_h (when s_h_out is NULL)
  w += kScalars;
  void* stage = w;
  w += dx_wht_stage_ws(M, N, K, block);
  void* gws = w;
  hipStream_t s = as_stream(stream);
  hipError_t e;
  float* s_h = s_h_out ? s_h_out : scal + 3;
  if ((e = wht_quant_x(q_w, N, K, block, q_ht, s_h, stage, s)) != hipSuccess) return hip_status(e);
  if ((e = wht_rows_quant(dy, dy_dtype, M, N, s_w, block, q_g, s_g_out, scal, stage, dflags, s)) !=
      hipSuccess)
    return hip_status(e);
  int lb = 0;
  while ((1 << lb) < block) ++lb;
  // c = fl(fl(fl(s_g * s_h) * 1) * 2^-lb)
  EpiArgs epi{EPI_DW, scal, s_h, scal + 2, 0, ldexpf(1.0f, -lb)};
  return hip_status(gemm_i8(q_g, q_ht, M, K, N, dx, epi, gws, gemm_ws(M, K, N, tune), tune, s));
}

int brq_quantize_dy_bwd(const void* dy, int dy_dtype, int64_t M, int64_t N, const float* s_w,
                        int block, int8_t* q_g, float* s_g, float* amax_g, int8_t* q_vt,
                        float* s_v, void* ws, size_t ws_bytes, int32_t* dflags,
                        const brq_tune* tune, void* stream) {
  if (!fp_dtype(dy_dtype)) return BRQ_E_DTYPE;
  int st = check_dw_shape(M, N, 64, block);
  if (st != BRQ_OK) return st;
  if (!s_g || !s_v || (M * N > 0 && (!dy || !s_w || !q_g || !q_vt))) return BRQ_E_NULL;
  if (!aligned16(dy) || !aligned16(q_g) || !aligned16(q_vt) || !aligned16(s_w)) return BRQ_E_ALIGN;
  if (!ws || ws_bytes < dy_bwd_ws(M, N, block, tune)) return BRQ_E_WORKSPACE;
  hipStream_t s = as_stream(stream);
  if (M * N > 0 && dy_fused_ok(dy_dtype, M, N, block))
    return hip_status(quantize_dy_fused(dy, M, N, s_w, block, q_g, s_g, amax_g, q_vt, s_v, ws,
                                        flat_chunk_log2(tune), dflags, s));
  // other shapes: the two definitions one after the other
  int r = brq_quantize_lsq(dy, dy_dtype, M, N, BRQ_PER_TENSOR, s_w, q_g, nullptr, s_g, amax_g, ws,
                           ws_bytes, dflags, tune, stream);
  if (r != BRQ_OK) return r;
  return brq_wht_quant_dy(dy, dy_dtype, M, N, block, q_vt, s_v, ws, ws_bytes, dflags, tune,
                          stream);
}

int brq_rmsnorm_fixed_fwd(const void* x, const void* g, int dtype, int64_t T, int64_t D, float eps,
                          void* y, float* rstd, int32_t* dflags, const brq_tune* tune,
                          void* stream) {
  (void)tune;
  if (!fp_dtype(dtype)) return BRQ_E_DTYPE;
  if (T < 0 || D <= 0) return BRQ_E_SHAPE;
  if (D % 8 || D > 64 * vec_elems(dtype) * 32) return BRQ_E_UNSUPPORTED;
  if (T > 0 && (!x || !g || !y || !rstd)) return BRQ_E_NULL;
  if (!aligned16(x) || !aligned16(g) || !aligned16(y)) return BRQ_E_ALIGN;
  if (T == 0) return BRQ_OK;
  return hip_status(rmsnorm_fwd(x, g, dtype, T, D, eps, y, rstd, dflags, as_stream(stream)));
}

int brq_rmsnorm_fixed_bwd(const void* x, const void* g, const float* rstd, const void* dy,
                          int dtype, int64_t T, int64_t D, void* dx, float* dg, void* ws,
                          size_t ws_bytes, const brq_tune* tune, void* stream) {
  if (!fp_dtype(dtype)) return BRQ_E_DTYPE;
  if (T < 0 || D <= 0) return BRQ_E_SHAPE;
  if (D % 8 || D > 256 * vec_elems(dtype) * 2) return BRQ_E_UNSUPPORTED;
  if (!dg || (T > 0 && (!x || !g || !rstd || !dy || !dx))) return BRQ_E_NULL;
  if (!aligned16(x) || !aligned16(g) || !aligned16(dy) || !aligned16(dx) || !aligned16(dg))
    return BRQ_E_ALIGN;
  if (!ws || ws_bytes < rmsnorm_bwd_ws(T, D, dtype, tune)) return BRQ_E_WORKSPACE;
  return hip_status(rmsnorm_bwd(x, g, rstd, dy, dtype, T, D, dx, dg, ws, tune, as_stream(stream)));
}

int brq_grad_norm(const float* v, int64_t n, float* sumsq, float* norm, void* ws, size_t ws_bytes,
                  int32_t* dflags, const brq_tune* tune, void* stream) {
  if (n < 0) return BRQ_E_SHAPE;
  if (!sumsq || !norm || (n > 0 && !v)) return BRQ_E_NULL;
  if (!aligned16(v)) return BRQ_E_ALIGN;
  const int c = flat_chunk_log2(tune);
  if (!ws || ws_bytes < kScalars + flat_reduce_ws(n, c)) return BRQ_E_WORKSPACE;
  return hip_status(grad_norm(v, n, sumsq, norm, ws, c, dflags, as_stream(stream)));
}

int brq_adamw_bias_corrections(int64_t t, float beta1, float beta2, float* bc1, float* bc2) {
  if (t < 1 || !bc1 || !bc2) return BRQ_E_ARG;
  // host binary32 arithmetic (no contraction); a subnormal product is
  // flushed to zero, after which the power stays zero
  auto flush_h = [](float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0u) u &= 0x80000000u;
    memcpy(&f, &u, 4);
    return f;
  };
  float p1 = 1.0f, p2 = 1.0f;
  for (int64_t i = 0; i < t; ++i) {
    if (p1 == 0.0f && p2 == 0.0f) break;
    p1 = flush_h(p1 * beta1);
    p2 = flush_h(p2 * beta2);
  }
  *bc1 = flush_h(1.0f - p1);
  *bc2 = flush_h(1.0f - p2);
  return BRQ_OK;
}

int brq_adamw_decide(const float* norm, float max_norm, float spike_threshold, int skip_steps,
                     int32_t* skip_state, float* ctl, int32_t* dflags, void* stream) {
  if (!norm || !skip_state || !ctl) return BRQ_E_NULL;
  if (skip_steps < 0) return BRQ_E_ARG;
  return hip_status(adamw_decide(norm, max_norm, spike_threshold, skip_steps, skip_state, ctl,
                                 dflags, as_stream(stream)));
}

int brq_adamw_step(void* param, int param_dtype, const void* grad, int grad_dtype, float* m,
                   float* v, int64_t n, const brq_adamw_hparams* hp, const float* ctl,
                   void* stream) {
  if (n < 0) return BRQ_E_SHAPE;
  if (!fp_dtype(param_dtype) || !fp_dtype(grad_dtype)) return BRQ_E_DTYPE;
  if (!hp || !ctl || (n > 0 && (!param || !grad || !m || !v))) return BRQ_E_NULL;
  if (!aligned16(param) || !aligned16(grad) || !aligned16(m) || !aligned16(v))
    return BRQ_E_ALIGN;
  return hip_status(
      adamw_step(param, param_dtype, grad, grad_dtype, m, v, n, *hp, ctl, as_stream(stream)));
}

int brq_dp_reduce(const float* const* parts, int replicas, int shards, int accum, int64_t n,
                  int average, float* out, int32_t* dflags, void* stream) {
  if (n < 0) return BRQ_E_SHAPE;
  if (replicas < 1 || shards < 1 || accum < 1) return BRQ_E_ARG;
  if ((int64_t)replicas * shards * accum > BRQ_DP_MAX_PARTS) return BRQ_E_UNSUPPORTED;
  if (!parts) return BRQ_E_NULL;
  const int P = replicas * shards * accum;
  if (n > 0) {
    if (!out) return BRQ_E_NULL;
    for (int j = 0; j < P; ++j)
      if (!parts[j]) return BRQ_E_NULL;
  }
  if (!aligned16(out)) return BRQ_E_ALIGN;
  for (int j = 0; j < P; ++j)
    if (!aligned16(parts[j])) return BRQ_E_ALIGN;
  return hip_status(
      dp_reduce(parts, replicas, shards, accum, n, average, out, dflags, as_stream(stream)));
}

int brq_fp32_primitive(int prim, uint32_t first, int64_t count, uint32_t* out, void* stream) {
  if (prim < BRQ_PRIM_SQRT || prim > BRQ_PRIM_BF16_INT) return BRQ_E_ARG;
  if (count < 0 || count > ((int64_t)1 << 32)) return BRQ_E_SHAPE;
  if (count > 0 && !out) return BRQ_E_NULL;
  if (!aligned16(out)) return BRQ_E_ALIGN;
  return hip_status(fp32_primitive(prim, first, count, out, as_stream(stream)));
}

size_t brq_hash_workspace_size(const brq_tensor_ref* t, int n) {
  if (n < 0 || (n > 0 && !t)) return 0;
  return hash_ws(t, n);
}

static int check_refs(const brq_tensor_ref* t, int n) {
  if (n < 0) return BRQ_E_SHAPE;
  if (n > 0 && !t) return BRQ_E_NULL;
  for (int i = 0; i < n; ++i) {
    if (t[i].dtype < BRQ_F32 || t[i].dtype > BRQ_U8) return BRQ_E_DTYPE;
    if (t[i].ndim < 0 || t[i].ndim > 8) return BRQ_E_SHAPE;
    int64_t cnt = 1;
    for (int d = 0; d < t[i].ndim; ++d) {
      if (t[i].dims[d] < 0) return BRQ_E_SHAPE;
      cnt *= t[i].dims[d];
    }
    if (cnt > 0 && !t[i].data) return BRQ_E_NULL;
    if (!aligned16(t[i].data)) return BRQ_E_ALIGN;
    if (t[i].name && strlen(t[i].name) > 255) return BRQ_E_ARG;
  }
  return BRQ_OK;
}

int brq_hash_state(const brq_tensor_ref* t, int n, uint8_t* digest32, void* ws, size_t ws_bytes,
                   void* stream) {
  int st = check_refs(t, n);
  if (st != BRQ_OK) return st;
  if (!digest32) return BRQ_E_NULL;
  if (!aligned16(digest32)) return BRQ_E_ALIGN;
  if (!ws || ws_bytes < hash_ws(t, n)) return BRQ_E_WORKSPACE;
  return hip_status(hash_state(t, n, digest32, ws, as_stream(stream)));
}

size_t brq_hash_digests_workspace_size(const brq_tensor_ref* t, int n) {
  if (n < 0 || (n > 0 && !t)) return 0;
  return hash_digests_ws(t, n);
}

int brq_hash_tensor_digests(const brq_tensor_ref* t, int n, uint8_t* digests, void* ws,
                            size_t ws_bytes, void* stream) {
  int st = check_refs(t, n);
  if (st != BRQ_OK) return st;
  if (n > 0 && !digests) return BRQ_E_NULL;
  if (!aligned16(digests)) return BRQ_E_ALIGN;
  if (!ws || ws_bytes < hash_digests_ws(t, n)) return BRQ_E_WORKSPACE;
  return hip_status(hash_tensor_digests(t, n, digests, ws, as_stream(stream)));
}

int brq_hash_tensor_leaves(const brq_tensor_ref* t, int n, void* ws, size_t ws_bytes,
                           void* stream) {
  int st = check_refs(t, n);
  if (st != BRQ_OK) return st;
  if (!ws || ws_bytes < hash_digests_ws(t, n)) return BRQ_E_WORKSPACE;
  return hip_status(hash_tensor_leaves(t, n, ws, as_stream(stream)));
}

int brq_hash_tensor_finish(const brq_tensor_ref* t, int n, uint8_t* digests, void* ws,
                           size_t ws_bytes, void* stream) {
  int st = check_refs(t, n);
  if (st != BRQ_OK) return st;
  if (n > 0 && !digests) return BRQ_E_NULL;
  if (!aligned16(digests)) return BRQ_E_ALIGN;
  if (!ws || ws_bytes < hash_digests_ws(t, n)) return BRQ_E_WORKSPACE;
  return hip_status(hash_tensor_finish(t, n, digests, ws, as_stream(stream)));
}

int brq_hash_combine(const uint8_t* digests, int n, uint8_t* digest32, void* stream) {
  if (n < 0) return BRQ_E_SHAPE;
  if (!digest32 || (n > 0 && !digests)) return BRQ_E_NULL;
  if (!aligned16(digests) || !aligned16(digest32)) return BRQ_E_ALIGN;
  return hip_status(hash_combine(digests, n, digest32, as_stream(stream)));
}

}  // extern "C"
