// Plain projections around the attention hot path, on hipBLASLt: the linear maps
// that feed it and the grouped output projection of "CSA And HCA: Definition,
// State, And Cost Model" section 5.4,
//   o_hat_t = W^{O,B} [ W^{O,A}_1 o^G_{t,1}; ... ; W^{O,A}_g o^G_{t,g} ],
// where o^G_{t,i} concatenates the c-wide outputs of the n_h/g heads of group i.
// The g group products are one strided-batched GEMM reading the attention output
// in place (group i is a column block of the [T][n_h c] output rows), the final
// map one more GEMM.  bf16 operands, float32 accumulation; the intermediate
// [T][g d_g] is rounded to bf16 like any other layer activation.
//
// Row-major Y[T][N] = X[T][K] W[N][K]^T is, in hipBLASLt's column-major terms,
// D = A^T B with A = W (K x N, ld K), B = X (K x T, ld K), D = Y (N x T, ld N).
#include "../../include/v4a.h"

#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "internal.h"

namespace {

constexpr size_t kBlasWs = 32u << 20;  // hipBLASLt workspace carved from the caller's
constexpr int kMaxDevices = 64;

std::mutex g_mu;
hipblasLtHandle_t g_handle[kMaxDevices] = {};

struct GemmKey {
  int dev, M, N, K, batch, out_dt;
  int64_t ldx, sx, sw, ldy, sy;
  bool operator<(const GemmKey& o) const {
    return std::tie(dev, M, N, K, batch, out_dt, ldx, sx, sw, ldy, sy) <
           std::tie(o.dev, o.M, o.N, o.K, o.batch, o.out_dt, o.ldx, o.sx, o.sw, o.ldy, o.sy);
  }
};
std::map<GemmKey, hipblasLtMatmulAlgo_t> g_algo;

int blas_fail(int code, const char* what, int st) {
  char msg[256];
  snprintf(msg, sizeof(msg), "%s failed (hipBLASLt status %d)", what, st);
  return v4a::report_error(code, msg);
}

// Y[b][t][n] = sum_k X[b][t][k] W[b][n][k]  (row strides ldx, ldy; batch strides sx, sw, sy,
// in elements).  X, W bf16; Y bf16 (out_dt V4A_BF16) or float32.
int gemm_xwt(const void* X, const void* W, void* Y, int M /*T*/, int N, int K, int batch,
             int64_t ldx, int64_t sx, int64_t sw, int64_t ldy, int64_t sy, int out_dt, void* ws,
             size_t ws_bytes, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return v4a::report_error(V4A_EIO, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_handle[dev]) {
    const hipblasStatus_t st = hipblasLtCreate(&g_handle[dev]);
    if (st != HIPBLAS_STATUS_SUCCESS) return blas_fail(V4A_EIO, "hipblasLtCreate", st);
  }
  hipblasLtHandle_t h = g_handle[dev];
  const hipDataType ty = out_dt == V4A_F32 ? HIP_R_32F : HIP_R_16BF;
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  int rc = V4A_OK;
  hipblasStatus_t st = hipblasLtMatmulDescCreate(&op, HIPBLAS_COMPUTE_32F, HIP_R_32F);
  const hipblasOperation_t tA = HIPBLAS_OP_T, tB = HIPBLAS_OP_N;
  if (st == HIPBLAS_STATUS_SUCCESS)
    st = hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSA, &tA, sizeof(tA));
  if (st == HIPBLAS_STATUS_SUCCESS)
    st = hipblasLtMatmulDescSetAttribute(op, HIPBLASLT_MATMUL_DESC_TRANSB, &tB, sizeof(tB));
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, K, N, K);
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, K, M, ldx);
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&ld, ty, N, M, ldy);
  if (st == HIPBLAS_STATUS_SUCCESS && batch > 1) {
    const int32_t bc = batch;
    hipblasLtMatrixLayoutSetAttribute(la, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof(bc));
    hipblasLtMatrixLayoutSetAttribute(lb, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof(bc));
    hipblasLtMatrixLayoutSetAttribute(ld, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &bc, sizeof(bc));
    hipblasLtMatrixLayoutSetAttribute(la, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &sw, sizeof(sw));
    hipblasLtMatrixLayoutSetAttribute(lb, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &sx, sizeof(sx));
    st = hipblasLtMatrixLayoutSetAttribute(ld, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &sy,
                                           sizeof(sy));
  }
  const uint64_t wsb = ws_bytes < kBlasWs ? ws_bytes : kBlasWs;
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatmulPreferenceCreate(&pref);
  if (st == HIPBLAS_STATUS_SUCCESS)
    st = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                               sizeof(wsb));
  hipblasLtMatmulAlgo_t algo{};
  if (st == HIPBLAS_STATUS_SUCCESS) {
    const GemmKey key{dev, M, N, K, batch, out_dt, ldx, sx, sw, ldy, sy};
    auto it = g_algo.find(key);
    if (it != g_algo.end()) {
      algo = it->second;
    } else {
      hipblasLtMatmulHeuristicResult_t res[1];
      int n = 0;
      st = hipblasLtMatmulAlgoGetHeuristic(h, op, la, lb, ld, ld, pref, 1, res, &n);
      if (st == HIPBLAS_STATUS_SUCCESS && n < 1) st = HIPBLAS_STATUS_NOT_SUPPORTED;
      if (st == HIPBLAS_STATUS_SUCCESS) {
        algo = res[0].algo;
        g_algo[key] = algo;
      }
    }
  }
  if (st == HIPBLAS_STATUS_SUCCESS) {
    const float alpha = 1.0f, beta = 0.0f;
    st = hipblasLtMatmul(h, op, &alpha, W, la, X, lb, &beta, Y, ld, Y, ld, &algo, ws, wsb, s);
  }
  if (st != HIPBLAS_STATUS_SUCCESS) rc = blas_fail(st == HIPBLAS_STATUS_NOT_SUPPORTED ? V4A_ENOTSUP : V4A_EIO,
                                                   "hipblasLtMatmul", st);
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (op) hipblasLtMatmulDescDestroy(op);
  return rc;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

size_t v4a_linear_workspace(int T, int K, int N) {
  if (T < 1 || K < 1 || N < 1) return 0;
  return kBlasWs;
}

int v4a_linear(const void* X, const void* W, int T, int K, int N, void* Y, v4a_dtype out_dt,
               void* ws, size_t ws_bytes, void* stream) {
  if (!X || !W || !Y) return v4a::report_error(V4A_EINVAL, "v4a_linear: null X, W or Y");
  if (T < 1 || K < 1 || N < 1) return v4a::report_error(V4A_EINVAL, "v4a_linear: T, K, N must be >= 1");
  if (K % 8 || N % 8) return v4a::report_error(V4A_ENOTSUP, "v4a_linear: K and N must be multiples of 8");
  if (out_dt != V4A_BF16 && out_dt != V4A_F32)
    return v4a::report_error(V4A_ENOTSUP, "v4a_linear: out_dt must be BF16 or F32");
  if (ws_bytes < kBlasWs || !ws || !aligned16(ws))
    return v4a::report_error(V4A_ENOSPC, "v4a_linear: workspace must be >= v4a_linear_workspace() bytes, 16-byte aligned");
  return gemm_xwt(X, W, Y, T, N, K, 1, K, 0, 0, N, 0, out_dt, ws, ws_bytes, (hipStream_t)stream);
}

size_t v4a_grouped_out_proj_workspace(int T, int n_h, int c, int g, int d_g, int d) {
  if (T < 1 || n_h < 1 || c < 1 || g < 1 || d_g < 1 || d < 1 || n_h % g) return 0;
  const size_t mid = ((size_t)T * g * d_g * 2 + 255) / 256 * 256;
  return mid + kBlasWs;
}

int v4a_grouped_out_proj(const void* o, const void* W_A, const void* W_B, int T, int n_h, int c,
                         int g, int d_g, int d, void* out, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!o || !W_A || !W_B || !out)
    return v4a::report_error(V4A_EINVAL, "v4a_grouped_out_proj: null o, W_A, W_B or out");
  if (T < 1 || n_h < 1 || c < 1 || g < 1 || d_g < 1 || d < 1)
    return v4a::report_error(V4A_EINVAL, "v4a_grouped_out_proj: sizes must be >= 1");
  if (n_h % g) return v4a::report_error(V4A_EINVAL, "v4a_grouped_out_proj: n_h must be a multiple of g");
  const int64_t Kg = (int64_t)c * (n_h / g);
  if (Kg % 8 || d_g % 8 || d % 8)
    return v4a::report_error(V4A_ENOTSUP, "v4a_grouped_out_proj: c n_h/g, d_g and d must be multiples of 8");
  const size_t need = v4a_grouped_out_proj_workspace(T, n_h, c, g, d_g, d);
  if (ws_bytes < need || !ws || (reinterpret_cast<uintptr_t>(ws) & 255))
    return v4a::report_error(V4A_ENOSPC, "v4a_grouped_out_proj: workspace too small or not 256-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  void* mid = ws;
  char* bws = reinterpret_cast<char*>(ws) + (need - kBlasWs);
  // group products: batch i reads columns [i Kg, (i+1) Kg) of every output row
  int rc = gemm_xwt(o, W_A, mid, T, d_g, (int)Kg, g, (int64_t)n_h * c, Kg, (int64_t)d_g * Kg,
                    (int64_t)g * d_g, d_g, V4A_BF16, bws, kBlasWs, s);
  if (rc != V4A_OK) return rc;
  return gemm_xwt(mid, W_B, out, T, d, g * d_g, 1, (int64_t)g * d_g, 0, 0, d, 0, V4A_BF16, bws,
                  kBlasWs, s);
}

}  // extern "C"
