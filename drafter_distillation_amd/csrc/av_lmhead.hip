// Backward of the drafter's LM head (the step after the verify + OPD pass):
//   d_hid[r, h] = sum_v dz[r, v] W[v, h]        d_W[v, h] = sum_r dz[r, v] hid[r, h]
// Two plain bfloat16 GEMMs with float32 accumulation and output, run by
// hipBLASLt on the matrix cores.  Row-major operands are passed as their
// column-major transposes: d_hid^T = W^T dz^T and d_W^T = hid^T dz.
// Semantics are documented in include/av.h.

#include <hipblaslt/hipblaslt.h>
#include <stdint.h>
#include <stdio.h>

#include <map>
#include <mutex>
#include <tuple>

#include "av.h"

namespace {

constexpr int kMaxDevices = 64;
thread_local char g_err[256] = "";

struct Blas {
  hipblasLtHandle_t h = nullptr;
  hipblasStatus_t st = HIPBLAS_STATUS_SUCCESS;
};
Blas g_blas[kMaxDevices];
std::once_flag g_blas_once[kMaxDevices];

// Chosen algorithm per (device, m, n, k, transB, workspace bytes).
using AlgoKey = std::tuple<int, int, int, int, int, size_t>;
std::mutex g_algo_mu;
std::map<AlgoKey, hipblasLtMatmulAlgo_t> g_algo;

int blas_fail(const char* what, int code) {
  snprintf(g_err, sizeof(g_err), "hipBLASLt %s: status %d", what, code);
  return AV_EHIP;
}

struct Desc {  // matmul and matrix descriptors of one call, destroyed on exit
  hipblasLtMatmulDesc_t md = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  ~Desc() {
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (c) hipblasLtMatrixLayoutDestroy(c);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (md) hipblasLtMatmulDescDestroy(md);
  }
};

#define AV_BLAS(call)                                                     \
  do {                                                                    \
    const hipblasStatus_t s_ = (call);                                    \
    if (s_ != HIPBLAS_STATUS_SUCCESS) return blas_fail(#call, (int)s_);   \
  } while (0)

// Column-major C[m, n] = A[m, k] op(B)[k, n], A not transposed (lda = m),
// B stored [k, n] (ldb = k) or, transposed, [n, k] (ldb = n); bf16 inputs,
// float32 accumulation and output (ldc = m).
int gemm(int dev, hipblasLtHandle_t h, int m, int n, int k, bool transb, const void* A, const void* B, float* C,
         void* ws, size_t wsb, hipStream_t stream) {
  Desc d;
  const hipblasOperation_t opn = HIPBLAS_OP_N, opb = transb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  AV_BLAS(hipblasLtMatmulDescCreate(&d.md, HIPBLAS_COMPUTE_32F, HIP_R_32F));
  AV_BLAS(hipblasLtMatmulDescSetAttribute(d.md, HIPBLASLT_MATMUL_DESC_TRANSA, &opn, sizeof(opn)));
  AV_BLAS(hipblasLtMatmulDescSetAttribute(d.md, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)));
  AV_BLAS(hipblasLtMatrixLayoutCreate(&d.a, HIP_R_16BF, m, k, m));
  AV_BLAS(hipblasLtMatrixLayoutCreate(&d.b, HIP_R_16BF, transb ? n : k, transb ? k : n, transb ? n : k));
  AV_BLAS(hipblasLtMatrixLayoutCreate(&d.c, HIP_R_32F, m, n, m));
  hipblasLtMatmulAlgo_t algo;
  const AlgoKey key{dev, m, n, k, transb ? 1 : 0, wsb};
  bool have = false;
  {
    std::lock_guard<std::mutex> g(g_algo_mu);
    auto it = g_algo.find(key);
    if (it != g_algo.end()) {
      algo = it->second;
      have = true;
    }
  }
  if (!have) {
    AV_BLAS(hipblasLtMatmulPreferenceCreate(&d.pref));
    AV_BLAS(hipblasLtMatmulPreferenceSetAttribute(d.pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                                  sizeof(wsb)));
    hipblasLtMatmulHeuristicResult_t res;
    int nres = 0;
    AV_BLAS(hipblasLtMatmulAlgoGetHeuristic(h, d.md, d.a, d.b, d.c, d.c, d.pref, 1, &res, &nres));
    if (nres < 1) return AV_EUNSUPPORTED;
    algo = res.algo;
    std::lock_guard<std::mutex> g(g_algo_mu);
    g_algo[key] = algo;
  }
  const float alpha = 1.0f, beta = 0.0f;
  AV_BLAS(hipblasLtMatmul(h, d.md, &alpha, A, d.a, B, d.b, &beta, C, d.c, C, d.c, &algo, ws, wsb, stream));
  return AV_OK;
}

}  // namespace

extern "C" {

size_t av_lm_head_workspace_bytes(void) { return (size_t)64 << 20; }

const char* av_lm_head_last_error(void) { return g_err; }

int av_lm_head_bwd(int R, int V, int H, const void* dz, const void* w, const void* hid, float* d_hid,
                   float* d_w, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dz || R < 1 || V < 1 || H < 1) return AV_EINVAL;
  if ((d_hid && !w) || (d_w && !hid)) return AV_EINVAL;
  if (workspace_bytes > 0 && !workspace) return AV_EINVAL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AV_EHIP;
  std::call_once(g_blas_once[dev], [dev]() { g_blas[dev].st = hipblasLtCreate(&g_blas[dev].h); });
  if (g_blas[dev].st != HIPBLAS_STATUS_SUCCESS) return blas_fail("hipblasLtCreate", (int)g_blas[dev].st);
  const hipblasLtHandle_t h = g_blas[dev].h;
  const hipStream_t s = (hipStream_t)stream;
  int rc = AV_OK;
  // d_hid^T [H, R] = W^T [H, V] dz^T [V, R]
  if (d_hid) rc = gemm(dev, h, H, R, V, false, w, dz, d_hid, workspace, workspace_bytes, s);
  // d_W^T [H, V] = hid^T [H, R] dz [R, V]  (dz^T stored [V, R], transposed)
  if (rc == AV_OK && d_w) rc = gemm(dev, h, H, V, R, true, hid, dz, d_w, workspace, workspace_bytes, s);
  return rc;
}

}  // extern "C"
