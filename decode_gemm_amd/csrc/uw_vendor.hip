// uw_vendor.hip -- the full-decode pipeline's plain GEMM on the vendor library.
//
// The full-decode pipeline rebuilds the bf16 weights in HBM and hands them to the
// vendor's standard matrix multiply ("Four ways to use compressed weights": full decode
// followed by the library GEMM on ordinary data). On MI355X that library is hipBLASLt.
// This file only marshals the call: Y[M][N] (fp32, row-major, ldy) = X[M][K] (bf16,
// row-major, ldx) * W[N][K]^T (bf16, row-major), i.e. in hipBLASLt's column-major terms
// D (N x M, ldd = ldy) = A^T B with A = W as a K x N column-major matrix (lda = K) and
// B = X as a K x M column-major matrix (ldb = ldx); fp32 accumulation, beta = 0.
//
// Per device, one hipBLASLt handle is created on first use (hipBLASLt allocates its own
// internal resources then). Per (device, M, N, K, ldx, ldy) the descriptors and the
// heuristic's first algorithm that needs no workspace are built once and kept for the life
// of the process (one small entry per distinct problem). One mutex covers the cache and the
// enqueue, so threads may share a device's handle; the enqueue is a short host call.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "uw_internal.h"

namespace uw {
namespace {

struct VendorPlan {
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    bool ok = false;
};

using PlanKey = std::tuple<int, int64_t, int64_t, int64_t, int64_t, int64_t>;

std::mutex g_mu;
hipblasLtHandle_t g_handle[64] = {};
std::map<PlanKey, VendorPlan> g_plans;

// Build the plan of one problem; false (with the plan's resources released) when hipBLASLt
// offers no algorithm for it.
bool build_plan(hipblasLtHandle_t hd, int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldy, VendorPlan& p)
{
    hipblasLtMatmulPreference_t pref = nullptr;
    bool ok = hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    ok = ok && hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, static_cast<uint64_t>(K), static_cast<uint64_t>(N), K) ==
                   HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, static_cast<uint64_t>(K), static_cast<uint64_t>(M), ldx) ==
                   HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&p.d, HIP_R_32F, static_cast<uint64_t>(N), static_cast<uint64_t>(M), ldy) ==
                   HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
    const uint64_t no_ws = 0;
    ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &no_ws,
                                                     sizeof no_ws) == HIPBLAS_STATUS_SUCCESS;
    if (ok) {
        hipblasLtMatmulHeuristicResult_t res[4];
        int n = 0;
        ok = hipblasLtMatmulAlgoGetHeuristic(hd, p.op, p.a, p.b, p.d, p.d, pref, 4, res, &n) == HIPBLAS_STATUS_SUCCESS;
        ok = ok && n > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize == 0;
        if (ok) p.algo = res[0].algo;
    }
    if (pref) (void)hipblasLtMatmulPreferenceDestroy(pref);
    if (!ok) {
        if (p.d) (void)hipblasLtMatrixLayoutDestroy(p.d);
        if (p.b) (void)hipblasLtMatrixLayoutDestroy(p.b);
        if (p.a) (void)hipblasLtMatrixLayoutDestroy(p.a);
        if (p.op) (void)hipblasLtMatmulDescDestroy(p.op);
        p = VendorPlan{};
    }
    p.ok = ok;
    return ok;
}

}  // namespace

hipError_t vendor_gemm_bf16(const uint16_t* w, const uint16_t* x, float* y, int64_t M, int64_t N, int64_t K,
                            int64_t ldx, int64_t ldy, hipStream_t s)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_handle[dev] && hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
        g_handle[dev] = nullptr;
        return hipErrorNotSupported;
    }
    const hipblasLtHandle_t hd = g_handle[dev];
    const PlanKey key{dev, M, N, K, ldx, ldy};
    auto it = g_plans.find(key);
    if (it == g_plans.end()) {
        VendorPlan p;
        build_plan(hd, M, N, K, ldx, ldy, p);
        it = g_plans.emplace(key, p).first;  // a failed plan is kept too: asked again, it fails at once
    }
    const VendorPlan& plan = it->second;
    if (!plan.ok) return hipErrorNotSupported;
    const float alpha = 1.0f, beta = 0.0f;
    const hipblasStatus_t st = hipblasLtMatmul(hd, plan.op, &alpha, w, plan.a, x, plan.b, &beta, y, plan.d, y, plan.d,
                                               &plan.algo, nullptr, 0, s);
    return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace uw
