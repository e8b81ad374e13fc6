// The projection through the vendor library, as a comparator for the hand-written kernel
// (speakrs 0.6.0, page `lstm.rs`, `Oxide` and its locked projection helper: the same stack
// with the input projection handed to the vendor GEMM). hipBLASLt computes, per layer,
//   gates (row-major [rows][1024]) = x [rows][in] · Wᵀ + bias
// in FP32 (no reduced-precision compute type), with the bias added by its epilogue. In
// column-major terms: D (1024 x rows) = op_T(W: kpad x 1024) · x (in x rows) + bias.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include "bilstm_host.h"

namespace bl {

namespace {

const char *blas_name(hipblasStatus_t s) {
    switch (s) {
        case HIPBLAS_STATUS_SUCCESS: return "success";
        case HIPBLAS_STATUS_NOT_INITIALIZED: return "not initialized";
        case HIPBLAS_STATUS_ALLOC_FAILED: return "allocation failed";
        case HIPBLAS_STATUS_INVALID_VALUE: return "invalid value";
        case HIPBLAS_STATUS_ARCH_MISMATCH: return "architecture mismatch";
        case HIPBLAS_STATUS_EXECUTION_FAILED: return "execution failed";
        case HIPBLAS_STATUS_NOT_SUPPORTED: return "not supported";
        default: return "error";
    }
}

#define BL_BLAS(expr, context)                                                                   \
    do {                                                                                         \
        hipblasStatus_t bl_s_ = (expr);                                                          \
        if (bl_s_ != HIPBLAS_STATUS_SUCCESS) {                                                   \
            return fail(BILSTM_HIP_ERROR, "%s: %s failed: %s", context, #expr, blas_name(bl_s_)); \
        }                                                                                        \
    } while (0)

constexpr size_t kWorkspaceBytes = 64ull << 20;

}  // namespace

struct LibraryProjection {
    hipblasLtHandle_t handle = nullptr;
    void *workspace = nullptr;
    struct Layer {
        hipblasLtMatmulDesc_t desc = nullptr;
        hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
        hipblasLtMatmulAlgo_t algo{};
        size_t workspace = 0;
        long rows = 0;
    } layer[kLayers];
};

void library_projection_destroy(LibraryProjection *lp) {
    if (lp == nullptr) return;
    for (auto &L : lp->layer) {
        if (L.desc) (void)hipblasLtMatmulDescDestroy(L.desc);
        if (L.a) (void)hipblasLtMatrixLayoutDestroy(L.a);
        if (L.b) (void)hipblasLtMatrixLayoutDestroy(L.b);
        if (L.d) (void)hipblasLtMatrixLayoutDestroy(L.d);
    }
    if (lp->workspace) (void)hipFree(lp->workspace);
    if (lp->handle) (void)hipblasLtDestroy(lp->handle);
    delete lp;
}

bilstm_status library_projection_create(long rows, const int in[kLayers], const int kpad[kLayers],
                                        float *const bias[kLayers], LibraryProjection **out) {
    auto *lp = new LibraryProjection();
    *out = lp;  // the caller destroys it, also on failure
    BL_BLAS(hipblasLtCreate(&lp->handle), "library projection");
    hipError_t e = hipMalloc(&lp->workspace, kWorkspaceBytes);
    if (e != hipSuccess) {
        lp->workspace = nullptr;
        return fail(BILSTM_HIP_ERROR, "library projection: workspace: %s", hipGetErrorString(e));
    }
    for (int l = 0; l < kLayers; ++l) {
        auto &L = lp->layer[l];
        L.rows = rows;
        BL_BLAS(hipblasLtMatmulDescCreate(&L.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F), "library projection");
        const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
        BL_BLAS(hipblasLtMatmulDescSetAttribute(L.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)), "library projection");
        BL_BLAS(hipblasLtMatmulDescSetAttribute(L.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)), "library projection");
        const hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_BIAS;
        BL_BLAS(hipblasLtMatmulDescSetAttribute(L.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)), "library projection");
        const void *bp = bias[l];
        BL_BLAS(hipblasLtMatmulDescSetAttribute(L.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bp, sizeof(bp)), "library projection");
        const hipDataType bt = HIP_R_32F;
        BL_BLAS(hipblasLtMatmulDescSetAttribute(L.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt, sizeof(bt)), "library projection");
        BL_BLAS(hipblasLtMatrixLayoutCreate(&L.a, HIP_R_32F, in[l], kGateCols, kpad[l]), "library projection");
        BL_BLAS(hipblasLtMatrixLayoutCreate(&L.b, HIP_R_32F, in[l], rows, in[l]), "library projection");
        BL_BLAS(hipblasLtMatrixLayoutCreate(&L.d, HIP_R_32F, kGateCols, rows, kGateCols), "library projection");
        hipblasLtMatmulPreference_t pref = nullptr;
        BL_BLAS(hipblasLtMatmulPreferenceCreate(&pref), "library projection");
        const uint64_t ws = kWorkspaceBytes;
        hipblasStatus_t s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                                  &ws, sizeof(ws));
        hipblasLtMatmulHeuristicResult_t result{};
        int found = 0;
        if (s == HIPBLAS_STATUS_SUCCESS) {
            s = hipblasLtMatmulAlgoGetHeuristic(lp->handle, L.desc, L.a, L.b, L.d, L.d, pref, 1, &result, &found);
        }
        (void)hipblasLtMatmulPreferenceDestroy(pref);
        BL_BLAS(s, "library projection heuristic");
        if (found < 1 || result.state != HIPBLAS_STATUS_SUCCESS) {
            return fail(BILSTM_UNSUPPORTED, "library projection: hipBLASLt has no FP32 algorithm for layer %d", l);
        }
        L.algo = result.algo;
        L.workspace = result.workspaceSize;
    }
    return BILSTM_OK;
}

bilstm_status library_projection_run(LibraryProjection *lp, int layer, const float *x, const float *w,
                                     float *gates, hipStream_t stream) {
    auto &L = lp->layer[layer];
    const float alpha = 1.0f, beta = 0.0f;
    BL_BLAS(hipblasLtMatmul(lp->handle, L.desc, &alpha, w, L.a, x, L.b, &beta, gates, L.d, gates, L.d, &L.algo,
                            lp->workspace, L.workspace, stream),
            "library projection");
    return BILSTM_OK;
}

}  // namespace bl
