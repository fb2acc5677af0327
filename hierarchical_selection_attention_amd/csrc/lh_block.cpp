// The attention block around the Lighthouse layer: the projections of
// "Long Context Pre-Training with Lighthouse Attention", Sec. 3.1 Eq. (1)
// (q = x W_Q, k = x W_K, v = x W_V) feed the pyramid pool (Fig. 1), and the
// layer output leaves through an output projection, as in the Llama-style
// models of the experiments (Sec. 4).  The four weight products of each pass
// are plain GEMMs and run in hipBLASLt (bf16 operands, fp32 accumulation);
// everything between them is the layer's own kernels.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <tuple>

#include "lighthouse.h"
#include "lh_internal.h"

namespace lh {
namespace {

constexpr size_t kGemmWs = size_t(64) << 20;   // hipBLASLt workspace inside the block workspace
constexpr int kMaxDevices = 64;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct GemmKey {
    int dev, ta, tb, c_f32;
    int64_t M, N, K, lda, ldb, ldc;
    bool operator<(const GemmKey& o) const {
        return std::tie(dev, ta, tb, c_f32, M, N, K, lda, ldb, ldc) <
               std::tie(o.dev, o.ta, o.tb, o.c_f32, o.M, o.N, o.K, o.lda, o.ldb, o.ldc);
    }
};

struct GemmPlan {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
};

std::mutex g_gemm_mu;
hipblasLtHandle_t g_handle[kMaxDevices] = {};
std::map<GemmKey, GemmPlan> g_plans;

// Row-major C[M][N] = op(A) op(B) with op(A) M x K and op(B) K x N; A is
// stored [M][K] (lda) or, when ta, [K][M]; B is stored [K][N] (ldb) or, when
// tb, [N][K].  A and B bf16; C bf16 or fp32 (c_f32), overwritten.  hipBLASLt
// is column-major, so the call computes C^T = op(B)^T op(A)^T: its first
// operand is B and its second is A.
int gemm_rm(bool ta, bool tb, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
            int64_t ldb, void* C, int64_t ldc, bool c_f32, void* gws, hipStream_t s) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LH_ERR_HIP;
    std::lock_guard<std::mutex> g(g_gemm_mu);
    if (!g_handle[dev] && hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
        g_handle[dev] = nullptr;
        return LH_ERR_GEMM;
    }
    const GemmKey key{dev, ta, tb, c_f32, M, N, K, lda, ldb, ldc};
    auto it = g_plans.find(key);
    if (it == g_plans.end()) {
        GemmPlan p;
        const hipDataType ct = c_f32 ? HIP_R_32F : HIP_R_16BF;
        const hipblasOperation_t opa = tb ? HIPBLAS_OP_T : HIPBLAS_OP_N, opb = ta ? HIPBLAS_OP_T : HIPBLAS_OP_N;
        bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
        ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)) ==
                       HIPBLAS_STATUS_SUCCESS;
        ok = ok && hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)) ==
                       HIPBLAS_STATUS_SUCCESS;
        // stored shapes, column-major: B is N x K (or K x N when tb), A is K x M (or M x K when ta)
        ok = ok && hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, tb ? K : N, tb ? N : K, ldb) ==
                       HIPBLAS_STATUS_SUCCESS;
        ok = ok && hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, ta ? M : K, ta ? K : M, lda) ==
                       HIPBLAS_STATUS_SUCCESS;
        ok = ok && hipblasLtMatrixLayoutCreate(&p.lc, ct, N, M, ldc) == HIPBLAS_STATUS_SUCCESS;
        hipblasLtMatmulPreference_t pref = nullptr;
        ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
        const uint64_t wsmax = kGemmWs;
        ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax,
                                                         sizeof(wsmax)) == HIPBLAS_STATUS_SUCCESS;
        hipblasLtMatmulHeuristicResult_t res[8];
        int n = 0;
        ok = ok && hipblasLtMatmulAlgoGetHeuristic(g_handle[dev], p.desc, p.la, p.lb, p.lc, p.lc, pref, 8, res, &n) ==
                       HIPBLAS_STATUS_SUCCESS;
        if (pref) hipblasLtMatmulPreferenceDestroy(pref);
        int pick = -1;
        for (int i = 0; ok && i < n; ++i)
            if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= kGemmWs) {
                pick = i;
                break;
            }
        if (pick < 0) {
            if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
            if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
            if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
            if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
            return LH_ERR_GEMM;
        }
        p.algo = res[pick].algo;
        p.ws = res[pick].workspaceSize;
        it = g_plans.emplace(key, p).first;
    }
    const GemmPlan& p = it->second;
    const float alpha = 1.0f, beta = 0.0f;
    const hipblasStatus_t st = hipblasLtMatmul(g_handle[dev], p.desc, &alpha, B, p.la, A, p.lb, &beta, C, p.lc, C,
                                               p.lc, &p.algo, gws, kGemmWs, s);
    return st == HIPBLAS_STATUS_SUCCESS ? LH_OK : LH_ERR_GEMM;
}

// Block workspace: [layer workspace][q, k, v as [N][3Hd] bf16, reused as the
// gradient [N][3Hd] in the backward][dO: N*Hd bf16][GEMM workspace]
struct BlockPlan {
    size_t lh_bytes, off_qkv, off_do, off_gemm, total;
};

int block_plan(int N, int H, int d, int dm, int p, int L, int K, BlockPlan* b) {
    if (dm <= 0 || dm % 8 != 0) return LH_ERR_SHAPE;
    const size_t lhb = lh_workspace_bytes(N, H, d, p, L, K, LH_BF16);
    if (lhb == 0) {
        const int64_t S = lh_subseq_len(N, p, L, K);
        return S < 0 ? (int)S : LH_ERR_SHAPE;
    }
    const size_t nhd = (size_t)N * H * d;
    b->lh_bytes = lhb;
    b->off_qkv = align256(lhb);
    b->off_do = align256(b->off_qkv + 3 * nhd * 2);
    b->off_gemm = align256(b->off_do + nhd * 2);
    b->total = b->off_gemm + kGemmWs;
    return LH_OK;
}

bool al16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// The GEMM handle is the current device's: a stream of another device is refused.
int check_stream_device(hipStream_t s) {
    if (!s) return LH_OK;
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(s, &sdev) != hipSuccess) return LH_ERR_HIP;
    return sdev == cur ? LH_OK : LH_ERR_ARG;
}

}  // namespace
}  // namespace lh

using namespace lh;

#define LH_GEMM(id, call)                                  \
    do {                                                   \
        const StageMark m_ = stage_open(s);                \
        const int rc_ = (call);                            \
        stage_close((id), s, m_);                          \
        if (rc_ != LH_OK) return rc_;                      \
    } while (0)

extern "C" {

size_t lh_block_workspace_bytes(int N, int H, int d, int dm, int p, int L, int K) {
    BlockPlan b;
    return block_plan(N, H, d, dm, p, L, K, &b) == LH_OK ? b.total : 0;
}

int lh_block_forward(const void* x, const void* w_qkv, const void* w_o, void* o, void* y, int N, int H, int d,
                     int dm, int p, int L, int K, void* ws, size_t ws_bytes, void* stream) {
    BlockPlan b;
    int rc = block_plan(N, H, d, dm, p, L, K, &b);
    if (rc) return rc;
    if (!x || !w_qkv || !w_o || !o || !y) return LH_ERR_ARG;
    if (!al16(x) || !al16(w_qkv) || !al16(w_o) || !al16(o) || !al16(y)) return LH_ERR_ARG;
    if (!ws || reinterpret_cast<uintptr_t>(ws) % 256 != 0 || ws_bytes < b.total) return LH_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((rc = check_stream_device(s))) return rc;
    char* w = reinterpret_cast<char*>(ws);
    const int64_t hd = (int64_t)H * d;
    uint16_t* qkv = reinterpret_cast<uint16_t*>(w + b.off_qkv);
    void* gws = w + b.off_gemm;
    // [q k v] = x w_qkv in one product: token t's q, k and v rows side by side
    LH_GEMM(ST_PROJ_QKV, gemm_rm(false, false, N, 3 * hd, dm, x, dm, w_qkv, 3 * hd, qkv, 3 * hd, false, gws, s));
    rc = forward_strided(qkv, qkv + hd, qkv + 2 * hd, o, N, H, d, p, L, K, LH_BF16, LH_SCORE_QK,
                         LH_SELECT_PARTITION, w, b.lh_bytes, stream, 3 * hd);
    if (rc) return rc;
    LH_GEMM(ST_PROJ_OUT, gemm_rm(false, false, N, dm, hd, o, hd, w_o, dm, y, dm, false, gws, s));
    return LH_OK;
}

int lh_block_backward(const void* x, const void* w_qkv, const void* w_o, const void* o, const void* dy, void* dx,
                      float* dw_qkv, float* dw_o, int N, int H, int d, int dm, int p, int L, int K,
                      int scatter_mode, void* ws, size_t ws_bytes, void* stream) {
    BlockPlan b;
    int rc = block_plan(N, H, d, dm, p, L, K, &b);
    if (rc) return rc;
    if (!x || !w_qkv || !w_o || !o || !dy || !dx || !dw_qkv || !dw_o) return LH_ERR_ARG;
    if (!al16(x) || !al16(w_qkv) || !al16(w_o) || !al16(o) || !al16(dy) || !al16(dx) || !al16(dw_qkv) ||
        !al16(dw_o))
        return LH_ERR_ARG;
    if (!ws || reinterpret_cast<uintptr_t>(ws) % 256 != 0 || ws_bytes < b.total) return LH_ERR_WORKSPACE;
    if (scatter_mode != LH_SCATTER_FP_ATOMIC && scatter_mode != LH_SCATTER_INT_ATOMIC) return LH_ERR_DTYPE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((rc = check_stream_device(s))) return rc;
    char* w = reinterpret_cast<char*>(ws);
    const int64_t hd = (int64_t)H * d;
    uint16_t* g = reinterpret_cast<uint16_t*>(w + b.off_qkv);   // [N][3Hd]: dq | dk | dv per token
    uint16_t* dout = reinterpret_cast<uint16_t*>(w + b.off_do);
    void* gws = w + b.off_gemm;
    // dO = dy w_o^T, and dw_o = o^T dy
    LH_GEMM(ST_PROJ_OUT_DX, gemm_rm(false, true, N, hd, dm, dy, dm, w_o, dm, dout, hd, false, gws, s));
    LH_GEMM(ST_PROJ_OUT_DW, gemm_rm(true, false, hd, dm, N, o, hd, dy, dm, dw_o, dm, true, gws, s));
    rc = backward_strided(dout, g, g + hd, g + 2 * hd, N, H, d, p, L, K, LH_BF16, scatter_mode, w, b.lh_bytes,
                             stream, 3 * hd);
    if (rc) return rc;
    // dx = [dq dk dv] w_qkv^T, and dw_qkv = x^T [dq dk dv]
    LH_GEMM(ST_PROJ_QKV_DX, gemm_rm(false, true, N, dm, 3 * hd, g, 3 * hd, w_qkv, 3 * hd, dx, dm, false, gws, s));
    LH_GEMM(ST_PROJ_QKV_DW, gemm_rm(true, false, dm, 3 * hd, N, x, dm, g, 3 * hd, dw_qkv, 3 * hd, true, gws, s));
    return LH_OK;
}

}  // extern "C"
