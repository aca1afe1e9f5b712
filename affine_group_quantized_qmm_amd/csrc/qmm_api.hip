// C ABI of the library: argument validation, kernel choice and launches.
// Declarations and the full contract are in include/qmm.h.
#include "qmm.h"
#include "qmm_kernels.hpp"

#include <stdint.h>
#include <string.h>

namespace {

constexpr int kMaxRowsPerLaunch = 16;  // rows of one multi-row launch (one MFMA tile)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bits_supported(int bits) { return bits == 4 || bits == 5 || bits == 6 || bits == 8; }
bool group_supported(int G) { return G == 32 || G == 64 || G == 128; }

// Shape checks shared by every product entry point.
int check_shape(int M, int K, int N, int bits, int G)
{
    if (!bits_supported(bits))
        return QMM_ERR_BITS;
    if (!group_supported(G))
        return QMM_ERR_GROUP;
    if (M < 1 || K < 1 || N < 1 || K % G != 0)
        return QMM_ERR_SHAPE;
    // Kernels index K*bits and per-row group counts in 32-bit integers.
    if ((int64_t)K * bits >= (int64_t)1 << 31 || M >= (1 << 30) || N >= (1 << 30))
        return QMM_ERR_SHAPE;
    return QMM_OK;
}

enum class Kernel { qmv, mfma };

Kernel choose_kernel(int M) { return M == 1 ? Kernel::qmv : Kernel::mfma; }

const char *kernel_label(Kernel k) { return k == Kernel::qmv ? "qmv" : "mfma"; }

// Launch one product (all of M, in 16-row steps for the multi-row kernel)
// writing either y (split == 1) or the split partials (y = workspace).
int launch_product(Kernel kind, const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                   const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                   int split, hipStream_t stream)
{
    qmm::ProductArgs a{};
    a.wq = wq;
    a.scales = scales;
    a.biases = biases;
    a.K = K;
    a.N = N;
    a.split = split;
    a.y_slice_stride = (size_t)M * N;
    const int step = kind == Kernel::qmv ? 1 : kMaxRowsPerLaunch;
    for (int m0 = 0; m0 < M; m0 += step) {
        a.M = M - m0 < step ? M - m0 : step;
        a.x = x + (size_t)m0 * K;
        a.y = y + (size_t)m0 * N;
        const hipError_t e = kind == Kernel::qmv ? qmm::launch_qmv(a, bits, G, stream)
                                                 : qmm::launch_mfma(a, bits, G, stream);
        if (e != hipSuccess)
            return QMM_ERR_LAUNCH;
    }
    return QMM_OK;
}

}  // namespace

extern "C" {

const char *qmm_strerror(int code)
{
    switch (code) {
    case QMM_OK: return "success";
    case QMM_ERR_NULL: return "a required pointer is NULL";
    case QMM_ERR_SHAPE: return "bad shape: need M, K, N >= 1, K a multiple of G, sizes in range";
    case QMM_ERR_BITS: return "unsupported bit width (supported: 4, 5, 6, 8)";
    case QMM_ERR_GROUP: return "unsupported group size (supported: 32, 64, 128)";
    case QMM_ERR_SPLIT: return "bad split_k: need 1 <= split_k <= K/G";
    case QMM_ERR_WORKSPACE: return "workspace smaller than qmm_splitk_workspace_bytes(M, N, split_k)";
    case QMM_ERR_ALIGN: return "x, wq, scales, biases, y and workspace must be 16-byte aligned";
    case QMM_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    default: return "unknown error code";
    }
}

size_t qmm_splitk_workspace_bytes(int M, int N, int split_k)
{
    if (M < 1 || N < 1 || split_k < 2)
        return 0;
    return (size_t)split_k * (size_t)M * (size_t)N * sizeof(float);
}

int qmm_validate(const void *x, const void *wq, const void *scales, const void *biases,
                 const void *y, int M, int K, int N, int bits, int G, int split_k,
                 const void *workspace, size_t workspace_bytes)
{
    if (!x || !wq || !scales || !biases || !y || (split_k > 1 && !workspace))
        return QMM_ERR_NULL;
    const int rc = check_shape(M, K, N, bits, G);
    if (rc != QMM_OK)
        return rc;
    if (split_k != 0) {
        if (split_k < 1 || split_k > K / G)
            return QMM_ERR_SPLIT;
        if (workspace_bytes < qmm_splitk_workspace_bytes(M, N, split_k))
            return QMM_ERR_WORKSPACE;
    }
    if (!aligned16(x) || !aligned16(wq) || !aligned16(scales) || !aligned16(biases) ||
        !aligned16(y) || (split_k > 1 && !aligned16(workspace)))
        return QMM_ERR_ALIGN;
    return QMM_OK;
}

const char *qmm_kernel_name(int M, int K, int N, int bits, int G)
{
    if (check_shape(M, K, N, bits, G) != QMM_OK)
        return nullptr;
    return kernel_label(choose_kernel(M));
}

int qmm_pack(const uint8_t *codes, uint32_t *packed, int N, int K, int bits, hipStream_t stream)
{
    if (!codes || !packed)
        return QMM_ERR_NULL;
    if (!bits_supported(bits))
        return QMM_ERR_BITS;
    if (N < 1 || K < 1 || ((int64_t)K * bits) % 32 != 0 || (int64_t)K * bits >= (int64_t)1 << 31 ||
        N >= (1 << 30))
        return QMM_ERR_SHAPE;
    if (!aligned16(packed))
        return QMM_ERR_ALIGN;
    return qmm::launch_pack(codes, packed, N, K, bits, stream) == hipSuccess ? QMM_OK
                                                                              : QMM_ERR_LAUNCH;
}

int qmm_forward(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                hipStream_t stream)
{
    const int rc = qmm_validate(x, wq, scales, biases, y, M, K, N, bits, G, 0, nullptr, 0);
    if (rc != QMM_OK)
        return rc;
    return launch_product(choose_kernel(M), x, wq, scales, biases, y, M, K, N, bits, G, 1, stream);
}

int qmm_forward_splitk(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                       const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                       int split_k, float *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const int rc = qmm_validate(x, wq, scales, biases, y, M, K, N, bits, G,
                                split_k < 1 ? -1 : split_k, workspace, workspace_bytes);
    if (rc != QMM_OK)
        return rc;
    const Kernel kind = choose_kernel(M);
    if (split_k == 1)
        return launch_product(kind, x, wq, scales, biases, y, M, K, N, bits, G, 1, stream);
    const int rc1 = launch_product(kind, x, wq, scales, biases, workspace, M, K, N, bits, G,
                                   split_k, stream);
    if (rc1 != QMM_OK)
        return rc1;
    return qmm::launch_splitk_reduce(workspace, y, split_k, (size_t)M * N, stream) == hipSuccess
               ? QMM_OK
               : QMM_ERR_LAUNCH;
}

int qmm_forward_kernel(const char *kernel, const uint16_t *x, const uint32_t *wq,
                       const uint16_t *scales, const uint16_t *biases, float *y, int M, int K,
                       int N, int bits, int G, hipStream_t stream)
{
    const int rc = qmm_validate(x, wq, scales, biases, y, M, K, N, bits, G, 0, nullptr, 0);
    if (rc != QMM_OK)
        return rc;
    if (!kernel)
        return QMM_ERR_NULL;
    Kernel kind;
    if (strcmp(kernel, "qmv") == 0)
        kind = Kernel::qmv;
    else if (strcmp(kernel, "mfma") == 0)
        kind = Kernel::mfma;
    else
        return QMM_ERR_SHAPE;
    return launch_product(kind, x, wq, scales, biases, y, M, K, N, bits, G, 1, stream);
}

}  // extern "C"
