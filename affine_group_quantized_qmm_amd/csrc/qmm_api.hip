// C ABI of the library: argument validation, kernel choice and launches.
// Declarations and the full contract are in include/qmm.h.
#include "qmm.h"
#include "qmm_kernels.hpp"

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

namespace {

constexpr int kMaxRowsPerLaunch = 16;  // rows of one multi-row launch (one MFMA tile)
constexpr int kQmvRowsPerLaunch = 8;   // rows of one launch of the row-exact VALU kernel
constexpr int kQmvMaxRows = 2;         // qmm_forward takes the VALU kernel up to this many rows
static_assert(QMM_MAX_FUSED <= qmm::kMaxProj, "the launch arguments hold every fused projection");

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bits_supported(int bits) { return bits >= 2 && bits <= 8 && bits != 7; }
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

enum class Kernel { qmv, mfma, mfma_lds };

const char *kernel_label(Kernel k)
{
    return k == Kernel::qmv ? "qmv" : k == Kernel::mfma ? "mfma" : "mfma_lds";
}

qmm::ProductArgs product_args(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                              const uint16_t *biases, float *y, int M, int K, int N, int split)
{
    qmm::ProductArgs a{};
    a.x = x;
    a.wq = wq;
    a.scales = scales;
    a.biases = biases;
    a.y = y;
    a.M = M;
    a.K = K;
    a.N = N;
    a.split = split;
    a.y_slice_stride = (size_t)M * N;
    return a;
}

// The register-resident kernel's support depends on K, bits, G and the
// split only; M and the pointers do not matter.
bool xr_supported(int K, int N, int bits, int G, int split)
{
    const qmm::ProductArgs a = product_args(nullptr, nullptr, nullptr, nullptr, nullptr,
                                            kMaxRowsPerLaunch, K, N, split);
    return qmm::mfma_xr_supported(a, bits, G);
}

// One and two rows: the row-exact VALU kernel (measured on the 5120 x 17408
// 4-bit projection: 12.8 and 17.9 us against 21.9 us for the matrix-core
// kernel at two rows; from three rows on the matrix cores win). A shape that
// neither matrix-core kernel takes (3-bit codes at G = 32 with K past the
// register-resident kernel) runs on the VALU kernel, 8 rows per launch.
Kernel choose_kernel(int M, int K, int N, int bits, int G, int split)
{
    if (M <= kQmvMaxRows)
        return Kernel::qmv;
    if (xr_supported(K, N, bits, G, split))
        return Kernel::mfma;
    return qmm::mfma_supported(bits, G) ? Kernel::mfma_lds : Kernel::qmv;
}

// Launch one product (all of M, in 16-row steps for the multi-row kernels)
// writing either y (split == 1) or the split partials (y = workspace).
int launch_args(Kernel kind, const qmm::ProductArgs &full, int bits, int G, hipStream_t stream)
{
    if ((kind == Kernel::mfma && !xr_supported(full.K, full.N, bits, G, full.split)) ||
        (kind == Kernel::mfma_lds && !qmm::mfma_supported(bits, G)))
        return QMM_ERR_UNSUPPORTED;
    const int M = full.M;
    const int step = kind == Kernel::qmv ? kQmvRowsPerLaunch : kMaxRowsPerLaunch;
    for (int m0 = 0; m0 < M; m0 += step) {
        const qmm::ProductArgs a = qmm::rows_of(full, m0, M - m0 < step ? M - m0 : step);
        hipError_t e;
        switch (kind) {
        case Kernel::qmv: e = qmm::launch_qmv(a, bits, G, false, stream); break;
        case Kernel::mfma: e = qmm::launch_mfma_xr(a, bits, G, false, stream); break;
        default: e = qmm::launch_mfma(a, bits, G, false, stream); break;
        }
        if (e != hipSuccess)
            return QMM_ERR_LAUNCH;
    }
    return QMM_OK;
}

int launch_product(Kernel kind, const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                   const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                   int split, hipStream_t stream)
{
    return launch_args(kind, product_args(x, wq, scales, biases, y, M, K, N, split), bits, G, stream);
}

// The original one-row kernel, once per row: the reference a multi-row
// kernel is admitted against.
int launch_rows_one_by_one(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                           const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                           hipStream_t stream)
{
    const qmm::ProductArgs full = product_args(x, wq, scales, biases, y, M, K, N, 1);
    for (int m = 0; m < M; ++m)
        if (qmm::launch_qmv(qmm::rows_of(full, m, 1), bits, G, false, stream) != hipSuccess)
            return QMM_ERR_LAUNCH;
    return QMM_OK;
}

// Admission verdicts per (kind, K, N, M, bits, G): 1 admitted, 0 rejected.
enum class AdmitKind { rowexact, forward };
using AdmitKey = std::tuple<int, int, int, int, int, int>;
std::mutex admit_mutex;
std::map<AdmitKey, int> &admit_table()
{
    static std::map<AdmitKey, int> table;
    return table;
}

bool admit_kind(const char *name, AdmitKind &k)
{
    if (strcmp(name, "rowexact") == 0)
        k = AdmitKind::rowexact;
    else if (strcmp(name, "forward") == 0)
        k = AdmitKind::forward;
    else
        return false;
    return true;
}

int admission_of(AdmitKind k, int M, int K, int N, int bits, int G)
{
    std::lock_guard<std::mutex> lock(admit_mutex);
    const auto it = admit_table().find(std::make_tuple((int)k, K, N, M, bits, G));
    return it == admit_table().end() ? QMM_ADMISSION_UNKNOWN : it->second;
}

// ---------------------------------------------------------------------------
// Static scratch of qmm_forward_splitk_noalloc: the fp32 split-K partials of
// callers that cannot allocate device memory. Every device that loads the
// library holds its own copy until the process ends. In host code the
// array's name is only a host-side stand-in, never a device address: the
// device address is looked up once per device with hipGetSymbolAddress
// (scratch_on_device) and only that address reaches the kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[QMM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

std::atomic<float *> scratch_address[64];  // per device ordinal; null until looked up

// Device address of `scratch` on the current device. Racing first calls
// look it up twice and store the same value.
int scratch_on_device(float **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return QMM_ERR_LAUNCH;
    float *p = scratch_address[dev].load(std::memory_order_acquire);
    if (!p) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr)
            return QMM_ERR_LAUNCH;
        p = static_cast<float *>(addr);
        scratch_address[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return QMM_OK;
}

// The split-K product with `workspace` (at least split_k*M*N floats) holding
// the partials: one slice launch and the in-order reduction.
int splitk_into(const uint16_t *x, const uint32_t *wq, const uint16_t *scales, const uint16_t *biases,
                float *y, int M, int K, int N, int bits, int G, int split_k, float *workspace,
                hipStream_t stream)
{
    const Kernel kind = choose_kernel(M, K, N, bits, G, split_k);
    if (split_k == 1)
        return launch_product(kind, x, wq, scales, biases, y, M, K, N, bits, G, 1, stream);
    const int rc = launch_product(kind, x, wq, scales, biases, workspace, M, K, N, bits, G, split_k, stream);
    if (rc != QMM_OK)
        return rc;
    return qmm::launch_splitk_reduce(workspace, y, split_k, (size_t)M * N, stream) == hipSuccess
               ? QMM_OK
               : QMM_ERR_LAUNCH;
}

}  // namespace

namespace qmm {

int device_cu_count()
{
    static std::atomic<int> cached[64];  // zero until queried; racing queries store the same value
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace qmm

extern "C" {

const char *qmm_strerror(int code)
{
    switch (code) {
    case QMM_OK: return "success";
    case QMM_ERR_NULL: return "a required pointer is NULL";
    case QMM_ERR_SHAPE: return "bad shape: need M, K, N >= 1, K a multiple of G, sizes in range";
    case QMM_ERR_BITS: return "unsupported bit width (supported: 2, 3, 4, 5, 6, 8)";
    case QMM_ERR_GROUP: return "unsupported group size (supported: 32, 64, 128)";
    case QMM_ERR_SPLIT: return "bad split_k: need 1 <= split_k <= K/G";
    case QMM_ERR_WORKSPACE: return "workspace smaller than qmm_splitk_workspace_bytes(M, N, split_k)";
    case QMM_ERR_ALIGN: return "x, wq, scales, biases, y and workspace must be 16-byte aligned";
    case QMM_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case QMM_ERR_UNSUPPORTED: return "the requested kernel cannot run this shape";
    case QMM_ERR_SCRATCH: return "split_k * M * N * 4 bytes exceed the static scratch (QMM_NOALLOC_SCRATCH_BYTES)";
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
    return kernel_label(choose_kernel(M, K, N, bits, G, 1));
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
    return launch_product(choose_kernel(M, K, N, bits, G, 1), x, wq, scales, biases, y, M, K, N,
                          bits, G, 1, stream);
}

int qmm_forward_splitk(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                       const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                       int split_k, float *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const int rc = qmm_validate(x, wq, scales, biases, y, M, K, N, bits, G,
                                split_k < 1 ? -1 : split_k, workspace, workspace_bytes);
    if (rc != QMM_OK)
        return rc;
    return splitk_into(x, wq, scales, biases, y, M, K, N, bits, G, split_k, workspace, stream);
}

int qmm_forward_splitk_noalloc(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                               const uint16_t *biases, float *y, int M, int K, int N, int bits,
                               int G, int split_k, hipStream_t stream)
{
    int rc = qmm_validate(x, wq, scales, biases, y, M, K, N, bits, G, 0, nullptr, 0);
    if (rc != QMM_OK)
        return rc;
    if (split_k < 1 || split_k > K / G)
        return QMM_ERR_SPLIT;
    if (qmm_splitk_workspace_bytes(M, N, split_k) > (size_t)QMM_NOALLOC_SCRATCH_BYTES)
        return QMM_ERR_SCRATCH;
    float *ws = nullptr;
    if (split_k > 1) {
        rc = scratch_on_device(&ws);
        if (rc != QMM_OK)
            return rc;
    }
    return splitk_into(x, wq, scales, biases, y, M, K, N, bits, G, split_k, ws, stream);
}

int qmm_forward_rowexact(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                         const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                         hipStream_t stream)
{
    const int rc = qmm_validate(x, wq, scales, biases, y, M, K, N, bits, G, 0, nullptr, 0);
    if (rc != QMM_OK)
        return rc;
    if (M > 1 && admission_of(AdmitKind::rowexact, M, K, N, bits, G) == 0)
        return launch_rows_one_by_one(x, wq, scales, biases, y, M, K, N, bits, G, stream);
    return launch_product(Kernel::qmv, x, wq, scales, biases, y, M, K, N, bits, G, 1, stream);
}

size_t qmm_admit_workspace_bytes(int M, int N)
{
    if (M < 1 || N < 1 || M >= (1 << 30) || N >= (1 << 30))
        return 0;
    return 2 * (size_t)M * N * sizeof(float) + 16;
}

int qmm_admit(const char *kind, const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
              const uint16_t *biases, int M, int K, int N, int bits, int G, void *workspace,
              size_t workspace_bytes, hipStream_t stream, int *admitted)
{
    if (!kind || !admitted || !workspace)
        return QMM_ERR_NULL;
    AdmitKind k;
    if (!admit_kind(kind, k))
        return QMM_ERR_SHAPE;
    // y is checked as the workspace (both results live there)
    const int rc = qmm_validate(x, wq, scales, biases, workspace, M, K, N, bits, G, 0, nullptr, 0);
    if (rc != QMM_OK)
        return rc;
    if (workspace_bytes < qmm_admit_workspace_bytes(M, N))
        return QMM_ERR_WORKSPACE;
    float *cand = static_cast<float *>(workspace);
    float *orig = cand + (size_t)M * N;
    uint32_t *count = reinterpret_cast<uint32_t *>(orig + (size_t)M * N);
    int lrc = k == AdmitKind::rowexact
                  ? launch_product(Kernel::qmv, x, wq, scales, biases, cand, M, K, N, bits, G, 1, stream)
                  : launch_product(choose_kernel(M, K, N, bits, G, 1), x, wq, scales, biases, cand, M, K, N,
                                   bits, G, 1, stream);
    if (lrc != QMM_OK)
        return lrc;
    lrc = launch_rows_one_by_one(x, wq, scales, biases, orig, M, K, N, bits, G, stream);
    if (lrc != QMM_OK)
        return lrc;
    if (qmm::launch_compare_words(reinterpret_cast<const uint32_t *>(cand), reinterpret_cast<const uint32_t *>(orig),
                                  (size_t)M * N, count, stream) != hipSuccess)
        return QMM_ERR_LAUNCH;
    uint32_t mismatches = 0;
    if (hipMemcpyAsync(&mismatches, count, sizeof(mismatches), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return QMM_ERR_LAUNCH;
    *admitted = mismatches == 0 ? 1 : 0;
    std::lock_guard<std::mutex> lock(admit_mutex);
    admit_table()[std::make_tuple((int)k, K, N, M, bits, G)] = *admitted;
    return QMM_OK;
}

int qmm_admission(const char *kind, int M, int K, int N, int bits, int G)
{
    if (!kind)
        return QMM_ERR_NULL;
    AdmitKind k;
    if (!admit_kind(kind, k))
        return QMM_ERR_SHAPE;
    return admission_of(k, M, K, N, bits, G);
}

void qmm_admission_clear(void)
{
    std::lock_guard<std::mutex> lock(admit_mutex);
    admit_table().clear();
}

int qmm_forward_bf16(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                     const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                     hipStream_t stream)
{
    const int rc = qmm_validate(x, wq, scales, biases, y, M, K, N, bits, G, 0, nullptr, 0);
    if (rc != QMM_OK)
        return rc;
    // qmm_forward's kernel choice
    const Kernel kind = choose_kernel(M, K, N, bits, G, 1);
    const int step = kind == Kernel::qmv ? kQmvRowsPerLaunch : kMaxRowsPerLaunch;
    const qmm::ProductArgs full = product_args(x, wq, scales, biases, y, M, K, N, 1);
    for (int m0 = 0; m0 < M; m0 += step) {
        const qmm::ProductArgs a = qmm::rows_of(full, m0, M - m0 < step ? M - m0 : step);
        const hipError_t e = kind == Kernel::qmv    ? qmm::launch_qmv(a, bits, G, true, stream)
                             : kind == Kernel::mfma ? qmm::launch_mfma_xr(a, bits, G, true, stream)
                                                    : qmm::launch_mfma(a, bits, G, true, stream);
        if (e != hipSuccess)
            return QMM_ERR_LAUNCH;
    }
    return QMM_OK;
}

int qmm_forward_fused(const uint16_t *x, int count, const uint32_t *const *wq,
                      const uint16_t *const *scales, const uint16_t *const *biases, float *const *y,
                      const int *N, int M, int K, int bits, int G, hipStream_t stream)
{
    if (!x || !wq || !scales || !biases || !y || !N)
        return QMM_ERR_NULL;
    if (count < 1 || count > QMM_MAX_FUSED)
        return QMM_ERR_SHAPE;
    qmm::ProductArgs a = product_args(x, nullptr, nullptr, nullptr, nullptr, M, K, 0, 1);
    a.nproj = count;
    int tiles = 0;
    for (int p = 0; p < count; ++p) {
        const int rc = qmm_validate(x, wq[p], scales[p], biases[p], y[p], M, K, N[p], bits, G, 0,
                                    nullptr, 0);
        if (rc != QMM_OK)
            return rc;
        a.tile0[p] = tiles;
        a.proj[p] = qmm::Proj{wq[p], scales[p], biases[p], y[p], N[p]};
        tiles += (N[p] + 15) / 16;
        if (tiles >= (1 << 26))
            return QMM_ERR_SHAPE;
    }
    a.tile0[count] = tiles;
    if (count == 1)  // the plain single-projection launch
        return launch_product(choose_kernel(M, K, N[0], bits, G, 1), x, wq[0], scales[0], biases[0],
                              y[0], M, K, N[0], bits, G, 1, stream);
    a.N = 16 * tiles;  // the launch's row space: every projection padded to whole tiles
    return launch_args(choose_kernel(M, K, a.N, bits, G, 1), a, bits, G, stream);
}

// Layouts the tiled form exists for (the repack); the product additionally
// needs K parts that fit the kernel (qmm::tiled_supported).
static bool tiled_layout_ok(int N, int K, int bits, int G)
{
    return (bits == 2 || bits == 4 || bits == 8) && group_supported(G) && N >= 1 && K >= G &&
           K % (4 * G) == 0 && ((int64_t)K * bits) % 512 == 0 && (int64_t)K * bits < ((int64_t)1 << 31) &&
           N < (1 << 30);
}

size_t qmm_tiled_bytes(int N, int K, int bits, int G, size_t *sb_bytes)
{
    if (sb_bytes)
        *sb_bytes = 0;
    if (!tiled_layout_ok(N, K, bits, G))
        return 0;
    const size_t rows = ((size_t)N + 15) / 16 * 16;
    if (sb_bytes)
        *sb_bytes = rows * (size_t)(K / G) * 4;
    return rows * (size_t)K * bits / 8;
}

int qmm_repack_tiled(const uint32_t *wq, const uint16_t *scales, const uint16_t *biases,
                     uint8_t *tiled_w, uint32_t *tiled_sb, int N, int K, int bits, int G,
                     hipStream_t stream)
{
    if (!wq || !scales || !biases || !tiled_w || !tiled_sb)
        return QMM_ERR_NULL;
    const int rc = check_shape(1, K, N, bits, G);
    if (rc != QMM_OK)
        return rc;
    if (!tiled_layout_ok(N, K, bits, G))
        return QMM_ERR_UNSUPPORTED;
    if (!aligned16(wq) || !aligned16(scales) || !aligned16(biases) || !aligned16(tiled_w) ||
        !aligned16(tiled_sb))
        return QMM_ERR_ALIGN;
    return qmm::launch_repack_tiled(wq, scales, biases, tiled_w, tiled_sb, N, K, bits, G, stream) ==
                   hipSuccess
               ? QMM_OK
               : QMM_ERR_LAUNCH;
}

int qmm_forward_tiled(const uint16_t *x, const uint8_t *tiled_w, const uint32_t *tiled_sb, float *y,
                      int M, int K, int N, int bits, int G, hipStream_t stream)
{
    if (!x || !tiled_w || !tiled_sb || !y)
        return QMM_ERR_NULL;
    const int rc = check_shape(M, K, N, bits, G);
    if (rc != QMM_OK)
        return rc;
    if (!aligned16(x) || !aligned16(tiled_w) || !aligned16(tiled_sb) || !aligned16(y))
        return QMM_ERR_ALIGN;
    qmm::ProductArgs a = product_args(x, reinterpret_cast<const uint32_t *>(tiled_w),
                                      reinterpret_cast<const uint16_t *>(tiled_sb), nullptr, y, M, K,
                                      N, 1);
    if (!tiled_layout_ok(N, K, bits, G) || !qmm::tiled_supported(a, bits, G))
        return QMM_ERR_UNSUPPORTED;
    for (int m0 = 0; m0 < M; m0 += kMaxRowsPerLaunch) {
        const qmm::ProductArgs b = qmm::rows_of(a, m0, M - m0 < kMaxRowsPerLaunch ? M - m0 : kMaxRowsPerLaunch);
        if (qmm::launch_mfma_tiled(b, bits, G, stream) != hipSuccess)
            return QMM_ERR_LAUNCH;
    }
    return QMM_OK;
}

size_t qmm_stream_read_sink_words(size_t bytes)
{
    return bytes == 0 || bytes % 16 != 0 ? 0 : qmm::stream_read_sink_words(bytes);
}

int qmm_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (!src || !sink)
        return QMM_ERR_NULL;
    if (bytes == 0 || bytes % 16 != 0 || qmm::stream_read_sink_words(bytes) > 0x7FFFFFFFu)
        return QMM_ERR_SHAPE;
    if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return QMM_ERR_ALIGN;
    return qmm::launch_stream_read(src, bytes, sink, stream) == hipSuccess ? QMM_OK : QMM_ERR_LAUNCH;
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
    else if (strcmp(kernel, "mfma_lds") == 0)
        kind = Kernel::mfma_lds;
    else
        return QMM_ERR_SHAPE;
    return launch_product(kind, x, wq, scales, biases, y, M, K, N, bits, G, 1, stream);
}

}  // extern "C"
