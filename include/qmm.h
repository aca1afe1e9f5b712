/*
 * qmm.h - affine group-quantized matrix product for AMD Instinct MI355X (gfx950).
 *
 * Computes y[M,N] = x[M,K] . W[N,K]^T where W is stored as packed b-bit
 * unsigned codes q with one fp16 scale s and one fp16 bias b per group of G
 * consecutive codes along K:
 *
 *     W[n,k] = s[n, k/G] * q[n,k] + b[n, k/G]
 *
 * The library never forms W. It evaluates the factored form
 *
 *     y[m,n] = sum over groups g of  s[n,g] * P[m,n,g] + b[n,g] * XS[m,g]
 *     P[m,n,g] = sum_{k in g} q[n,k] * x[m,k],   XS[m,g] = sum_{k in g} x[m,k]
 *
 * with the dequantization applied after the dot product, as described in the
 * vmlx-swift pull request #565 page, commit "LaneQMM" (tensor-op matmul over
 * raw affine codes, C += s*P + b*XS, 5/6/8-bit codes widened on the GPU).
 * Products of exact fp16 codes and fp16 activations are accumulated in fp32;
 * the result is fp32 (the same page's "batched GDN tail" commit notes the
 * float32 promotion of batched quantized-matmul output).
 *
 * Data layout (all row-major, all device memory):
 *   x       fp16 [M, K]            IEEE binary16 bit patterns (uint16_t)
 *   wq      uint32 [N, K*bits/32]  row n holds one least-significant-bit-
 *                                  first bitstream of K codes: code k occupies
 *                                  stream bits k*bits .. k*bits+bits-1, stream
 *                                  bit t is bit (t mod 32) of word t/32.
 *   scales  fp16 [N, K/G]
 *   biases  fp16 [N, K/G]
 *   y       fp32 [M, N]            overwritten, never accumulated into
 *
 * Supported: bits in {2, 3, 4, 5, 6, 8} (the 2/4/8-bit formats consumed as
 * stored in the "Qwen3.8 Flash Next performance and parity receipt" page,
 * section "MTPLX logic review", the 5/6-bit widths of the "LaneQMM" commit of
 * the vmlx-swift pull request #565 page, and 3 bits between them);
 * G in {32, 64, 128}; K a positive multiple of G; N >= 1; M >= 1 (tuned for
 * M = 1..16 verify rows; larger M is processed 16 rows at a time).
 *
 * Ownership: the caller owns every buffer. Functions without a workspace
 * argument need no scratch memory, except qmm_forward_splitk_noalloc, which
 * uses a static array of the library (QMM_NOALLOC_SCRATCH_BYTES per GPU,
 * held from module load to process end); no entry point allocates device
 * memory. Work is enqueued on the caller's stream and the call returns
 * without waiting; results are visible after the stream is synchronized.
 *
 * Errors: every entry point validates its arguments on the host before any
 * GPU work and returns 0 on success or one of the negative codes below.
 * Argument errors launch nothing. A launch failure reported by the HIP
 * runtime returns QMM_ERR_LAUNCH; execution faults surface at stream
 * synchronization as with any HIP kernel. No exception or abort crosses
 * this interface. The library keeps no state between calls other than
 * cached device properties and the per-GPU address of that static array; it
 * may be called from several host threads at once (with the caveat on
 * qmm_forward_splitk_noalloc's shared scratch).
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMM_OK 0
#define QMM_ERR_NULL (-1)          /* a required pointer is NULL */
#define QMM_ERR_SHAPE (-2)         /* M < 1, K < 1, N < 1, K % G != 0 or a size overflows */
#define QMM_ERR_BITS (-3)          /* bits not in {2, 3, 4, 5, 6, 8} */
#define QMM_ERR_GROUP (-4)         /* G not in {32, 64, 128} */
#define QMM_ERR_SPLIT (-5)         /* split_k < 1 or split_k > K/G */
#define QMM_ERR_WORKSPACE (-6)     /* workspace smaller than qmm_splitk_workspace_bytes */
#define QMM_ERR_ALIGN (-7)         /* x, wq, scales, biases, y or workspace not 16-byte aligned */
#define QMM_ERR_LAUNCH (-8)        /* the HIP runtime rejected a kernel launch */
#define QMM_ERR_UNSUPPORTED (-9)   /* qmm_forward_kernel: that kernel cannot run this shape */
#define QMM_ERR_SCRATCH (-10)      /* qmm_forward_splitk_noalloc: partials exceed the static scratch */

/*
 * qmm_pack - pack unpacked codes into the bitstream layout above.
 *
 * The pages' quantized tensors are packed once and then consumed in their
 * stored form by every product ("Qwen3.8 Flash Next performance and parity
 * receipt" page, section "MTPLX logic review": its 4-bit group-32 and
 * group-64, 8-bit and 2-bit tensors are used in their stored form, neither
 * up-converted nor re-quantized). This is that one-time packing step, into
 * the layout defined at the top of this header, which every entry point then
 * reads as is.
 *
 * codes  [N, K] uint8, device memory; only the low `bits` bits of each byte
 *        are stored (higher bits are ignored).
 * packed [N, K*bits/32] uint32, device memory, 16-byte aligned, written in
 *        full. The caller owns both buffers.
 * Requires K*bits to be a multiple of 32 (true whenever 32 divides K).
 * Bit-exact with respect to the layout definition. Errors: QMM_ERR_NULL,
 * QMM_ERR_BITS, QMM_ERR_SHAPE (N < 1, K < 1, K*bits not a multiple of 32),
 * QMM_ERR_ALIGN, QMM_ERR_LAUNCH. Async on `stream`.
 */
int qmm_pack(const uint8_t *codes, uint32_t *packed, int N, int K, int bits,
             hipStream_t stream);

/*
 * qmm_forward - y = x . W^T for the packed affine weights (one call, one
 * or more kernel launches on `stream`, no scratch memory).
 *
 * x [M,K] fp16, wq [N, K*bits/32] uint32, scales/biases [N, K/G] fp16,
 * y [M,N] fp32; all device pointers, 16-byte aligned.
 * The kernel is chosen on the host from (M, bits, G, K, N): a
 * mat-vec kernel for one and two rows and a multi-row matrix-core kernel
 * that streams the weights once for all rows otherwise (the vmlx-swift pull
 * request #565 page, tiling-policy commit, routes fewer than four rows to
 * the one-row mat-vec because it is faster there; here the matrix cores win
 * from three rows on). When K is too long for one pass of the matrix-core
 * kernel, or N so small that one launch would leave half the CUs idle, a
 * first launch clears y and the two K halves then add into it with fp32
 * atomics: each output receives exactly two addends on +0, and their sum
 * does not depend on arrival order, so reruns stay bitwise identical (for
 * small N the halves are used only where they give the bits of the one-slice
 * launch). y must not alias the inputs.
 */
int qmm_forward(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                hipStream_t stream);

/*
 * qmm_forward_splitk - the same product with K divided into split_k slices.
 *
 * Slices are whole groups: with Kg = K/G groups, slice z covers
 * floor(Kg/split_k) groups plus one more for z < Kg mod split_k, in
 * ascending order. A first kernel writes slice z's fp32 partial product to
 * workspace[z][M][N]; a second kernel sums the split_k partials in order
 * z = 0 .. split_k-1 into y. There are no atomics: reruns are bitwise
 * identical. The summation order differs from qmm_forward, so the two
 * agree within the fp32 tolerance, not bitwise. This follows the split-K
 * verify tile of the vmlx-swift pull request #565 page (JANGH dense verify
 * split-K commit: K sliced across the grid, fp32 partials summed after).
 *
 * 1 <= split_k <= K/G. workspace: device memory of at least
 * qmm_splitk_workspace_bytes(M, N, split_k) bytes, 16-byte aligned, owned by
 * the caller; its contents on entry do not matter and are overwritten.
 * With split_k == 1 the product is written to y directly, no workspace is
 * needed and `workspace` may be NULL.
 */
int qmm_forward_splitk(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                       const uint16_t *biases, float *y, int M, int K, int N, int bits,
                       int G, int split_k, float *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * qmm_forward_splitk_noalloc - qmm_forward_splitk for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the fp32 partials go to a static scratch
 * array inside the library instead of a caller workspace.
 *
 * Arguments, layout, slices, kernels and results are those of
 * qmm_forward_splitk (bitwise equal to it for the same arguments), without
 * the workspace arguments. The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine. Requires
 * split_k * M * N * 4 <= QMM_NOALLOC_SCRATCH_BYTES, else QMM_ERR_SCRATCH
 * (checked on the host, nothing is launched); split_k == 1 uses no scratch.
 *
 * The scratch is one array per GPU, kept until the process ends; its device
 * address is looked up on the first call on each device. Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (several streams or
 * host threads without ordering between them) race on it and must be
 * serialized by the caller. Each call overwrites every partial it reads, so
 * nothing needs clearing between calls. Errors as qmm_forward_splitk, plus
 * QMM_ERR_SCRATCH; QMM_ERR_LAUNCH if the scratch address cannot be found.
 */
#define QMM_NOALLOC_SCRATCH_BYTES (16u << 20)  /* 16 MiB per GPU */
int qmm_forward_splitk_noalloc(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                               const uint16_t *biases, float *y, int M, int K, int N, int bits,
                               int G, int split_k, hipStream_t stream);

/* Row-exact product (vmlx-swift pull request #565 page, commit introducing
 * qwen_qmv_rows_full: every verify row keeps the one-row kernel's statement
 * order, so a multi-row call reproduces the one-row results bit for bit).
 * Same arguments, layout, ownership and errors as qmm_forward; every row m of
 * y is bitwise equal to qmm_forward on row m alone (M = 1) with the same K,
 * N, bits and G. Runs the one-row VALU kernel on up to 8 rows per launch
 * (the weights are read once per 8 rows). Async on `stream`. */
int qmm_forward_rowexact(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                         const uint16_t *biases, float *y, int M, int K, int N, int bits,
                         int G, hipStream_t stream);

/* Bitwise admission of a multi-row kernel (the same commit of the
 * vmlx-swift pull request #565 page: a (kind, K, N, rows) is used only after
 * its output matched the caller's original one-row kernel bit for bit on the
 * real weights, and a mismatch keeps the original kernel).
 *
 * qmm_admit runs the candidate `kind` on x [M,K] and the caller's weights,
 * runs the original (M launches of the one-row kernel, one row each) on the
 * same inputs, compares the two fp32 results word for word on the GPU, waits
 * for the stream and records the verdict for (kind, K, N, M, bits, G) in a
 * table of the library (per process, shared by every device and thread).
 * kind: "rowexact" (the multi-row launches of qmm_forward_rowexact) or
 * "forward" (the kernel qmm_forward chooses for M rows). *admitted receives
 * 1 (bitwise equal) or 0. workspace: device memory of at least
 * qmm_admit_workspace_bytes(M, N) bytes, 16-byte aligned, caller-owned, used
 * for both results and the mismatch count. Other arguments as qmm_forward.
 * Errors: those of qmm_forward, QMM_ERR_NULL (kind, admitted or workspace
 * NULL), QMM_ERR_SHAPE (unknown kind), QMM_ERR_WORKSPACE, QMM_ERR_LAUNCH (a
 * launch, the copy of the count or the wait failed; nothing is recorded).
 * Synchronous: it returns after `stream` has drained, so it is not for graph
 * capture; admission is done once per shape, before the serving loop.
 *
 * qmm_forward_rowexact keeps its multi-row launches for a (K, N, M, bits, G)
 * that is admitted or was never examined (the kernel is bitwise by
 * construction) and falls back to one one-row launch per row when "rowexact"
 * was rejected for it.
 *
 * qmm_admission: the recorded verdict, 1 admitted, 0 rejected, 2 never
 * examined; QMM_ERR_NULL / QMM_ERR_SHAPE for a NULL or unknown kind.
 * qmm_admission_clear forgets every verdict. Both are host-only. */
#define QMM_ADMISSION_UNKNOWN 2
size_t qmm_admit_workspace_bytes(int M, int N);
int qmm_admit(const char *kind, const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
              const uint16_t *biases, int M, int K, int N, int bits, int G, void *workspace,
              size_t workspace_bytes, hipStream_t stream, int *admitted);
int qmm_admission(const char *kind, int M, int K, int N, int bits, int G);
void qmm_admission_clear(void);

/* bf16 variant (the pages' kernels take bf16 as well as fp16 activations
 * and scales: vmlx-swift pull request #565 page, the split-K verify commit's
 * fp16/bf16 tests and the bf16-activation affine mat-vec of the tiling-policy
 * commit). Same as qmm_forward except that x [M,K], scales and biases [N,K/G]
 * hold bfloat16 bit patterns (uint16_t: the upper half of an IEEE binary32);
 * y is fp32. Codes are widened to exact bf16 integers and contracted with the
 * activations in fp32 (v_dot2_f32_bf16 or v_mfma_f32_16x16x32_bf16), on the
 * kernel qmm_forward takes for the same shape and row count (each kernel has
 * a bf16 mode). Results meet the same tolerance as qmm_forward; rows of
 * a one- or two-row call are bitwise equal to one-row calls. Same layout,
 * alignment, ownership and error codes as qmm_forward. */
int qmm_forward_bf16(const uint16_t *x, const uint32_t *wq, const uint16_t *scales,
                     const uint16_t *biases, float *y, int M, int K, int N, int bits, int G,
                     hipStream_t stream);

/*
 * qmm_forward_fused - several projections of the same activations in one
 * launch: y_p = x . W_p^T for p < count (count <= QMM_MAX_FUSED).
 *
 * The "Qwen3.8 Flash Next performance and parity receipt" page runs the gate
 * and up projections of a layer as one merged projection (section "MTPLX
 * logic review") and promotes the exact fused projection ("A/B evidence"); fusing q/k/v or gate/up
 * also fills the GPU when a single projection has few output rows.
 *
 * x          [M, K] fp16, shared by every projection.
 * wq, scales, biases, y, N: host arrays of `count` entries; entry p holds
 *            the device pointers and the output-row count of projection p,
 *            with the layouts and alignment of qmm_forward (y[p] is
 *            [M, N[p]] fp32, overwritten).
 * M, K, bits, G are common to all projections. The kernel is the one
 * qmm_forward picks for (M, K, bits, G); each y[p] is bitwise equal to the
 * qmm_forward result for projection p alone. Errors: those of qmm_forward for
 * any projection, QMM_ERR_NULL for a NULL array, QMM_ERR_SHAPE for count out
 * of range. The host arrays are read during the call only. Async on `stream`.
 */
#define QMM_MAX_FUSED 4
int qmm_forward_fused(const uint16_t *x, int count, const uint32_t *const *wq,
                      const uint16_t *const *scales, const uint16_t *const *biases,
                      float *const *y, const int *N, int M, int K, int bits, int G,
                      hipStream_t stream);

/*
 * Tiled (MFMA-native) weight layout: an optional offline re-layout of the
 * packed weights for the multi-row matrix-core path. The vmlx-swift pull
 * request #565 page tiles the weights of its lane matmul modules (commit
 * "LaneQMM", "Tiling policy") and keeps the packed layout for the readers
 * that consume it directly; here too the tiled copy is read only by
 * qmm_forward_tiled, and qmm_forward keeps reading the packed layout.
 *
 * Layout, for bits in {2, 4, 8}, G in {32, 64, 128}, K a multiple of 4*G with
 * K*bits a multiple of 512; rows grouped in 16-row tiles (N padded with zero
 * rows). Lane L = 16c + i (c = 0..3, i = 0..15) of tile t owns the bit stream
 * made of chunk c of every group of row 16t + i, in group order, where chunk
 * c of a group is its codes c*G/4 .. c*G/4 + G/4 - 1 in the packed bit order;
 * the stream is cut into 16-byte units and unit u of lane L of tile t is
 * stored at byte ((t*UB + u)*64 + L)*16 of tiled_w, UB = K*bits/512.
 * tiled_sb holds uint32 words (scale | bias << 16) (fp16 bit patterns): row
 * 16t + i, group g at word ((t*(K/G)/4 + g/4)*16 + i)*4 + g%4.
 *
 * qmm_tiled_bytes: bytes of tiled_w, and of tiled_sb in *sb_bytes (if not
 * NULL); 0 (and 0) when the layout does not exist for (N, K, bits, G).
 * qmm_repack_tiled: writes both from the packed wq, scales, biases (device
 * memory, caller-owned, 16-byte aligned); QMM_ERR_UNSUPPORTED when the layout
 * does not exist for the shape. Async on `stream`.
 * qmm_forward_tiled: y[M,N] = x . W^T from the tiled form; the arguments
 * mean what they mean for qmm_forward. It runs the multi-row matrix-core
 * kernel for every M (16 rows per launch); QMM_ERR_UNSUPPORTED when K is
 * too long for it (more than 8 parts of 768 activations, 512 for 8 bits).
 */
size_t qmm_tiled_bytes(int N, int K, int bits, int G, size_t *sb_bytes);
int qmm_repack_tiled(const uint32_t *wq, const uint16_t *scales, const uint16_t *biases,
                     uint8_t *tiled_w, uint32_t *tiled_sb, int N, int K, int bits, int G,
                     hipStream_t stream);
int qmm_forward_tiled(const uint16_t *x, const uint8_t *tiled_w, const uint32_t *tiled_sb,
                      float *y, int M, int K, int N, int bits, int G, hipStream_t stream);

/* Bytes of workspace qmm_forward_splitk needs: split_k * M * N * 4 for
 * split_k >= 2, 0 for split_k == 1 and for invalid arguments. */
size_t qmm_splitk_workspace_bytes(int M, int N, int split_k);

/* Host-only validation of qmm_forward / qmm_forward_splitk arguments
 * (split_k = 0 validates a qmm_forward call). Returns the code the entry
 * point would return before launching anything. Touches no GPU state. */
int qmm_validate(const void *x, const void *wq, const void *scales, const void *biases,
                 const void *y, int M, int K, int N, int bits, int G, int split_k,
                 const void *workspace, size_t workspace_bytes);

/* Static description of an error code (never NULL). */
const char *qmm_strerror(int code);

/* Name of the kernel qmm_forward would launch for these arguments
 * ("qmv", "mfma" or "mfma_lds", see qmm_forward_kernel) or NULL for invalid
 * ones. Host-only. */
const char *qmm_kernel_name(int M, int K, int N, int bits, int G);

/* qmm_forward with the kernel named explicitly instead of chosen from M
 * (a test and benchmark aid):
 *   "qmv"      the row-exact VALU kernel (qmm_forward_rowexact), up to 8
 *              rows per launch; qmm_forward's choice for M <= 2;
 *   "mfma"     the multi-row matrix-core kernel with each wave's K part of
 *              the activations in registers; qmm_forward's choice for M >= 3
 *              when the shape allows it (K * bits a multiple of 128, and K
 *              within 8 parts of 768 activations (640 for 8-bit codes) or,
 *              for longer K, within 8 passes of 8 parts of 640, each wave
 *              walking its parts one after the other); QMM_ERR_UNSUPPORTED
 *              otherwise;
 *   "mfma_lds" the multi-row matrix-core kernel that streams activations
 *              through LDS; any shape except 3-bit codes at G = 32
 *              (QMM_ERR_UNSUPPORTED); qmm_forward's choice for M >= 3 when
 *              "mfma" does not apply (and "qmv" when neither does).
 * Same arguments, layout and errors as qmm_forward; an unknown name returns
 * QMM_ERR_SHAPE, a NULL name QMM_ERR_NULL. */
int qmm_forward_kernel(const char *kernel, const uint16_t *x, const uint32_t *wq,
                       const uint16_t *scales, const uint16_t *biases, float *y, int M,
                       int K, int N, int bits, int G, hipStream_t stream);

/* Streaming-read ceiling (a measurement aid, not part of the product): reads
 * the `bytes` bytes at `src` once, with the 16-byte non-temporal loads the
 * product kernels use for packed codes, every load of a thread issued before
 * any is used, and writes one word per workgroup to `sink`: the XOR of the
 * 32-bit words that workgroup read (workgroup w reads the 8 KiB span
 * starting at byte w * 8192; the last span may be short). Its time bounds
 * what any kernel that must read those bytes can reach on this GPU, which is
 * how the one-row product's weight stream is judged (it reads each weight
 * byte once and writes almost nothing).
 *   src   device memory, 16-byte aligned; bytes a positive multiple of 16;
 *   sink  device memory of qmm_stream_read_sink_words(bytes) uint32 words,
 *         4-byte aligned, overwritten.
 * Errors: QMM_ERR_NULL, QMM_ERR_SHAPE (bytes 0 or not a multiple of 16),
 * QMM_ERR_ALIGN, QMM_ERR_LAUNCH. Async on `stream`.
 * qmm_stream_read_sink_words: the sink's length in words; 0 for an invalid
 * byte count. Host-only. */
size_t qmm_stream_read_sink_words(size_t bytes);
int qmm_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
