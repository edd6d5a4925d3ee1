/*
 * s3d8.h -- C ABI of libs3d8: the S3D8 weight-decode-fused linear layer on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page and section):
 *   [BLOG]  "11 billion parameters on a phone" (Graphcore Research blog):
 *           "S3D8: a 2.7-bit weight format for fast decoding", "Bit layout",
 *           "Output channel packing", "Fused matrix-vector product",
 *           "Fast? How fast?".
 *   [PAPER] "Llama-Mobile: Efficient 2.7-Bit Quantization of VLMs" (arXiv),
 *           Sec. 3.4 "The S3D8 Format" (Eq. 1 and the "Quantization"
 *           equations), Sec. 4 and Sec. 4.3, Appendix A.3.
 *
 * Format (canonical layout, used by every entry point):
 *   A weight matrix W has N output channels and K input columns (Y = X W^T,
 *   [PAPER] Sec. 4.3).  Channels are grouped in triples t = 0 .. T-1 with
 *   T = ceil(N/3); the channel count is padded to Npad = 3T ([PAPER] Sec. 3.4
 *   after Eq. 1).  Three buffers describe the matrix:
 *     centroids   uint8 [32][3], row-major: the absolute-value centroid table
 *                 C, integers in [0,127] ([BLOG] "S3D8"; [PAPER] Eq. 1).
 *     scales      uint16 [Npad]: bfloat16 bit patterns of the channel scales
 *                 alpha_i = max_j |W_ij| / 127 ([PAPER] "Quantization");
 *                 padded channels hold 0.
 *     packed      uint8 [T][K], row-major, K-contiguous per triple: byte
 *                 (t, j) holds channels 3t, 3t+1, 3t+2 at input column j
 *                 ([BLOG] "Output channel packing").  Its bits, from bit 7 to
 *                 bit 0, are [S2 xor S0, S1, Q4..Q0, S0] ([BLOG] "Bit
 *                 layout"): Q is the shared centroid index, S_d = 1 selects
 *                 the negative value for channel 3t+d.
 *   Decoded weight ([PAPER] Eq. 1):  W~_ij = alpha_i * s_ij * C[q][i mod 3]
 *   where q is the index of byte (floor(i/3), j) and s_ij = -1 if S_{i mod 3}
 *   is set, else +1.  The channel-INT8 weight w_ij = s_ij * C[q][i mod 3]
 *   lies in [-127, 127].
 *
 * Activations: per-token ("channel-scaled") INT8 ([PAPER] Sec. 4, A.3).  For
 *   row m of X: s_m = max_j |x_mj| / 127 (IEEE fp32 division), and
 *   xq_mj = clamp(round_half_even(x_mj / s_m), -127, 127); an all-zero row has
 *   s_m = 0 and xq = 0.
 *
 * Linear ([BLOG] "Fused matrix-vector product"):
 *   acc_mn = sum_j xq_mj * w_nj (exact INT32),
 *   y_mn   = (s_m * float(acc_mn)) * float(alpha_n)   (fp32, left to right).
 *
 * Conventions for every entry point:
 *   - Status codes: S3D8_OK (0) on success, a positive S3D8_ERR_* otherwise.
 *     s3d8_last_error() returns a message for the calling thread's most
 *     recent failure.  No C++ exception crosses the ABI.
 *   - All arguments are validated on the host before any GPU work is
 *     queued; a failed validation queues nothing.
 *   - Sizes are int64_t element counts.  K must be a positive multiple of 16
 *     (the blog's fused loop also steps 16 columns); M, N positive.
 *   - The caller allocates and owns every buffer.  The library keeps no
 *     pointer after a call returns.
 *   - Device entry points take device pointers (e.g. torch tensors'
 *     data_ptr()) and a hipStream_t passed as `void *` (NULL = the default
 *     stream).  They only enqueue work and return; results are ready when
 *     the stream is synchronised.  A fault inside a kernel surfaces at that
 *     synchronisation, not in the return code.
 *   - Pointers marked "16-B aligned" must be multiples of 16 bytes.
 */
#ifndef S3D8_H
#define S3D8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define S3D8_OK 0
#define S3D8_ERR_INVALID_ARG 1 /* null pointer, non-positive size, bad option   */
#define S3D8_ERR_SHAPE 2       /* K not a multiple of 16, or a size too large   */
#define S3D8_ERR_ALIGN 3       /* a pointer that must be 16-B aligned is not    */
#define S3D8_ERR_HIP 4         /* the HIP runtime reported an error             */
#define S3D8_ERR_NOMEM 5       /* host allocation failed                        */
#define S3D8_ERR_DEVICE 6      /* the current device is not a gfx950 GPU        */

/* ABI version of this header (major * 10000 + minor * 100 + patch). */
int32_t s3d8_version(void);

/* T = ceil(N/3), the number of channel triples ([PAPER] Eq. 1: q has
 * ceil(n/3) rows).  Returns -1 if N <= 0. */
int64_t s3d8_num_triples(int64_t N);

/* Bytes of the packed index/sign matrix: ceil(N/3) * K, the ceil(n/3) rows
 * of k bytes that [PAPER] Eq. 1 indexes (one byte per channel triple and
 * input column, [BLOG] "Output channel packing").  -1 on bad sizes. */
int64_t s3d8_packed_bytes(int64_t N, int64_t K);

/* Total storage of one matrix: packed bytes + 2 * 3*ceil(N/3) scale bytes +
 * 96 table bytes, i.e. about (8/3 + 16/K) bits per weight ([PAPER] Sec. 3.4).
 * -1 on bad sizes. */
int64_t s3d8_format_bytes(int64_t N, int64_t K);

/* Message describing the calling thread's most recent failed call (empty
 * string if none).  The pointer stays valid until the thread's next call. */
const char *s3d8_last_error(void);

/* ------------------------------------------------------------------ host */

/* Fit the centroid table and encode a matrix ([PAPER] Sec. 3.4
 * "Quantization"): alpha = bf16(max|W_i|/127), W' = |W|/alpha grouped into
 * 3-vectors (padded channels 0), k-means++ seeding then Lloyd-Max
 * iterations on all vectors, C = round-half-even(centres) clamped to
 * [0,127], then the frozen-centroid encode of s3d8_encode.
 *   W            host fp32 [N][K], row-major, finite values.
 *   seed         seed of the k-means++ draws (SplitMix64, counter form).
 *   max_iters    Lloyd iteration limit (>= 0); the fit also stops when no
 *                assignment changes.
 *   num_threads  host threads (0 = all hardware threads).  The result does
 *                not depend on it.
 *   centroids    out, host uint8 [32][3].
 *   scales_bf16  out, host uint16 [3*ceil(N/3)].
 *   packed       out, host uint8 [ceil(N/3)][K].
 *   distortion   optional out (NULL to skip), host double [max_iters + 1]:
 *                sum of squared distances of the vectors to their nearest
 *                centre after seeding (index 0) and after each iteration.
 *   iterations   optional out (NULL to skip): Lloyd iterations run.
 * Synchronous; touches no GPU.  Errors: INVALID_ARG, SHAPE, NOMEM. */
int32_t s3d8_pack(const float *W, int64_t N, int64_t K, uint64_t seed, int32_t max_iters,
                  int32_t num_threads, uint8_t *centroids, uint16_t *scales_bf16,
                  uint8_t *packed, double *distortion, int32_t *iterations);

/* Frozen-centroid quantiser ([PAPER] Sec. 3.4, QAT phase; also the
 * "direct cast" of the blog's QAT section): alpha as in s3d8_pack,
 * s_ij = +1 if W_ij >= 0 else -1 (so -0.0 is positive), q = the index of
 * the nearest centroid row to the scaled-absolute 3-vector in fp64, lowest
 * index on ties; bytes per the [BLOG] bit layout; padded channels have
 * alpha 0, value 0 and sign selector 0.
 *   W            host fp32 [N][K].
 *   centroids    host uint8 [32][3], every entry in [0,127].
 *   scales_bf16  out, host uint16 [3*ceil(N/3)].
 *   packed       out, host uint8 [ceil(N/3)][K].
 * Synchronous; touches no GPU.  Errors: INVALID_ARG, SHAPE. */
int32_t s3d8_encode(const float *W, int64_t N, int64_t K, const uint8_t *centroids,
                    int32_t num_threads, uint16_t *scales_bf16, uint8_t *packed);

/* ---------------------------------------------------------------- device */

/* Per-token INT8 activation quantisation (see "Activations" above).
 *   x    device fp32 [M][K], 16-B aligned, finite.
 *   xq   out, device int8 [M][K], 16-B aligned.
 *   xs   out, device fp32 [M].
 * Errors: INVALID_ARG, SHAPE, ALIGN, DEVICE, HIP. */
int32_t s3d8_quant_act(const float *x, int64_t M, int64_t K, int8_t *xq, float *xs, void *stream);

/* Bytes of the tiled device layout of a matrix (see s3d8_tile):
 * ceil(ceil(N/3)/16) * ceil(K/64) * 1024.  -1 on bad sizes. */
int64_t s3d8_tiled_bytes(int64_t N, int64_t K);

/* Re-lay a packed matrix into the tiled device layout read by s3d8_linear
 * and s3d8_forward.  The bytes are unchanged ([BLOG] "Bit layout"); only
 * their order in memory changes, once, before the weights are used (as the
 * blog permutes its lookup tables once before model load).  The matrix is cut
 * into fragments of 16 channel triples x 64 input columns; fragment
 * (tile i, column block b) occupies 1 KiB at byte offset (i*ceil(K/64) + b)
 * * 1024, and inside it the 16 bytes at offset 16*L (L = n + 16*g, n < 16,
 * g < 4) are packed[16i + n][64b + 16g .. 64b + 16g + 15], zero past the last
 * triple or past K.  This is the operand layout of the gfx950 instruction
 * v_mfma_i32_16x16x64_i8 for 16 triples, so each wave reads a fragment as one
 * contiguous 1 KiB load.
 *   packed  device uint8 [ceil(N/3)][K] (canonical layout).
 *   tiled   out, device uint8 [s3d8_tiled_bytes(N, K)], 16-B aligned.
 * Errors: INVALID_ARG, SHAPE (more than 2^31 tiled bytes), ALIGN, DEVICE, HIP. */
int32_t s3d8_tile(const uint8_t *packed, int64_t N, int64_t K, uint8_t *tiled, void *stream);

/* The fused linear layer on pre-quantised activations: decode S3D8 weights
 * on the fly, INT8 x INT8 products accumulated exactly in INT32, fp32
 * epilogue (see "Linear").
 *   xq           device int8 [M][K], 16-B aligned (from s3d8_quant_act).
 *   xs           device fp32 [M].
 *   tiled        device, the matrix in the tiled layout of s3d8_tile,
 *                16-B aligned.
 *   tiled_bytes  size of the tiled buffer; at least s3d8_tiled_bytes(N, K).
 *                A canonical [ceil(N/3)][K] buffer is smaller whenever
 *                ceil(N/3) is not a multiple of 16 or K not a multiple of
 *                64, and is then rejected (INVALID_ARG) instead of being
 *                misread; at other shapes the two layouts have the same
 *                size and only the caller can tell them apart.
 *   centroids    device uint8 [32][3], 4-B aligned.
 *   scales_bf16  device uint16 [3*ceil(N/3)] (entries >= N are not read).
 *   y            out, device fp32 [M][N], row-major.
 *   acc_out      optional out (NULL to skip), device int32 [M][N]: the
 *                accumulators before the epilogue, for verification.
 * Errors: INVALID_ARG (also tiled_bytes too small), SHAPE (also N > 3355442
 * when M > 16), ALIGN, DEVICE, HIP. */
int32_t s3d8_linear(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                    const uint8_t *tiled, int64_t tiled_bytes, const uint8_t *centroids,
                    const uint16_t *scales_bf16, float *y, int32_t *acc_out, void *stream);

/* The whole path from fp32 activations: per-token INT8 quantisation (as
 * s3d8_quant_act) followed by the fused linear (as s3d8_linear).  For M <= 4
 * (and M * ceil(ceil(K/64)/16) <= 16) both run in one kernel launch; otherwise
 * s3d8_quant_act and s3d8_linear are enqueued in turn.  Results are
 * identical to calling the two entry points.
 *   x            device fp32 [M][K], 16-B aligned, finite.
 *   tiled, tiled_bytes, centroids, scales_bf16, y, acc_out
 *                as for s3d8_linear.
 *   xq           out, device int8 [M][K], 16-B aligned: the activation codes.
 *   xs           out, device fp32 [M]: the activation scales.
 * Errors: INVALID_ARG, SHAPE, ALIGN, DEVICE, HIP. */
int32_t s3d8_forward(const float *x, int64_t M, int64_t K, int64_t N, const uint8_t *tiled,
                     int64_t tiled_bytes, const uint8_t *centroids, const uint16_t *scales_bf16,
                     float *y, int8_t *xq, float *xs, int32_t *acc_out, void *stream);

/* One item of s3d8_forward_batch: the arguments of one s3d8_forward call. */
typedef struct s3d8_forward_item {
    const float *x;               /* device fp32 [M][K], 16-B aligned, finite */
    int64_t M, K, N;
    const uint8_t *tiled;         /* as for s3d8_linear */
    int64_t tiled_bytes;          /* as for s3d8_linear */
    const uint8_t *centroids;     /* as for s3d8_linear */
    const uint16_t *scales_bf16;  /* as for s3d8_linear */
    float *y;                     /* out, device fp32 [M][N] */
    int8_t *xq;                   /* out, device int8 [M][K], 16-B aligned */
    float *xs;                    /* out, device fp32 [M] */
    int32_t *acc_out;             /* optional out, device int32 [M][N] */
} s3d8_forward_item;

/* Several independent s3d8_forward calls at once, e.g. the seven linears of
 * a decoder-layer step at one token (each matrix with its own activations,
 * table and scales).  When 1 <= count <= 8, every item has the same M <= 4
 * and each matrix fits the streaming GEMV (M * ceil(ceil(K/64)/16) <= 16),
 * all items run in ONE kernel launch whose workgroups are shared out among
 * the matrices in proportion to their work; otherwise the items run one
 * after the other as s3d8_forward calls.  Results are identical to calling
 * s3d8_forward on each item.  Outputs of different items must not overlap
 * (items may share x, and then write identical xq / xs).
 *   count  number of items (0: nothing to do).
 *   items  host array of count items; read before return, not kept.
 * Errors: INVALID_ARG, SHAPE, ALIGN, DEVICE, HIP (as s3d8_forward, for the
 * first failing item; nothing is launched when validation fails). */
int32_t s3d8_forward_batch(int32_t count, const s3d8_forward_item *items, void *stream);

/* The frozen-centroid quantiser of s3d8_encode on the GPU ([PAPER] Sec. 3.4
 * "Quantization", the QAT-phase Q(.)), with the same arithmetic and the
 * same results: alpha_i = bf16_rne(fp32(max_j |W_ij|) / 127.0f) (0 for
 * padded channels), W' = |W| / alpha in fp64, q = the first centroid row at
 * the smallest squared distance, signs S_d = (W < 0), bytes per the [BLOG]
 * bit layout.  Two launches on `stream`.
 *   W            device fp32 [N][K] row-major, 4-B aligned, finite.
 *   centroids    device uint8 [32][3]; every entry must be <= 127 (not
 *                checked: the table is in device memory).
 *   scales_bf16  out, device uint16 [3*ceil(N/3)], 2-B aligned.
 *   packed       out, device uint8 [ceil(N/3)][K] (canonical layout; pass
 *                it to s3d8_tile for the kernels' layout).
 * Errors: INVALID_ARG, SHAPE (K % 16 != 0, or N*K over 2^31), ALIGN,
 * DEVICE, HIP. */
int32_t s3d8_encode_device(const float *W, int64_t N, int64_t K, const uint8_t *centroids,
                           uint16_t *scales_bf16, uint8_t *packed, void *stream);

/* Size in bytes of the workspace of s3d8_linear_unfused: the whole matrix
 * decoded to channel-INT8 in 2 KiB fragments of 32 channels x 64 columns,
 * ceil(3 * ceil(N/3) / 32) * ceil(K/64) * 2048.  -1 on bad sizes. */
int64_t s3d8_unfused_workspace_bytes(int64_t N, int64_t K);

/* The linear layer of s3d8_linear computed the way the blog's CPU kernels
 * treat more than one token ("Fast? How fast?": dequantise to INT8, then an
 * INT8 matrix product): the tiled matrix is decoded once into `workspace`
 * as channel-INT8, then an INT8 x INT8 GEMM with INT32
 * accumulation and the same fp32 epilogue runs on it.  Results are
 * identical to s3d8_linear; for many token rows it decodes each weight once
 * per call instead of once per row tile.  (The workspace layout is
 * internal to the library.)
 *   xq, xs, M, K, N, tiled, tiled_bytes, centroids, scales_bf16, y, acc_out
 *                as for s3d8_linear.
 *   workspace    device scratch, 16-B aligned, at least
 *                s3d8_unfused_workspace_bytes(N, K) bytes, owned by the
 *                caller; overwritten.  Calls that may run concurrently
 *                need separate workspaces.
 *   workspace_bytes  its size.
 * Errors: INVALID_ARG (also a workspace or tiled_bytes too small), SHAPE (decoded matrix
 * over 2^31 bytes, or N > 3355442), ALIGN, DEVICE, HIP. */
int32_t s3d8_linear_unfused(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                            const uint8_t *tiled, int64_t tiled_bytes, const uint8_t *centroids,
                            const uint16_t *scales_bf16, float *y, int32_t *acc_out, int8_t *workspace,
                            int64_t workspace_bytes, void *stream);

/* Size of the device scratch array of s3d8_linear_unfused_noalloc: 64 MiB. */
#define S3D8_NOALLOC_SCRATCH_BYTES (64LL * 1024 * 1024)

/* s3d8_linear_unfused without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The call allocates nothing: the decoded
 * matrix goes to a device array of S3D8_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, which that GPU holds from the library's first use on
 * it until the process ends.  Results are identical to s3d8_linear_unfused.
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 * (e.g. on two streams) race and must be serialised by the caller.
 *   arguments  as for s3d8_linear_unfused, without the workspace.
 * Errors: as s3d8_linear_unfused; SHAPE also when the decoded matrix,
 * s3d8_unfused_workspace_bytes(N, K), is larger than
 * S3D8_NOALLOC_SCRATCH_BYTES (e.g. the 4096 x 128256 vocabulary projection,
 * 525 MB decoded). */
int32_t s3d8_linear_unfused_noalloc(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                                    const uint8_t *tiled, int64_t tiled_bytes, const uint8_t *centroids,
                                    const uint16_t *scales_bf16, float *y, int32_t *acc_out, void *stream);

/* Decode a whole matrix to channel-INT8 ([PAPER] Eq. 1 without alpha; the
 * blog's standalone S3D8 -> INT8 dequantisation).
 *   packed     device uint8 [ceil(N/3)][K], 16-B aligned.
 *   centroids  device uint8 [32][3], 4-B aligned.
 *   w          out, device int8 [N][K], 16-B aligned; padded channels are
 *              not written.
 * Errors: INVALID_ARG, SHAPE, ALIGN, DEVICE, HIP. */
int32_t s3d8_dequant(const uint8_t *packed, const uint8_t *centroids, int64_t N, int64_t K,
                     int8_t *w, void *stream);

/* ------------------------------------------------------- format variants */

/* Weight formats.  Both store three weights of channels 3t, 3t+1, 3t+2 per
 * byte in the same packed / tiled layout, with the same bf16 channel scales;
 * they differ in the table that turns a byte into three INT8 weights.
 *   S3D8_FORMAT_S3D8  table = uint8 [32][3] absolute-value centroids; the
 *                     byte holds a 5-bit row index and three sign selectors
 *                     (see "Format" above).
 *   S3D8_FORMAT_3D8   table = int8 [256][3] signed centroids, row-major,
 *                     768 bytes, entries in [-127, 127]; the whole byte is
 *                     the row index: w_{3t+d, j} = table[b][d].  This is the
 *                     unstructured 3-values-per-byte format that [BLOG]
 *                     "S3D8: a 2.7-bit weight format for fast decoding"
 *                     compares S3D8 with (256 signed centroids; S3D8's are
 *                     the 8 sign reflections of 32 absolute ones). */
#define S3D8_FORMAT_S3D8 0
#define S3D8_FORMAT_3D8 1

/* Output types of the linear layer.
 *   S3D8_OUT_F32   y fp32 [M][N] (as s3d8_linear).
 *   S3D8_OUT_BF16  y bfloat16 bit patterns, uint16 [M][N]: each fp32 result
 *                  of "Linear" rounded to nearest even, as the [BLOG] fused
 *                  matrix-vector listing converts its results on the way
 *                  out. */
#define S3D8_OUT_F32 0
#define S3D8_OUT_BF16 1

/* s3d8_linear for either weight format and either output type.
 *   table      device, 4-B aligned: the format's table (96 or 768 bytes).
 *   format     S3D8_FORMAT_S3D8 or S3D8_FORMAT_3D8.
 *   y          out, device [M][N] of fp32 or bf16 (per out_type).
 *   out_type   S3D8_OUT_F32 or S3D8_OUT_BF16.
 *   the rest   as for s3d8_linear (acc_out stays int32).
 * Errors: as s3d8_linear; INVALID_ARG also for an unknown format or output
 * type.  With S3D8_FORMAT_S3D8 and S3D8_OUT_F32 it is s3d8_linear. */
int32_t s3d8_linear_ex(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N, const uint8_t *tiled,
                       int64_t tiled_bytes, const void *table, int32_t format, const uint16_t *scales_bf16, void *y,
                       int32_t out_type, int32_t *acc_out, void *stream);

/* Split-K form of s3d8_linear_ex, for prefill shapes with few output tiles
 * and long rows, such as the vision encoder's MLP down-projection
 * (K = 5120, N = 1280 at 1601 tokens; [PAPER] Sec. 4.3, Table 2): the fused
 * GEMM for M > 16 with its input columns cut into `splits` ranges of whole
 * 64-column blocks, one workgroup per (output tile, range).  The ranges'
 * INT32 partial sums are added exactly before the epilogue ([BLOG] "Fused
 * matrix-vector product": accumulate in INT32, then scale), so results are
 * identical to s3d8_linear_ex for every split count.  M <= 16 runs the
 * GEMV paths of s3d8_linear_ex (no split, workspace unused).
 *   splits     ranges per tile: 0 = s3d8_splitk_auto for the current device;
 *              otherwise at least 1, clamped to ceil(K/64) and rounded so
 *              that no range is empty.
 *   workspace  device, 256-B aligned, at least
 *              s3d8_splitk_workspace_bytes(M, K, N, splits) bytes (splits as
 *              resolved for 0), owned by the caller; NULL allowed when that
 *              size is 0.  It holds two counters per output tile and the
 *              partial sums.  It must be filled with zeros once before its
 *              first use; every call leaves the counters at zero again, so
 *              later calls need no clearing.  Calls that may run
 *              concurrently need separate workspaces.
 *   workspace_bytes  its size.
 *   the rest   as for s3d8_linear_ex.
 * Errors: as s3d8_linear_ex; INVALID_ARG also for splits < 0 or a missing
 * or too small workspace; ALIGN for a misaligned workspace; SHAPE also when
 * the partial sums would exceed 2^31 bytes. */
int32_t s3d8_linear_splitk(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N, const uint8_t *tiled,
                           int64_t tiled_bytes, const void *table, int32_t format, const uint16_t *scales_bf16,
                           void *y, int32_t out_type, int32_t *acc_out, int32_t splits, void *workspace,
                           int64_t workspace_bytes, void *stream);

/* The split count s3d8_linear_splitk takes for splits = 0 on a GPU with
 * num_cus compute units: the S that minimises ceil(ceil(K/64)/S) + 9 S
 * (the main loop's 64-column blocks per workgroup plus the measured cost of
 * adding S slots of partial sums, in the same unit) among 1 and the counts
 * whose workgroups fit one round on the CUs (output tiles x S <= num_cus),
 * at most 16.  The output tiles are those of the fused GEMM's tile height
 * for this shape and CU count (64, 128 or 160 rows x 384 channels, the
 * height with the least estimated time).  1 for M <= 16.  -1 on bad
 * sizes. */
int32_t s3d8_splitk_auto(int64_t M, int64_t K, int64_t N, int32_t num_cus);

/* Workspace bytes of s3d8_linear_splitk at a split count >= 1 (0 for M <= 16
 * or a single range).  -1 on bad sizes. */
int64_t s3d8_splitk_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t splits);

/* s3d8_forward for either weight format and either output type (arguments
 * as s3d8_linear_ex and s3d8_forward; xq and xs as for s3d8_forward).  The
 * same launches as s3d8_forward.  Errors: as s3d8_forward, plus
 * INVALID_ARG for an unknown format or output type. */
int32_t s3d8_forward_ex(const float *x, int64_t M, int64_t K, int64_t N, const uint8_t *tiled, int64_t tiled_bytes,
                        const void *table, int32_t format, const uint16_t *scales_bf16, void *y, int32_t out_type,
                        int8_t *xq, float *xs, int32_t *acc_out, void *stream);

/* s3d8_linear_unfused for either weight format and either output type
 * (arguments as s3d8_linear_ex, workspace as s3d8_linear_unfused).
 * Errors: as s3d8_linear_unfused, plus INVALID_ARG for an unknown format or
 * output type. */
int32_t s3d8_linear_unfused_ex(const int8_t *xq, const float *xs, int64_t M, int64_t K, int64_t N,
                               const uint8_t *tiled, int64_t tiled_bytes, const void *table, int32_t format,
                               const uint16_t *scales_bf16, void *y, int32_t out_type, int32_t *acc_out,
                               int8_t *workspace, int64_t workspace_bytes, void *stream);

/* s3d8_dequant for either weight format: w = the table decode of every
 * byte, channel-INT8 [N][K] (padded channels not written).  table and
 * format as for s3d8_linear_ex; the rest as for s3d8_dequant.  Errors: as
 * s3d8_dequant, plus INVALID_ARG for an unknown format. */
int32_t s3d8_dequant_ex(const uint8_t *packed, const void *table, int32_t format, int64_t N, int64_t K, int8_t *w,
                        void *stream);

/* Matrix-core rate probe: a measurement utility for reading the GEMM's
 * INT8 rate against what the matrix cores sustain, not part of the method.
 * `workgroups` workgroups of 256 threads (4 waves) each run `iters` rounds
 * of four independent v_mfma_i32_32x32x32_i8 (a 32 x 32 x 32 INT8 product
 * into INT32, 65536 integer operations) on register operands whose bytes
 * all equal v; thread t of workgroup w then stores 2048 * v^2 * iters
 * (mod 2^32) to out[256 w + t].  A call performs
 * workgroups * 4 * 4 * iters * 65536 operations.
 *   out   out, device int32 [256 * workgroups], 4-B aligned.
 * Errors: INVALID_ARG (out NULL, iters < 1, workgroups outside
 * [1, 65536], v outside [-128, 127]), ALIGN, DEVICE, HIP. */
int32_t s3d8_mfma_rate_probe(int32_t iters, int32_t workgroups, int32_t v, int32_t *out, void *stream);

/* Memory read probe: a measurement utility for reading the memory-bound
 * kernels against the rate at which a buffer of the same size streams out of
 * device memory, not part of the method.  `workgroups` workgroups of 256
 * threads read the `bytes` bytes at p as 16-byte chunks (chunk c by
 * workgroup (c / 256) mod workgroups) and workgroup w stores the XOR of the
 * 32-bit words it read to out[w]; the XOR of all of out is therefore the
 * XOR of all words of p.
 *   p      device, 16-B aligned; bytes a positive multiple of 16.
 *   out    out, device uint32 [workgroups], 4-B aligned.
 * Errors: INVALID_ARG (null pointer, bytes not a positive multiple of 16,
 * workgroups outside [1, 65536]), ALIGN, DEVICE, HIP. */
int32_t s3d8_hbm_read_probe(const void *p, int64_t bytes, int32_t workgroups, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* S3D8_H */
