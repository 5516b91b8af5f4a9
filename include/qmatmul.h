/*
 * qmatmul.h -- C ABI of the MI355X (gfx950) GGUF quantized matmul library.
 *
 * Computes y[M x N] = x[M x K] . W[N x K]^T where W is stored as GGUF
 * quantized blocks exactly as a GGUF file stores a weight tensor: N rows, each
 * row K/QK consecutive blocks cut along K (page "自己量化", section
 * "2. q、k 投影的行重排": blocks run along a row).  x and y are f32, row-major,
 * contiguous.  y is overwritten.
 *
 * Two numerical modes, the two forms the page "同一个 GGUF，CPU 和 Metal
 * 生成的文字不一样" (section 出处) contrasts:
 *   QMM_MODE_F32ACT (a)  activations stay f32; weight blocks are dequantized
 *                        inside the kernel (the Metal form).  Accurate to f32.
 *   QMM_MODE_QACT   (b)  each activation row is first quantized on its own
 *                        (Q8_0 for Q8_0 weights, Q8K for Q4_K weights, per 32 or
 *                        256 values), then integer block dot products are
 *                        scaled by the weight and activation block scales (the
 *                        CPU form).
 * and the third form the same page (section 修法) sets against them:
 *   QMM_MODE_DEQUANT     every weight block decoded to f32 once, then a plain
 *                        f32 matmul (CANDLE_DEQUANTIZE_ALL): no activation
 *                        quantization, f32-sized weights.
 *
 * Block formats (little-endian; byte sizes fixed by the page "自己量化",
 * sections 和下载的 Q8_0 逐字节比 and 大小和误差):
 *   QMM_Q8_0   34 B per 32 values: f16 d, int8 q[32].
 *   QMM_Q4_K  144 B per 256 values: f16 d, f16 dmin, 12 B packed 6-bit
 *             sub-block scales and mins, 128 B of 4-bit values.
 *   QMM_Q8_K  292 B per 256 values (activations only): f32 d, int8 q[256],
 *             int16 bsums[16].
 * and the other formats of the pages' files (Q4_0 and Q5_0 sizes fixed by the
 * same page's byte counts, section 大小和误差 and the Q5_0 tensor totals of
 * 和下载的 Q8_0 逐字节比; Q6_K named there among the downloaded file's
 * tensors; the packings are the public GGUF layout, not printed by the pages):
 *   QMM_Q4_0   18 B per 32 values: f16 d, 16 B of 4-bit values (element j < 16
 *             in the low nibble of byte j, element j+16 in its high nibble);
 *             w = d*(q - 8).
 *   QMM_Q5_0   22 B per 32 values: f16 d, u32 of fifth bits (bit j of element
 *             j), 16 B of 4-bit values as Q4_0; w = d*(q - 16).
 *   QMM_Q6_K  210 B per 256 values: 128 B low 4 bits, 64 B high 2 bits, int8
 *             scales[16] (one per 16 values), f16 d; w = d*sc*(q - 32).
 * Mode (b) pairs Q4_0 and Q5_0 with Q8_0 activations and Q6_K with Q8K (page
 * "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处).  K must be a
 * multiple of the block size: 32 for Q8_0, Q4_0 and Q5_0, 256 for the
 * K-quants.  The kernels read 32-value blocks in pairs: rows with an odd
 * number of blocks run on copies one all-zero block longer, made in the plan's
 * workspace at every run (correct at any such K; the throughput is that of
 * the even case plus the copies).
 *
 * Pointers named "device" must be device memory of the current HIP device
 * (e.g. torch tensor data pointers); `stream` is a hipStream_t (NULL = the
 * null stream).  Every call that takes a stream is asynchronous: it enqueues
 * kernels and returns without synchronizing.  No call throws or aborts; each
 * returns a status code, and qmatmul_last_error() gives a message for the
 * calling thread.  Argument checks happen on the host before any HIP call.
 */
#ifndef QMATMUL_H
#define QMATMUL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* formats: the GGUF (ggml) type ids */
#define QMM_Q4_0 2
#define QMM_Q5_0 6
#define QMM_Q8_0 8
#define QMM_Q4_K 12
#define QMM_Q6_K 14
#define QMM_Q8_K 15

/* modes */
#define QMM_MODE_F32ACT 0
#define QMM_MODE_QACT 1
#define QMM_MODE_DEQUANT 2

/* status codes */
#define QMM_OK 0
#define QMM_EINVAL 1       /* null pointer, non-positive size, M > M_max, misaligned pointer */
#define QMM_EBLOCK 2       /* K not a multiple of the format's block size */
#define QMM_EUNSUPPORTED 3 /* unknown format or mode, or a format/mode pairing not offered */
#define QMM_ENOMEM 4       /* device allocation failed */
#define QMM_EHIP 5         /* a HIP runtime call or kernel launch failed */

typedef struct qmm_plan qmm_plan;

/*
 * Create a plan for one weight shape: format, N output rows, K inputs, up to
 * M_max activation rows per run, and a mode.  The mode is fixed here, as the
 * pages' QMatMul fixes its form when it is built (page "同一个 GGUF，CPU 和
 * Metal 生成的文字不一样", section 修法).  K must be a multiple of the block
 * size, 32 (Q8_0, Q4_0, Q5_0) or 256 (Q4_K, Q6_K), the shape check of page
 * "自己量化", section "3. 量化" (QMM_EBLOCK).
 * Allocates the plan's device workspace on the current device (hipMalloc).
 * On success *out receives the plan; on failure *out is set to NULL.
 */
int qmatmul_create(qmm_plan** out, int format, int64_t N, int64_t K, int64_t M_max, int mode);

/*
 * Run y = x . W^T on `stream`.  w_blocks: device, N * qmatmul_row_bytes(format, K)
 * bytes, 16-byte aligned.  x: device f32 [M x K].  y: device f32 [M x N],
 * overwritten.  0 <= M <= M_max; M == 0 enqueues nothing.  M <= 8 takes the
 * decode (GEMV) kernels, larger M the prefill (GEMM) kernels.  The caller owns
 * w, x and y; the plan keeps no pointer after the call.  The plan's workspace
 * is shared by its runs: do not run one plan concurrently on two streams.
 * At M > 8, Q8_0, Q4_0, Q5_0 and Q4_K runs with short rows (K <= 1536, at
 * most 8192 rows of W, a grid of at most one workgroup per compute unit) take
 * one launch that prepares its own activations; other Q4_0 and Q5_0 runs
 * first rewrite the weights as Q8_0 blocks (the same dequantized values) in
 * the plan's workspace and take the Q8_0 prefill kernels; Q6_K runs with
 * M > 8 take their own prefill kernel (both modes) on the f16 matrix cores.
 * A run only enqueues kernels (no allocation, memset or synchronization), so
 * runs may be captured in a HIP graph once each kernel has run eagerly (its
 * launch attributes are set on first use); the exception is a
 * QMM_MODE_DEQUANT plan, whose product is a rocBLAS call.
 */
int qmatmul_run(const qmm_plan* plan, const void* w_blocks, const float* x, float* y,
                int64_t M, void* stream);

/*
 * Grouped run: y[i] = x . W[i]^T for count plans that share format, K and mode
 * and one activation matrix x (M x K), such as the q, k and v (or gate and up)
 * projections of one layer; each product is the one qmatmul_run computes
 * (page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处).  plans,
 * w_blocks and y are host arrays of count entries (1 <= count <=
 * QMM_GROUP_MAX) holding each plan's device pointers, with qmatmul_run's
 * sizes and alignment; 0 <= M <= every plan's M_max.  At M == 1 for Q8_0 and
 * Q4_K (where the one-row decode kernel takes the rows), and at M <= 8 for
 * Q4_0, Q5_0 and Q6_K (where their activations fit in LDS), the plans' rows
 * go to one launch per four plans (the activations are loaded and quantized
 * once per workgroup for all of them), giving bit-for-bit the values
 * separate runs give; at M > 8 each plan takes the prefill kernel its own run
 * takes, the plans' output tiles going to one launch per four plans of that
 * kernel (the activations prepared once for the K-staged kernels; again the
 * separate runs' values bit for bit); otherwise the plans run one after
 * another as with qmatmul_run.  Errors: as
 * qmatmul_run for each plan, and QMM_EINVAL for null arrays, count out of
 * range or plans that differ in format, K or mode.
 */
#define QMM_GROUP_MAX 8
int qmatmul_run_group(const qmm_plan* const* plans, int count, const void* const* w_blocks, const float* x,
                      float* const* y, int64_t M, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Computes
 * what qmatmul_create(format, N, K, M, mode) followed by qmatmul_run(..., M,
 * stream) computes, with the same kernels and the same values, but without a
 * plan and without allocating: the workspace lives in a static device array
 * of QMM_NOALLOC_SCRATCH_BYTES that each GPU holds from the library's first
 * use on it until the process ends (qmatmul_workspace_bytes(format, N, K, M,
 * mode) says what a shape needs).  w_blocks, x, y: device, as in qmatmul_run.
 * Errors: those of qmatmul_create and qmatmul_run; QMM_EINVAL when the shape
 * needs more scratch than the array holds; QMM_EUNSUPPORTED for
 * QMM_MODE_DEQUANT (its product is a library GEMM that allocates).  Every call on a GPU uses that GPU's one
 * array: calls that overlap on one GPU (on two streams, or from two host
 * threads) race and must be serialized by the caller.  The first call on
 * each device looks up the array's address (no allocation); its kernels set
 * their launch attributes on first use, so capture a call in a HIP graph only
 * after one eager call of the same shape.
 */
#define QMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int qmatmul_run_noalloc(int format, int64_t N, int64_t K, int64_t M, int mode, const void* w_blocks,
                        const float* x, float* y, void* stream);

/* Free a plan and its workspace (NULL is a no-op).  Synchronizes the device
 * before freeing, so pending runs of the plan finish first. */
int qmatmul_destroy(qmm_plan* plan);

/*
 * Dequantize-all form (page "同一个 GGUF，CPU 和 Metal 生成的文字不一样",
 * section 修法: CANDLE_DEQUANTIZE_ALL decodes every quantized weight to f32 at
 * load, then both devices run a plain f32 matmul).
 *
 * qmatmul_dequantize_weights: GGUF blocks (device, N * qmatmul_row_bytes(format,
 * K) bytes, 16-byte aligned) -> f32 [N x K] (device, 16-byte aligned, caller
 * owned).  Every value is the exact dequantized weight (Q8_0 d*q; Q4_K
 * d*sc_j*q - dmin*m_j; Q4_0 d*(q-8); Q5_0 d*(q-16); Q6_K d*sc*(q-32)) rounded
 * once to f32.
 *
 * qmatmul_run_dequantized (QMM_MODE_DEQUANT plans only): y = x . W^T with W
 * given as that f32 [N x K] matrix; x, y as in qmatmul_run.  The product is the
 * library f32 GEMM (rocBLAS), deterministic.  qmatmul_run on a QMM_MODE_DEQUANT
 * plan decodes w_blocks into the plan's workspace (N*K*4 bytes) first and then
 * does the same; load-once callers decode with qmatmul_dequantize_weights and
 * call qmatmul_run_dequantized.
 */
int qmatmul_dequantize_weights(int format, const void* w_blocks, int64_t N, int64_t K, float* out,
                               void* stream);
int qmatmul_run_dequantized(const qmm_plan* plan, const float* w_f32, const float* x, float* y,
                            int64_t M, void* stream);

/*
 * Quantize activation rows the way mode (b) does, writing canonical blocks:
 * act_format QMM_Q8_0 (34 B per 32) or QMM_Q8_K (292 B per 256).  Row-local:
 * each row depends only on itself (page "自己量化", section 动脑筋答案).
 * x: device f32 [M x K]; out_blocks: device, M * qmatmul_row_bytes(act_format, K)
 * bytes.  Bit-identical to the quantization inside qmatmul_run.
 */
int qmatmul_quantize_act(int act_format, const float* x, int64_t M, int64_t K,
                         void* out_blocks, void* stream);

/*
 * Quantize f32 weights [N x K] (device) into GGUF blocks (device, N *
 * qmatmul_row_bytes(format, K) bytes), the role of QTensor::quantize on the
 * page "自己量化" (section "3. 量化").  Q8_0: d = max|w|/127, q = round(w/d).
 * Q4_K: per 32-value sub-block an affine min/max fit, 6-bit scales and mins
 * against the super-block maximum / 63, 4-bit values re-quantized against the
 * stored f16 scales (no importance matrix).  Q4_0 / Q5_0: the signed value of
 * largest magnitude takes the most negative code, d = max/-8 (-16), q =
 * floor(w/d + 8.5) (+ 16.5) capped at 15 (31).  Q6_K: per 16 values s = (signed
 * max)/-32, d = (signed s of largest magnitude)/-128, scales round(s/d) capped
 * at 127, q = clamp(round(w/(d*sc)), -32, 31) + 32.  w and out_blocks
 * 16-byte aligned.
 */
int qmatmul_quantize_weights(int format, const float* w, int64_t N, int64_t K,
                             void* out_blocks, void* stream);

/*
 * Q4_K weight quantizer with a search (the page "自己量化", section "3. 量化",
 * names QTensor::quantize(&w, Q4K) without describing its search): per
 * 32-value sub-block, candidate codes for 22 scales around the min/max
 * rule's (that rule's own among them), each refitted by least squares to a
 * scale and a non-negative min, the smallest squared error kept; then the
 * super-block's 6-bit scales and mins and the 4-bit values as
 * qmatmul_quantize_weights(QMM_Q4_K, ...) forms them.  w: device f32 [N x K],
 * K % 256 == 0; out_blocks: device, N * qmatmul_row_bytes(QMM_Q4_K, K) bytes;
 * both 16-byte aligned.  One thread per super-block (an offline step).
 */
int qmatmul_quantize_q4_k_search(const float* w, int64_t N, int64_t K, void* out_blocks, void* stream);

/*
 * Traced run (mode (b) plans only): qmatmul_run's own kernels, with the same
 * launch configuration, compiled with a flag that also writes out the integer
 * parts the method fixes exactly (page "同一个 GGUF，CPU 和 Metal 生成的文字不一样",
 * section 出处: integer block dot products, then the scales).
 *   y: as qmatmul_run writes it, bit for bit (NULL: not written).
 *   sums: device int32 [M x N x qmatmul_block_sums_per_row(format, K)]:
 *     Q8_0, Q4_0, Q5_0: S[m][n][b] = sum over block b of qw*qx, qw the signed
 *       weight value (q, q - 8, q - 16);
 *     Q4_K: per super-block ten values S_0..S_7 (per 32 values), sumi =
 *       sum_j sc_j*S_j and summins = sum_j m_j*(bsums[2j]+bsums[2j+1]);
 *     Q6_K: per super-block 17 values S_0..S_15 (per 16, qw = q - 32) and
 *       sumi = sum_j sc_j*S_j.
 *     At M > 8 the K-staged Q4_K prefill kernel scales each S_j on its own
 *     and never forms sumi; there sumi is summed from the S_j it wrote (the
 *     short-row kernel forms it in int32 itself).  The Q6_K
 *     prefill kernel (M > 8) carries the scales in its weight operand and
 *     forms sumi exactly but no per-16 sums: there S_0..S_15 read INT32_MIN.
 *   act_blocks: device, M * qmatmul_row_bytes(Q8_0 or Q8_K, K) bytes, 4-byte
 *     aligned, or NULL: the canonical quantized activation blocks, written by
 *     the kernel that quantizes them in this run (a decode kernel's own
 *     prologue, the short-row prefill's, or the prefill's activation
 *     preparation).
 * Same preconditions and errors as qmatmul_run; sums must not be NULL.
 */
int qmatmul_run_traced(const qmm_plan* plan, const void* w_blocks, const float* x, float* y, int32_t* sums,
                       void* act_blocks, int64_t M, void* stream);

/* qmatmul_run_traced(plan, w_blocks, x, NULL, sums, NULL, M, stream). */
int qmatmul_run_block_sums(const qmm_plan* plan, const void* w_blocks, const float* x,
                           int32_t* sums, int64_t M, void* stream);

/* Host-only helpers (no HIP calls; safe without a GPU). */
int qmatmul_check(int format, int64_t N, int64_t K, int64_t M_max, int mode); /* what create validates */
int64_t qmatmul_row_bytes(int format, int64_t K);           /* bytes of one row of blocks, -1 if invalid */
int64_t qmatmul_block_sums_per_row(int format, int64_t K);  /* int32 entries per (m, n), -1 if invalid */
int64_t qmatmul_workspace_bytes(int format, int64_t N, int64_t K, int64_t M_max, int mode); /* -1 if invalid */
const char* qmatmul_status_string(int status);
const char* qmatmul_last_error(void); /* message of the calling thread's last failure, "" if none */
int qmatmul_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QMATMUL_H */
