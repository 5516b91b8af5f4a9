// qmm_capi.cpp -- the C ABI declared in include/qmatmul.h: argument checks,
// plans and their workspace, and dispatch to the decode (M <= 8) or prefill
// kernels.  Every check runs on the host before any HIP call, so the error
// paths work without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <new>

#include "../../include/qmatmul.h"
#include "qmm_internal.h"

using namespace qmm;

struct qmm_plan {
    int fmt, mode;
    int64_t N, K, M_max;
    int device;
    void* ws;
    size_t ws_bytes;
    GemvBufs gv;
    GemmBufs gm;
    ExtBufs ex;    // Q4_0, Q5_0, Q6_K
    float* wdeq;   // dequantize-all plans: the decoded weights [N][K]
    void* dense;   // dequantize-all plans: the f32 GEMM handle
    // Q8_0, Q4_0, Q5_0 rows with an odd number of blocks run one all-zero
    // block longer: Kr = K + 32 (else K), the padded weights and activations
    int64_t Kr;
    uint8_t* wpad;
    float* xpad;
};

static thread_local char g_err[512];

static int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

static int64_t block_values(int fmt)
{
    switch (fmt) {
    case QMM_Q8_0: return 32;
    case QMM_Q4_K: return 256;
    case QMM_Q8_K: return 256;
    case QMM_Q4_0: return 32;
    case QMM_Q5_0: return 32;
    case QMM_Q6_K: return 256;
    default: return -1;
    }
}

static int64_t block_bytes(int fmt)
{
    switch (fmt) {
    case QMM_Q8_0: return 34;
    case QMM_Q4_K: return 144;
    case QMM_Q8_K: return 292;
    case QMM_Q4_0: return 18;
    case QMM_Q5_0: return 22;
    case QMM_Q6_K: return 210;
    default: return -1;
    }
}

extern "C" int64_t qmatmul_row_bytes(int format, int64_t K)
{
    const int64_t qk = block_values(format);
    if (qk < 0 || K <= 0 || K % qk) return -1;
    return K / qk * block_bytes(format);
}

extern "C" int64_t qmatmul_block_sums_per_row(int format, int64_t K)
{
    if ((format == QMM_Q8_0 || format == QMM_Q4_0 || format == QMM_Q5_0) && K > 0 && K % 32 == 0) return K / 32;
    if (format == QMM_Q4_K && K > 0 && K % 256 == 0) return K / 256 * 10;
    if (format == QMM_Q6_K && K > 0 && K % 256 == 0) return K / 256 * 17;
    return -1;
}

static bool weight_format(int f)
{
    return f == QMM_Q8_0 || f == QMM_Q4_K || f == QMM_Q4_0 || f == QMM_Q5_0 || f == QMM_Q6_K;
}

static int check_shape(int format, int64_t N, int64_t K, int64_t M_max, int mode)
{
    if (!weight_format(format))
        return fail(QMM_EUNSUPPORTED,
                    "unsupported weight format %d (expected %d Q4_0, %d Q5_0, %d Q8_0, %d Q4_K or %d Q6_K)", format,
                    QMM_Q4_0, QMM_Q5_0, QMM_Q8_0, QMM_Q4_K, QMM_Q6_K);
    if (mode != QMM_MODE_F32ACT && mode != QMM_MODE_QACT && mode != QMM_MODE_DEQUANT)
        return fail(QMM_EUNSUPPORTED,
                    "unsupported mode %d (expected 0 f32 activations, 1 quantized activations or 2 dequantize-all)",
                    mode);
    if (N <= 0 || K <= 0 || M_max <= 0)
        return fail(QMM_EINVAL, "sizes must be positive: N=%lld K=%lld M_max=%lld", (long long)N, (long long)K,
                    (long long)M_max);
    const int64_t qk = block_values(format);
    if (K % qk)
        return fail(QMM_EBLOCK, "quantized tensor must have their last dim divisible by block size [%lld, %lld] %lld",
                    (long long)N, (long long)K, (long long)qk);
    if (N > (1ll << 30) || K > (1ll << 20) || M_max > (1ll << 24) || N * (K / qk) * block_bytes(format) > (1ll << 40))
        return fail(QMM_EINVAL, "shape too large: N=%lld K=%lld M_max=%lld", (long long)N, (long long)K,
                    (long long)M_max);
    return QMM_OK;
}

extern "C" int qmatmul_check(int format, int64_t N, int64_t K, int64_t M_max, int mode)
{
    g_err[0] = 0;
    return check_shape(format, N, K, M_max, mode);
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Rows of a 32-value format with an odd number of blocks: the kernels read
// blocks in pairs, so such rows run on a copy one all-zero block longer.
static bool odd_blocks(int fmt, int64_t K)
{
    return (fmt == QMM_Q8_0 || fmt == QMM_Q4_0 || fmt == QMM_Q5_0) && (K / 32) % 2 == 1;
}

// Byte layout of the workspace; fills the buffer pointers when base != null.
static size_t layout(qmm_plan* p, char* base)
{
    const bool pad = p->mode != QMM_MODE_DEQUANT && odd_blocks(p->fmt, p->K);
    p->Kr = pad ? p->K + 32 : p->K;
    const int64_t K = p->Kr, N = p->N;
    const int64_t units = p->fmt == QMM_Q4_K ? K / 256 : K / 32;
    const bool a = p->mode == QMM_MODE_F32ACT, q4 = p->fmt == QMM_Q4_K;
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* r = base ? base + off : nullptr;
        off += align256(bytes ? bytes : 16);
        return r;
    };
    p->ex = ExtBufs{};
    p->wpad = pad ? (uint8_t*)take((size_t)N * (K / 32) * block_bytes(p->fmt)) : nullptr;
    p->xpad = pad ? (float*)take(4 * (size_t)p->M_max * K) : nullptr;
    if (p->mode == QMM_MODE_DEQUANT) {  // the decoded weights only
        p->wdeq = (float*)take(4 * (size_t)N * K);
        p->gv = GemvBufs{};
        p->gm = GemmBufs{};
        return off;
    }
    if (is_ext_format(p->fmt)) {
        // Decode runs take the ext kernels; prefill runs: Q6_K its f16 prefill
        // kernel, Q4_0/Q5_0 the Q8_0 kernels on transcoded weights.
        const bool q6 = p->fmt == QMM_Q6_K, pre = !q6 && p->M_max > GEMV_MAX_M;
        const int64_t Mx = std::min<int64_t>(p->M_max, GEMV_MAX_M);
        p->gv = GemvBufs{};
        p->gm = GemmBufs{};
        if (!a) {
            p->ex.xq = (int8_t*)take((size_t)Mx * K);
            p->ex.xd = (float*)take(4 * (size_t)Mx * (q6 ? K / 256 : K / 32));
            p->ex.xs = (int32_t*)take(4 * (size_t)Mx * (q6 ? K / 16 : K / 32));
        }
        if (q6 && p->M_max > GEMV_MAX_M) {
            // mode (a): hi, lo of x*s and 1/s; mode (b): the Q8K values as f16 and the block scales
            const int64_t M = p->M_max;
            p->gm.a0 = (_Float16*)take(2 * M * K);
            p->gm.a1 = (_Float16*)take(a ? 2 * M * K : 0);
            p->gm.rs = (float*)take(a ? 4 * M : 0);
            p->gm.xs = nullptr;
            p->gm.sd = (float*)take(a ? 0 : 4 * M * (K / 256));
        }
        if (pre) {
            p->ex.tw = (uint8_t*)take((size_t)N * (K / 32) * 34);
            const int64_t M = p->M_max;
            p->gm.a0 = (_Float16*)take(a ? 2 * M * K : M * K);
            p->gm.a1 = (_Float16*)take(a ? 2 * M * K : 0);
            p->gm.rs = (float*)take(a ? 4 * M : 0);
            p->gm.xs = nullptr;
            p->gm.sd = (float*)take(a ? 0 : 4 * M * (K / 32));
        }
        return off;
    }
    // decode path
    const int splits = gemv_max_splits(p->fmt, K);
    p->gv.part = (float*)take(splits > 1 ? 4 * (size_t)splits * GEMV_MAX_M * N : 0);
    // prefill path
    if (p->M_max > GEMV_MAX_M) {
        const int64_t M = p->M_max;
        p->gm.a0 = (_Float16*)take(a ? 2 * M * K : M * K);  // mode (b): int8 values
        p->gm.a1 = (_Float16*)take(a ? 2 * M * K : 0);
        p->gm.rs = (float*)take(a ? 4 * M : 0);
        p->gm.xs = (_Float16*)take(q4 ? 2 * M * (K / 256) * 16 : 0);
        p->gm.sd = (float*)take(a ? 0 : 4 * M * units);
    } else {
        p->gm = GemmBufs{};
    }
    return off;
}

extern "C" int64_t qmatmul_workspace_bytes(int format, int64_t N, int64_t K, int64_t M_max, int mode)
{
    if (check_shape(format, N, K, M_max, mode) != QMM_OK) return -1;
    qmm_plan p{};
    p.fmt = format;
    p.mode = mode;
    p.N = N;
    p.K = K;
    p.M_max = M_max;
    return (int64_t)layout(&p, nullptr);
}

extern "C" int qmatmul_create(qmm_plan** out, int format, int64_t N, int64_t K, int64_t M_max, int mode)
{
    g_err[0] = 0;
    if (!out) return fail(QMM_EINVAL, "out is NULL");
    *out = nullptr;
    int st = check_shape(format, N, K, M_max, mode);
    if (st != QMM_OK) return st;
    qmm_plan* p = new (std::nothrow) qmm_plan{};
    if (!p) return fail(QMM_ENOMEM, "host allocation failed");
    p->fmt = format;
    p->mode = mode;
    p->N = N;
    p->K = K;
    p->M_max = M_max;
    p->ws_bytes = layout(p, nullptr);
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) {
        delete p;
        return fail(QMM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    }
    e = hipMalloc(&p->ws, p->ws_bytes);
    if (e != hipSuccess) {
        delete p;
        return fail(e == hipErrorOutOfMemory ? QMM_ENOMEM : QMM_EHIP, "hipMalloc(%zu): %s", p->ws_bytes,
                    hipGetErrorString(e));
    }
    layout(p, (char*)p->ws);
    const bool dense = mode == QMM_MODE_DEQUANT;
    if (dense && dense_create(&p->dense) != 0) {
        (void)hipFree(p->ws);
        delete p;
        return fail(QMM_EHIP, "rocblas_create_handle failed");
    }
    *out = p;
    return QMM_OK;
}

extern "C" int qmatmul_destroy(qmm_plan* p)
{
    g_err[0] = 0;
    if (!p) return QMM_OK;
    hipError_t e = hipDeviceSynchronize();
    dense_destroy(p->dense);
    hipError_t f = hipFree(p->ws);
    delete p;
    if (e != hipSuccess) return fail(QMM_EHIP, "hipDeviceSynchronize: %s", hipGetErrorString(e));
    if (f != hipSuccess) return fail(QMM_EHIP, "hipFree: %s", hipGetErrorString(f));
    return QMM_OK;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

constexpr int PG_GROUP_S = 4;  // problems per short-row launch

static int check_run(const qmm_plan* p, const void* w, const float* x, const void* y, int64_t M)
{
    if (!p) return fail(QMM_EINVAL, "plan is NULL");
    if (M < 0 || M > p->M_max)
        return fail(QMM_EINVAL, "M=%lld outside [0, M_max=%lld]", (long long)M, (long long)p->M_max);
    if (M == 0) return QMM_OK;
    if (!w || !x || !y) return fail(QMM_EINVAL, "null pointer: w=%p x=%p out=%p", w, (const void*)x, y);
    if (!aligned(w, 16)) return fail(QMM_EINVAL, "w_blocks must be 16-byte aligned");
    if (!aligned(x, 16)) return fail(QMM_EINVAL, "x must be 16-byte aligned");
    if (!aligned(y, 4)) return fail(QMM_EINVAL, "output must be 4-byte aligned");
    return QMM_OK;
}

// tr: a traced run (mode (b)), whose kernels also write their integer parts;
// y may then be null.
static int run_impl(const qmm_plan* p, const void* w, const float* x, float* y, const Trace* tr, int64_t M,
                    void* stream)
{
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (p->mode == QMM_MODE_DEQUANT) {
        e = is_ext_format(p->fmt) ? launch_ext_dequantize(p->fmt, w, p->N, p->K, p->wdeq, s)
                                  : launch_dequantize(p->fmt, w, p->N, p->K, p->wdeq, s);
        if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
        const int st = dense_gemm(p->dense, p->wdeq, x, y, M, p->N, p->K, s);
        if (st != 0) return fail(QMM_EHIP, "rocblas_sgemm: status %d", st);
        return QMM_OK;
    }
    uint8_t* act = tr ? tr->act : nullptr;
    int32_t* sums = tr ? tr->sums : nullptr;
    const int64_t K = p->Kr;  // the row length the kernels run on
    if (K != p->K) {          // an odd block count: the padded copies
        const int bb = (int)block_bytes(p->fmt);
        e = launch_pad(w, p->N, (int)(p->K / 32) * bb, (int)(K / 32) * bb, p->wpad, x, M, p->K, K, p->xpad, s);
        if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
        w = p->wpad;
        x = p->xpad;
    }
    if (is_ext_format(p->fmt)) {
        if (M == 1 && gemv_row_supported(p->fmt, p->mode, 1, p->N, K, tr != nullptr)) {
            e = launch_gemv_row(p->fmt, p->mode, w, x, p->N, K, y, s, tr);  // Q4_0, Q5_0: the one-row kernel
        } else if (M <= GEMV_MAX_M && gemv_reg_supported(p->fmt, p->mode, (int)M, p->N, K)) {
            e = launch_gemv_reg(p->fmt, p->mode, w, x, p->N, K, (int)M, y, s, tr);  // 2..8 rows, K <= 4096
        } else if (M <= GEMV_MAX_M) {
            e = launch_ext_run(p->fmt, p->mode, w, x, p->N, K, M, p->ex, y, s, tr);
        } else if (p->fmt == QMM_Q6_K) {
            e = launch_gemm_prep(FMT_Q6_K, p->mode, x, M, K, p->gm, s, act);
            if (e == hipSuccess) e = launch_gemm(FMT_Q6_K, p->mode, w, p->N, K, M, p->gm, y, s, sums);
        } else {
            if (gemm_s_supported(p->fmt, p->mode, K, p->N, M)) {  // short rows: the blocks as they are
                e = launch_gemm_s(p->fmt, p->mode, 1, &w, &p->N, &y, x, K, M, s, tr);
            } else {
                e = launch_ext_to_q8_0(p->fmt, w, p->N, K, p->ex.tw, s);
                if (e == hipSuccess) e = launch_gemm_prep(FMT_Q8_0, p->mode, x, M, K, p->gm, s, act);
                if (e == hipSuccess) e = launch_gemm(FMT_Q8_0, p->mode, p->ex.tw, p->N, K, M, p->gm, y, s, sums);
            }
        }
    } else if (M <= GEMV_MAX_M) {
        e = launch_gemv(p->fmt, p->mode, w, x, p->N, K, (int)M, p->gv, y, s, tr);
    } else if (gemm_s_supported(p->fmt, p->mode, K, p->N, M)) {
        e = launch_gemm_s(p->fmt, p->mode, 1, &w, &p->N, &y, x, K, M, s, tr);  // short rows: one launch
    } else {
        e = launch_gemm_prep(p->fmt, p->mode, x, M, K, p->gm, s, act);
        if (e == hipSuccess) e = launch_gemm(p->fmt, p->mode, w, p->N, K, M, p->gm, y, s, sums);
    }
    if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
    return QMM_OK;
}

extern "C" int qmatmul_run(const qmm_plan* p, const void* w, const float* x, float* y, int64_t M, void* stream)
{
    g_err[0] = 0;
    int st = check_run(p, w, x, y, M);
    if (st != QMM_OK || M == 0) return st;
    return run_impl(p, w, x, y, nullptr, M, stream);
}

// The plan-free run of the no-allocation entry point (qmm_noalloc.hip): the
// same checks and kernels as create + run, with the workspace laid out in the
// caller's device memory `scratch` of `scratch_bytes` bytes.  dry_run: the
// checks only (no HIP call).
int qmm::run_on_scratch(int format, int64_t N, int64_t K, int64_t M, int mode, const void* w, const float* x,
                        float* y, void* scratch, size_t scratch_bytes, void* stream, bool dry_run)
{
    g_err[0] = 0;
    int st = check_shape(format, N, K, M > 0 ? M : 1, mode);
    if (st != QMM_OK) return st;
    if (M < 0) return fail(QMM_EINVAL, "M=%lld is negative", (long long)M);
    if (M == 0) return QMM_OK;
    if (mode == QMM_MODE_DEQUANT)
        return fail(QMM_EUNSUPPORTED, "the dequantize-all form (mode 2) takes a library GEMM that allocates; "
                    "use qmatmul_create and qmatmul_run");
    qmm_plan p{};
    p.fmt = format;
    p.mode = mode;
    p.N = N;
    p.K = K;
    p.M_max = M;
    p.ws_bytes = layout(&p, nullptr);
    if (p.ws_bytes > scratch_bytes)
        return fail(QMM_EINVAL, "format %d N=%lld K=%lld M=%lld mode %d needs %zu bytes of scratch, more than the "
                    "%zu bytes of the static scratch buffer", format, (long long)N, (long long)K, (long long)M,
                    mode, p.ws_bytes, scratch_bytes);
    st = check_run(&p, w, x, y, M);
    if (st != QMM_OK || dry_run) return st;
    if (!scratch) return fail(QMM_EINVAL, "scratch is NULL");
    hipError_t e = hipGetDevice(&p.device);
    if (e != hipSuccess) return fail(QMM_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    p.ws = scratch;
    layout(&p, (char*)scratch);
    return run_impl(&p, w, x, y, nullptr, M, stream);
}

int qmm::set_error(int code, const char* msg)
{
    return fail(code, "%s", msg);
}

extern "C" int qmatmul_run_group(const qmm_plan* const* plans, int count, const void* const* w, const float* x,
                                 float* const* y, int64_t M, void* stream)
{
    g_err[0] = 0;
    if (!plans || !w || !y) return fail(QMM_EINVAL, "null array: plans=%p w=%p y=%p", (const void*)plans,
                                        (const void*)w, (const void*)y);
    if (count < 1 || count > QMM_GROUP_MAX) return fail(QMM_EINVAL, "count=%d outside [1, %d]", count, QMM_GROUP_MAX);
    for (int i = 0; i < count; ++i) {
        const int st = check_run(plans[i], w[i], x, y[i], M);
        if (st != QMM_OK) return st;
        if (plans[i]->fmt != plans[0]->fmt || plans[i]->K != plans[0]->K || plans[i]->mode != plans[0]->mode)
            return fail(QMM_EINVAL, "the plans of a group must share format, K and mode (plan %d differs from plan 0)",
                        i);
    }
    if (M == 0) return QMM_OK;
    const qmm_plan* p0 = plans[0];
    const hipStream_t s = (hipStream_t)stream;
    if (M == 1 && p0->mode != QMM_MODE_DEQUANT && p0->Kr == p0->K) {
        // one launch per gemv_row_group_max() plans, when the one-row kernel takes their rows
        int64_t total = 0;
        for (int i = 0; i < count; ++i) total += plans[i]->N;
        if (gemv_row_supported(p0->fmt, p0->mode, 1, total, p0->K, false)) {
            const int gmax = gemv_row_group_max();
            for (int i = 0; i < count; i += gmax) {
                const int c = count - i < gmax ? count - i : gmax;
                int64_t Ns[QMM_GROUP_MAX];
                for (int j = 0; j < c; ++j) Ns[j] = plans[i + j]->N;
                const hipError_t e = launch_gemv_row_group(p0->fmt, p0->mode, c, w + i, Ns, y + i, x, p0->K, s);
                if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
            }
            return QMM_OK;
        }
    }
    if (is_ext_format(p0->fmt) && p0->Kr == p0->K && ext_group_supported(p0->fmt, p0->mode, p0->K, M) &&
        !gemv_reg_supported(p0->fmt, p0->mode, (int)M, 1, p0->K)) {
        // Q4_0, Q5_0, Q6_K decode: one launch per ext_group_max() plans, unless
        // a plan's separate run would take the one-row or the register-operand
        // kernel (the grouped values must be those of the separate runs)
        int64_t total = 0;
        bool row_alone = false;
        for (int i = 0; i < count; ++i) {
            total += plans[i]->N;
            row_alone = row_alone || (M == 1 && gemv_row_supported(p0->fmt, p0->mode, 1, plans[i]->N, p0->K, false));
        }
        if (total <= (1ll << 30) && !row_alone) {
            const int gmax = ext_group_max();
            for (int i = 0; i < count; i += gmax) {
                const int c = count - i < gmax ? count - i : gmax;
                int64_t Ns[QMM_GROUP_MAX];
                for (int j = 0; j < c; ++j) Ns[j] = plans[i + j]->N;
                const hipError_t e =
                    launch_ext_group(p0->fmt, p0->mode, c, w + i, Ns, y + i, x, p0->K, M, plans[i]->ex, s);
                if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
            }
            return QMM_OK;
        }
    }
    if (M > GEMV_MAX_M && p0->mode != QMM_MODE_DEQUANT && p0->Kr == p0->K) {
        // prefill: the activations prepared once (in plan 0's workspace), then one
        // launch per gemm_group_max() plans; Q4_0/Q5_0 weights first rewritten as
        // Q8_0 blocks in each plan's workspace, as in their separate runs
        const int kf = p0->fmt == QMM_Q4_0 || p0->fmt == QMM_Q5_0 ? FMT_Q8_0 : p0->fmt;
        // Each plan takes the kernel its own run takes (so grouped outputs equal
        // separate runs bit for bit): plans with short rows and a one-round grid
        // go to the short-row kernel, which prepares its own activations; the
        // rest share one preparation and the K-staged kernels.
        int sp[QMM_GROUP_MAX], op[QMM_GROUP_MAX], ns = 0, no = 0;
        for (int i = 0; i < count; ++i) {
            if (gemm_s_supported(p0->fmt, p0->mode, p0->K, plans[i]->N, M)) sp[ns++] = i;
            else op[no++] = i;
        }
        hipError_t e = no > 0 ? launch_gemm_prep(kf, p0->mode, x, M, p0->K, p0->gm, s) : hipSuccess;
        for (int part = 0; part < 2; ++part) {
            const int* idx = part == 0 ? sp : op;
            const int cnt = part == 0 ? ns : no;
            const int gmax = part == 0 ? PG_GROUP_S : gemm_group_max();
            for (int i = 0; i < cnt && e == hipSuccess; i += gmax) {
                const int c = cnt - i < gmax ? cnt - i : gmax;
                const void* wk[QMM_GROUP_MAX];
                int64_t Ns[QMM_GROUP_MAX];
                float* ys[QMM_GROUP_MAX];
                for (int j = 0; j < c && e == hipSuccess; ++j) {
                    const int q = idx[i + j];
                    const qmm_plan* pj = plans[q];
                    Ns[j] = pj->N;
                    wk[j] = w[q];
                    ys[j] = y[q];
                    if (part == 1 && kf != p0->fmt) {  // Q4_0/Q5_0: rewritten as Q8_0 blocks, as in their separate runs
                        e = launch_ext_to_q8_0(pj->fmt, w[q], pj->N, pj->K, pj->ex.tw, s);
                        wk[j] = pj->ex.tw;
                    }
                }
                if (e == hipSuccess)
                    e = part == 0 ? launch_gemm_s(p0->fmt, p0->mode, c, wk, Ns, ys, x, p0->K, M, s)
                                  : launch_gemm_group(kf, p0->mode, c, wk, Ns, ys, p0->K, M, p0->gm, s);
            }
        }
        if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
        return QMM_OK;
    }
    for (int i = 0; i < count; ++i) {
        const int st = run_impl(plans[i], w[i], x, y[i], nullptr, M, stream);
        if (st != QMM_OK) return st;
    }
    return QMM_OK;
}

extern "C" int qmatmul_run_traced(const qmm_plan* p, const void* w, const float* x, float* y, int32_t* sums,
                                  void* act_blocks, int64_t M, void* stream)
{
    g_err[0] = 0;
    int st = check_run(p, w, x, sums, M);
    if (st != QMM_OK || M == 0) return st;
    if (p->mode != QMM_MODE_QACT) return fail(QMM_EUNSUPPORTED, "block sums exist only for quantized activations (mode 1)");
    if (y && !aligned(y, 4)) return fail(QMM_EINVAL, "y must be 4-byte aligned");
    if (act_blocks && !aligned(act_blocks, 4)) return fail(QMM_EINVAL, "act_blocks must be 4-byte aligned");
    if (p->Kr == p->K) {
        const Trace tr{sums, (uint8_t*)act_blocks};
        return run_impl(p, w, x, y, &tr, M, stream);
    }
    // padded rows: the kernels' outputs (one block more per row) go to
    // stream-ordered temporaries, then the real blocks are copied out
    hipStream_t s = (hipStream_t)stream;
    const int64_t from = p->Kr / 32, keep = p->K / 32;
    void* ts = nullptr;
    void* ta = nullptr;
    hipError_t e = hipMallocAsync(&ts, (size_t)M * p->N * from * 4, s);
    if (e == hipSuccess) e = hipMallocAsync(&ta, (size_t)M * from * 34, s);
    if (e != hipSuccess) {
        if (ts) (void)hipFreeAsync(ts, s);
        return fail(e == hipErrorOutOfMemory ? QMM_ENOMEM : QMM_EHIP, "hipMallocAsync: %s", hipGetErrorString(e));
    }
    const Trace tr{(int32_t*)ts, (uint8_t*)ta};
    st = run_impl(p, w, x, y, &tr, M, stream);
    if (st == QMM_OK) {
        e = launch_unpad(ts, M * p->N, (int)from, (int)keep, 4, sums, s);
        if (e == hipSuccess && act_blocks) e = launch_unpad(ta, M, (int)from, (int)keep, 34, act_blocks, s);
        if (e != hipSuccess) st = fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
    }
    (void)hipFreeAsync(ts, s);
    (void)hipFreeAsync(ta, s);
    return st;
}

extern "C" int qmatmul_run_block_sums(const qmm_plan* p, const void* w, const float* x, int32_t* sums, int64_t M,
                                      void* stream)
{
    return qmatmul_run_traced(p, w, x, nullptr, sums, nullptr, M, stream);
}

extern "C" int qmatmul_run_dequantized(const qmm_plan* p, const float* w, const float* x, float* y, int64_t M,
                                       void* stream)
{
    g_err[0] = 0;
    int st = check_run(p, w, x, y, M);
    if (st != QMM_OK || M == 0) return st;
    if (p->mode != QMM_MODE_DEQUANT)
        return fail(QMM_EUNSUPPORTED, "f32 weights need a dequantize-all plan (mode 2)");
    st = dense_gemm(p->dense, w, x, y, M, p->N, p->K, (hipStream_t)stream);
    if (st != 0) return fail(QMM_EHIP, "rocblas_sgemm: status %d", st);
    return QMM_OK;
}

extern "C" int qmatmul_dequantize_weights(int format, const void* w, int64_t N, int64_t K, float* out, void* stream)
{
    g_err[0] = 0;
    if (!weight_format(format)) return fail(QMM_EUNSUPPORTED, "unsupported weight format %d", format);
    if (N < 0 || K <= 0) return fail(QMM_EINVAL, "bad sizes N=%lld K=%lld", (long long)N, (long long)K);
    if (K % block_values(format))
        return fail(QMM_EBLOCK, "quantized tensor must have their last dim divisible by block size [%lld, %lld] %lld",
                    (long long)N, (long long)K, (long long)block_values(format));
    if (N == 0) return QMM_OK;
    if (!w || !out) return fail(QMM_EINVAL, "null pointer");
    if (!aligned(w, 16)) return fail(QMM_EINVAL, "w_blocks must be 16-byte aligned");
    if (!aligned(out, 16)) return fail(QMM_EINVAL, "out must be 16-byte aligned");
    hipError_t e = is_ext_format(format) ? launch_ext_dequantize(format, w, N, K, out, (hipStream_t)stream)
                                         : launch_dequantize(format, w, N, K, out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
    return QMM_OK;
}

extern "C" int qmatmul_quantize_act(int act_format, const float* x, int64_t M, int64_t K, void* out, void* stream)
{
    g_err[0] = 0;
    if (act_format != QMM_Q8_0 && act_format != QMM_Q8_K)
        return fail(QMM_EUNSUPPORTED, "unsupported activation format %d (expected %d Q8_0 or %d Q8_K)", act_format,
                    QMM_Q8_0, QMM_Q8_K);
    if (M < 0 || K <= 0) return fail(QMM_EINVAL, "bad sizes M=%lld K=%lld", (long long)M, (long long)K);
    if (K % block_values(act_format))
        return fail(QMM_EBLOCK, "last dim %lld not divisible by block size %lld", (long long)K,
                    (long long)block_values(act_format));
    if (M == 0) return QMM_OK;
    if (!x || !out) return fail(QMM_EINVAL, "null pointer");
    if (!aligned(x, 16)) return fail(QMM_EINVAL, "x must be 16-byte aligned");
    if (!aligned(out, 4)) return fail(QMM_EINVAL, "out_blocks must be 4-byte aligned");
    hipError_t e = launch_quantize_act(act_format, x, M, K, out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
    return QMM_OK;
}

extern "C" int qmatmul_quantize_weights(int format, const float* w, int64_t N, int64_t K, void* out, void* stream)
{
    g_err[0] = 0;
    if (!weight_format(format)) return fail(QMM_EUNSUPPORTED, "unsupported weight format %d", format);
    if (N < 0 || K <= 0) return fail(QMM_EINVAL, "bad sizes N=%lld K=%lld", (long long)N, (long long)K);
    if (K % block_values(format))
        return fail(QMM_EBLOCK, "quantized tensor must have their last dim divisible by block size [%lld, %lld] %lld",
                    (long long)N, (long long)K, (long long)block_values(format));
    if (N == 0) return QMM_OK;
    if (!w || !out) return fail(QMM_EINVAL, "null pointer");
    if (!aligned(w, 16)) return fail(QMM_EINVAL, "w must be 16-byte aligned");
    if (!aligned(out, 16)) return fail(QMM_EINVAL, "out_blocks must be 16-byte aligned");
    hipError_t e = is_ext_format(format) ? launch_ext_quantize_weights(format, w, N, K, out, (hipStream_t)stream)
                                         : launch_quantize_weights(format, w, N, K, out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
    return QMM_OK;
}

extern "C" int qmatmul_quantize_q4_k_search(const float* w, int64_t N, int64_t K, void* out, void* stream)
{
    g_err[0] = 0;
    if (N < 0 || K <= 0) return fail(QMM_EINVAL, "bad sizes N=%lld K=%lld", (long long)N, (long long)K);
    if (K % 256)
        return fail(QMM_EBLOCK, "quantized tensor must have their last dim divisible by block size [%lld, %lld] 256",
                    (long long)N, (long long)K);
    if (N == 0) return QMM_OK;
    if (!w || !out) return fail(QMM_EINVAL, "null pointer");
    if (!aligned(w, 16)) return fail(QMM_EINVAL, "w must be 16-byte aligned");
    if (!aligned(out, 16)) return fail(QMM_EINVAL, "out_blocks must be 16-byte aligned");
    hipError_t e = launch_quantize_q4_k_search(w, N, K, out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(QMM_EHIP, "kernel launch: %s", hipGetErrorString(e));
    return QMM_OK;
}

extern "C" const char* qmatmul_status_string(int status)
{
    switch (status) {
    case QMM_OK: return "ok";
    case QMM_EINVAL: return "invalid argument";
    case QMM_EBLOCK: return "K is not a multiple of the block size";
    case QMM_EUNSUPPORTED: return "unsupported format, mode or shape";
    case QMM_ENOMEM: return "out of device memory";
    case QMM_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

extern "C" const char* qmatmul_last_error(void) { return g_err; }

extern "C" int qmatmul_version(void) { return 1; }
