// qmm_gemv.hip -- decode kernel (M <= 8) for y = x . W^T on GGUF blocks: the
// launchers, the geometry, the split-K reduction and the mode (a) instances of
// the kernel in qmm_gemv_kernel.h.
#include <algorithm>
#include <map>
#include <mutex>
#include <set>
#include <utility>

#include "qmm_gemv_kernel.h"

namespace qmm {

// Split-K: y[m][n] = sum over K splits of the partials, in split order.
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float* __restrict__ part, int ks, int M, int N,
                                                          float* __restrict__ y)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int m = (int)(i / N), n = (int)(i - (int64_t)m * N);
    float s = 0.0f;
    for (int sp = 0; sp < ks; ++sp) s += part[((int64_t)sp * GEMV_MAX_M + m) * N + n];
    y[i] = s;
}

// ------------------------------------------------------------- kernels ----

// Stage sizes (load units) compiled for each format.  The LDS-direct ring
// (up to kRingMax stage buffers per wave) is compiled for the stage sizes whose
// rows are an odd number of 16-byte chunks: then the unpadded row-major stage
// layout starts the 16 rows in different banks, as the padded one does.
static const int kStageQ8[] = {4, 3, 2, 1};
static const int kStageQ4[] = {2, 3, 1};
static const int kNStageQ8 = 4, kNStageQ4 = 3;

static GvKernel gv_kernel(int fmt, int mode, int P, int R, bool emit, int D)
{
    if (mode == MODE_B) return emit ? gv_kernel_emit(fmt, P, R, D) : gv_kernel_b(fmt, P, R, D);
    return fmt == FMT_Q8_0 ? gv_pick<FMT_Q8_0, MODE_A, false>(P, R, D) : gv_pick<FMT_Q4_K, MODE_A, false>(P, R, D);
}

// Compute units of the current device, cached per device.
int device_cus()
{
    static std::map<int, int> cache;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
    (void)hipGetLastError();
    return cache[dev] = cus;
}

// Raises a kernel's dynamic LDS limit to the full 160 KB, once per device.
static void allow_full_lds(GvKernel k)
{
    static std::set<std::pair<int, const void*>> done;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!done.insert(std::make_pair(dev, (const void*)k)).second) return;
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, GV_LDS_MAX);
    (void)hipGetLastError();
}

// ------------------------------------------------------------- geometry ----

bool gemv_supported(int fmt, int64_t K)
{
    return (fmt == FMT_Q4_K || fmt == FMT_Q6_K) ? K % 256 == 0 : K % 64 == 0;
}

// LDS bytes of the eight waves' weight stage buffers (one each, register staging).
static int stage_bytes(int fmt, int P) { return GV_WAVES * 16 * (fmt == FMT_Q8_0 ? gv_rs(FMT_Q8_0, P) : gv_rs(FMT_Q4_K, P)); }

// K splits of one run: enough that the activation operand of a split (with
// the smallest weight stage) fits in LDS and one workgroup prepares at most
// 64 values per thread.
static int gemv_splits(int fmt, int mode, int64_t K, int M, int ms, int& lus_split)
{
    int lub, ops, vpl, opb, scb;
    gv_fmt(fmt, mode, ms, lub, ops, vpl, opb, scb);
    const int64_t nlu = K / vpl;
    const int64_t per_lu = (int64_t)ops * opb + scb;
    const int64_t room = GV_LDS_MAX - GV_RED_BYTES - GV_MISC_BYTES - stage_bytes(fmt, 1);
    const int64_t lus_max = std::max<int64_t>(1, std::min<int64_t>(room / per_lu, GV_XMAX / ((int64_t)M * vpl)));
    const int64_t ks = (nlu + lus_max - 1) / lus_max;
    lus_split = (int)((nlu + ks - 1) / ks);
    return (int)ks;
}

int gemv_max_splits(int fmt, int64_t K)
{
    int l;
    int ks = 1;
    for (int mode = 0; mode < 2; ++mode)
        for (int M = 1; M <= GEMV_MAX_M; ++M) ks = std::max(ks, gemv_splits(fmt, mode, K, M, M == 1 ? 1 : 8, l));
    return ks;
}

// Geometry of one run: K splits, waves per tile (kw), stage size (P) and tile
// groups per workgroup (gpw), chosen to minimise the work of the busiest
// compute unit: the workgroups it runs times (the prologue, which loads and
// prepares the activations once per workgroup, plus the busiest wave's stages,
// priced by the 16-byte chunks they load plus a fixed overhead).  The prologue
// term makes one workgroup per compute unit beat two half-sized ones.  Ties go
// to larger stages, then to fewer waves per tile, then to more workgroups.
GemvGeom gemv_geom(int fmt, int mode, int64_t N, int64_t K, int M, bool emit)
{
    GemvGeom g{};
    (void)emit;  // a traced run takes the geometry of the plain run
    g.R = M == 1 ? 1 : 4;
    const int ms = g.R == 1 ? 1 : 8;
    int lub, ops, vpl, opb, scb;
    gv_fmt(fmt, mode, ms, lub, ops, vpl, opb, scb);
    g.nlu = (int)(K / vpl);
    g.row_bytes = (int64_t)g.nlu * lub;
    g.tiles = (int)((N + 15) / 16);
    g.ks = gemv_splits(fmt, mode, K, M, ms, g.lus_split);
    const int* stages = fmt == FMT_Q8_0 ? kStageQ8 : kStageQ4;
    const int nstages = fmt == FMT_Q8_0 ? kNStageQ8 : kNStageQ4;
    const int64_t cus = device_cus();
    // prologue price: a fixed part plus one unit per activation value it prepares
    const int64_t pro = 8192 + (int64_t)M * g.lus_split * vpl;
    int64_t best = -1;
    for (int kw = 1; kw <= GV_WAVES; kw *= 2) {
        for (int si = 0; si < nstages; ++si) {
            const int P = stages[si];
            const int raw = (g.lus_split + kw - 1) / kw;
            const int slice = (raw + P - 1) / P * P;
            if ((kw - 1) * slice >= g.lus_split) continue;  // an empty slice
            const int G = GV_WAVES / kw;
            const int groups = (g.tiles + G - 1) / G;
            const int img = kw * slice * ops * opb;
            const int sc = kw * slice * scb;
            const int fixed = img + sc + GV_RED_BYTES + GV_MISC_BYTES;
            // the deepest LDS-direct ring that fits, else one register-staged buffer per wave
            int D = 0;
            if (gv_ring_ok(fmt, P))
                for (int d = kRingMax; d >= kRingMin && !D; --d)
                    if (fixed + d * stage_bytes(fmt, P) <= GV_LDS_MAX) D = d;
            const int lds = fixed + (D > 0 ? D : 1) * stage_bytes(fmt, P);
            if (lds > GV_LDS_MAX) continue;
            const int cpr = fmt == FMT_Q8_0 ? gv_cpr(FMT_Q8_0, P) : gv_cpr(FMT_Q4_K, P);
            const int64_t loop = (int64_t)(slice / P) * (256 * cpr + 512);
            for (int gpw = 1; gpw <= GV_GPW_MAX; ++gpw) {
                const int64_t grid = (int64_t)g.ks * ((groups + gpw - 1) / gpw);
                const int64_t cost = (grid + cus - 1) / cus * (pro + gpw * loop);
                if (best >= 0 && !(cost < best || (cost == best && P > g.P))) continue;
                best = cost;
                g.kw = kw;
                g.slice = slice;
                g.P = P;
                g.G = G;
                g.groups = groups;
                g.gpw = gpw;
                g.rs = fmt == FMT_Q8_0 ? gv_rs(FMT_Q8_0, P) : gv_rs(FMT_Q4_K, P);
                g.D = D;
                g.sc_off = img;
                g.red_off = img + sc;
                g.misc_off = g.red_off + GV_RED_BYTES;
                g.stg_off = g.misc_off + GV_MISC_BYTES;
                g.lds = lds;
                g.grid = g.ks * ((groups + gpw - 1) / gpw);
            }
        }
    }
    return g;
}

// ------------------------------------------------------------ launchers ----

hipError_t launch_gemv(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, int M,
                       const GemvBufs& b, float* y, hipStream_t s, const Trace* tr)
{
    const bool emit = tr != nullptr;
    if (emit && mode != MODE_B) return hipErrorInvalidValue;
    if (gemv_row_supported(fmt, mode, M, N, K, emit)) return launch_gemv_row(fmt, mode, w, x, N, K, y, s, tr);
    if (!emit && gemv_reg_supported(fmt, mode, M, N, K)) return launch_gemv_reg(fmt, mode, w, x, N, K, M, y, s, nullptr);
    const GemvGeom g = gemv_geom(fmt, mode, N, K, M, emit);
    if (g.grid <= 0) return hipErrorInvalidConfiguration;
    GemvArgs a{};
    a.w = (const uint8_t*)w;
    a.w_bytes = N * g.row_bytes;
    a.row_bytes = (int)g.row_bytes;
    a.N = (int)N;
    a.K = (int)K;
    a.M = M;
    a.nlu = g.nlu;
    a.lus_split = g.lus_split;
    a.ks = g.ks;
    a.kw = g.kw;
    a.slice = g.slice;
    a.G = g.G;
    a.groups = g.groups;
    a.gpw = g.gpw;
    a.sc_off = g.sc_off;
    a.red_off = g.red_off;
    a.misc_off = g.misc_off;
    a.stg_off = g.stg_off;
    a.x = x;
    a.part = b.part;
    a.y = y;
    a.sums = emit ? tr->sums : nullptr;
    a.act = emit ? tr->act : nullptr;
    GvKernel k = gv_kernel(fmt, mode, g.P, g.R, emit, g.D);
    allow_full_lds(k);
    void* args[] = {&a};
    hipError_t e = hipLaunchKernel((const void*)k, dim3(g.grid), dim3(GV_THREADS), args, g.lds, s);
    if (e != hipSuccess) return e;
    if (y != nullptr && g.ks > 1) {
        const int64_t total = (int64_t)M * N;
        hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, b.part, g.ks,
                           M, (int)N, y);
    }
    return hipGetLastError();
}

}  // namespace qmm
