// qmm_gemv_row.hip -- decode kernel for one activation row (M == 1), mode (b),
// Q8_0 weights.
//
// Mode (b) is the CPU form of page "同一个 GGUF，CPU 和 Metal 生成的文字不一样"
// (section 出处): the activation row is quantized per 32 values to Q8_0 (page
// "自己量化", section 和下载的 Q8_0 逐字节比), and
//     y[n] = sum over blocks b of  d_w[n][b] * d_x[b] * S[n][b],
// S being the int8 dot product of the weight block with the activation block.
//
// With a single activation row no weight byte is used twice: the kernel is a
// weight stream, laid out for what this chip's memory system rewards.
//   * Every weight row is read as one contiguous run: 16-byte non-temporal
//     loads, 1 KB per instruction, landing directly in LDS (lane i of a load
//     writes its base + 16 i).  Wave g of W takes rows g, g + W, g + 2W, ...,
//     so at any moment the whole chip reads one contiguous window of the
//     matrix.  A plain read of the 14336 x 4096 Q8_0 matrix (eight copies
//     rotated) in this order runs at about 6.2 TB/s, against about 5.3 TB/s
//     for 16-row tiles read 272 bytes of each row at a time.
//   * A row is cut into segments of up to 64 block pairs (4352 bytes).  Lane l
//     owns pair l of a segment: it reads the pair's 68 bytes from LDS, aligns
//     the even block's values (they start two bytes into a dword) and takes
//     both int8 dot products with v_dot4 against the activation pair it holds
//     in registers.
//   * Each wave has a ring of two segment buffers, so the next segment's loads
//     are in flight while the current one is summed.  Every segment issues the
//     same number of load instructions with every lane on (lanes past the
//     segment re-read its first bytes into the buffer's tail), which keeps the
//     explicit waits exact and the issue free of branches.
//   * The activation row is brought into LDS ahead of the stream and
//     quantized once per workgroup with the device functions every other Q8_0
//     activation quantizer uses, so its blocks are the same bytes; each lane
//     then holds its activation pairs in registers for all of its rows.
//   * A row's per-lane f32 sums are added across the wave in a fixed order:
//     a run is deterministic.
#include <algorithm>
#include <mutex>
#include <set>
#include <utility>

#include "qmm_act.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int GR_WAVES = 8;
constexpr int GR_THREADS = 64 * GR_WAVES;
constexpr int GR_SEG_PAIRS = 64;                 // block pairs per segment, one per lane
constexpr int GR_SEG_BYTES = 68 * GR_SEG_PAIRS;  // 4352
constexpr int GR_RING = 2;                       // segment buffers per wave
constexpr int GR_SLOT_MAX = 5 * 1024;            // a segment buffer: its load instructions x 1 KB
constexpr int GR_NSEG_MAX = 4;                   // segments per row (K <= 16384)
constexpr int GR_LDS_MAX = 160 * 1024;

struct GemvRowArgs {
    const uint8_t* w;
    const float* x;
    float* y;
    int N, K;
    int row_bytes;  // K/32 blocks of 34 bytes
    int npair;      // K/64 block pairs per row
    int nxi;        // 1 KB load instructions that bring x into LDS
    int xq_off, xd_off, ring_off;  // LDS byte offsets (f32 x staged at 0)
};

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// 16 bytes per lane from src (per lane) to LDS at dst + 16 * lane (dst the same
// in every lane).  AUX 2: non-temporal (the weight stream is read once).
template <int AUX>
QMM_DEV void ldg16_lds(const uint8_t* src, uint8_t* dst)
{
    __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)dst, 16, 0, AUX);
}

// Sum over the wave in a fixed order, the same value in every lane: within each
// 16-lane row by lane exchanges, then the four rows.
QMM_DEV float wave_sum(float v)
{
    v += dpp_f<DPP_X1>(v);
    v += dpp_f<DPP_X2>(v);
    v += dpp_f<DPP_HMIRROR>(v);
    v += dpp_f<DPP_MIRROR>(v);
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// LPU: load instructions per segment, ceil(min(row bytes, 4352) / 1024); a
// segment buffer holds LPU KB.  NSEG: segments per row.  Every global load of
// the kernel writes LDS directly, so all waits on them are the explicit ones.
template <int LPU, int NSEG>
__global__ __launch_bounds__(GR_THREADS) void gemv_row_q8_0_kernel(GemvRowArgs a)
{
    constexpr int SLOT = 1024 * LPU;
    extern __shared__ __align__(16) uint8_t lds[];
    const float* s_xf = reinterpret_cast<const float*>(lds);
    int8_t* s_xq = reinterpret_cast<int8_t*>(lds + a.xq_off);
    float* s_xd = reinterpret_cast<float*>(lds + a.xd_off);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = (int)gridDim.x * GR_WAVES, gw = (int)blockIdx.x * GR_WAVES + wave;
    const int N = a.N, K = a.K;
    const int nrows = gw < N ? (N - 1 - gw) / nw + 1 : 0;  // rows gw, gw + nw, ...
    const int U = nrows * NSEG;                             // segments this wave streams
    uint8_t* ring = lds + a.ring_off + wave * (GR_RING * SLOT);

    // ---- x (f32) into LDS first, so it is not queued behind the stream ----
    {
        const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x);
        const int xbytes = 4 * K;
        for (int i = wave; i < a.nxi; i += GR_WAVES) {
            const int off = 1024 * i + 16 * lane;  // past the end: x's first bytes again, into the pad
            ldg16_lds<0>(xb + (off < xbytes ? off : 0), lds + 1024 * i);
        }
    }

    // ---- the first segments of the stream (they need no activations) ----
    // segment u of this wave into ring buffer `slot`; a wave with fewer than two
    // segments loads its last row (or the matrix's) again for the missing ones.
    // Every lane loads: lanes past the segment re-read its first bytes into the
    // buffer's tail, so each segment is exactly LPU instructions.
    auto issue = [&](int u, int slot) {
        const int j = u / NSEG, sg = u - j * NSEG;
        const int row = min(gw + nw * j, N - 1);
        const uint8_t* src = a.w + (int64_t)row * a.row_bytes + sg * GR_SEG_BYTES;
        const int bytes = min(GR_SEG_BYTES, a.row_bytes - sg * GR_SEG_BYTES);
        uint8_t* dst = ring + slot * SLOT;
#pragma unroll
        for (int t = 0; t < LPU; ++t) {
            const int off = 1024 * t + 16 * lane;
            ldg16_lds<2>(src + (off < bytes ? off : 0), dst + 1024 * t);
        }
    };
#pragma unroll
    for (int u = 0; u < GR_RING; ++u) issue(u < U ? u : max(U - 1, 0), u);

    // ---- quantize x: 8 values per task, the four tasks of a 32-value block a lane quad ----
    vm_wait<GR_RING * LPU>();  // this wave's share of x has landed (loads retire in order)
    asm volatile("s_barrier" ::: "memory");  // ... and every other wave's
    for (int t = tid; t < K / 8; t += GR_THREADS) {
        const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(s_xf + 8 * t);
        const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(s_xf + 8 * t + 4);
        const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
        am = fmaxf(am, dpp_f<DPP_X1>(am));
        am = fmaxf(am, dpp_f<DPP_X2>(am));
        float id, dval;
        uint16_t dbits;
        q8_0_scale(am, id, dbits, dval);
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = q8_0_q(v[i], id);
        *reinterpret_cast<u32x2_t*>(s_xq + 8 * t) = u32x2_t{pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7])};
        if ((t & 3) == 0) s_xd[t >> 2] = dval;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- this lane's activation pairs (pair sg*64 + lane of each segment), held for every row ----
    int X[NSEG][16];
    float DX[NSEG][2];
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
        const int p = min(sg * GR_SEG_PAIRS + lane, a.npair - 1);
        const u32x4_t* q = reinterpret_cast<const u32x4_t*>(s_xq + 64 * p);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4_t v = q[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) X[sg][4 * c + e] = (int)v[e];
        }
        DX[sg][0] = s_xd[2 * p];
        DX[sg][1] = s_xd[2 * p + 1];
    }

    // ---- the stream ----
    float yv = 0.0f;
    int u = 0;
    for (int j = 0; j < nrows; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int sg = 0; sg < NSEG; ++sg, ++u) {
            const int slot = u & 1;
            vm_wait_ahead<LPU, GR_RING - 1>(min(GR_RING - 1, U - 1 - u));  // segment u has landed
            const int pairs = min(GR_SEG_PAIRS, a.npair - sg * GR_SEG_PAIRS);
            if (lane < pairs) {
                const uint32_t* wp = reinterpret_cast<const uint32_t*>(ring + slot * SLOT + 68 * lane);
                uint32_t W[17];
#pragma unroll
                for (int k = 0; k < 17; ++k) W[k] = wp[k];
                // even block: d in bytes 0-1, values in 2-33; odd block: d in 34-35, values in 36-67
                int s0 = 0, s1 = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    s0 = __builtin_amdgcn_sdot4((int)__builtin_amdgcn_alignbyte(W[k + 1], W[k], 2), X[sg][k], s0, false);
                    s1 = __builtin_amdgcn_sdot4((int)W[9 + k], X[sg][8 + k], s1, false);
                }
                acc = fmaf((float)s0, f16lo(W[0]) * DX[sg][0], acc);
                acc = fmaf((float)s1, f16hi(W[8]) * DX[sg][1], acc);
            }
            if (u + GR_RING < U) {
                lgkm_wait0();  // this buffer's reads are done before it is refilled
                issue(u + GR_RING, slot);
            }
        }
        // the row is complete: add the lanes' sums (fixed order), park it in lane j % 64;
        // outputs leave 64 rows at a time, or after the last row
        const float t = wave_sum(acc);
        if (lane == (j & 63)) yv = t;
        if ((j & 63) == 63 || j == nrows - 1) {
            const int j0 = j & ~63;
            if (lane <= (j & 63)) a.y[gw + nw * (j0 + lane)] = yv;
        }
    }
}

typedef void (*GrKernel)(GemvRowArgs);

static GrKernel gr_kernel(int lpu, int nseg)
{
    if (nseg == 4) return gemv_row_q8_0_kernel<5, 4>;
    if (nseg == 3) return gemv_row_q8_0_kernel<5, 3>;
    if (nseg == 2) return gemv_row_q8_0_kernel<5, 2>;
    switch (lpu) {
    case 1: return gemv_row_q8_0_kernel<1, 1>;
    case 2: return gemv_row_q8_0_kernel<2, 1>;
    case 3: return gemv_row_q8_0_kernel<3, 1>;
    case 4: return gemv_row_q8_0_kernel<4, 1>;
    default: return gemv_row_q8_0_kernel<5, 1>;
    }
}

// LDS layout: x as f32 (padded to whole 1 KB loads), x as int8, the x block
// scales, then the eight waves' segment rings.
struct GrLayout {
    int nxi, xq_off, xd_off, ring_off, bytes;
};
static GrLayout gr_layout(int64_t K)
{
    GrLayout l{};
    l.nxi = (int)((4 * K + 1023) / 1024);
    l.xq_off = 1024 * l.nxi;
    l.xd_off = l.xq_off + (int)K;
    l.ring_off = (l.xd_off + (int)(K / 8) + 15) / 16 * 16;
    l.bytes = l.ring_off + GR_WAVES * GR_RING * GR_SLOT_MAX;
    return l;
}

bool gemv_row_supported(int fmt, int mode, int M, int64_t K, bool emit)
{
    return fmt == FMT_Q8_0 && mode == MODE_B && M == 1 && !emit && K % 64 == 0 &&
           K <= (int64_t)GR_NSEG_MAX * GR_SEG_PAIRS * 64 && gr_layout(K).bytes <= GR_LDS_MAX;
}

hipError_t launch_gemv_row(int fmt, const void* w, const float* x, int64_t N, int64_t K, float* y, hipStream_t s)
{
    if (!gemv_row_supported(fmt, MODE_B, 1, K, false) || N <= 0 || N > 0x7fffffff) return hipErrorInvalidValue;
    const GrLayout l = gr_layout(K);
    GemvRowArgs a{};
    a.w = (const uint8_t*)w;
    a.x = x;
    a.y = y;
    a.N = (int)N;
    a.K = (int)K;
    a.row_bytes = (int)(K / 32 * 34);
    a.npair = (int)(K / 64);
    a.nxi = l.nxi;
    a.xq_off = l.xq_off;
    a.xd_off = l.xd_off;
    a.ring_off = l.ring_off;
    const int nseg = (a.npair + GR_SEG_PAIRS - 1) / GR_SEG_PAIRS;
    const int lpu = (std::min(a.row_bytes, GR_SEG_BYTES) + 1023) / 1024;
    // the fewest rows per wave that spread N over every compute unit, then the
    // workgroups that this takes
    const int64_t cus = device_cus();
    const int64_t rpw = (N + GR_WAVES * cus - 1) / (GR_WAVES * cus);
    const int64_t grid = (N + GR_WAVES * rpw - 1) / (GR_WAVES * rpw);
    const GrKernel k = gr_kernel(lpu, nseg);
    static std::set<std::pair<int, const void*>> done;  // dynamic LDS above 64 KB, once per device
    static std::mutex mu;
    {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        std::lock_guard<std::mutex> lock(mu);
        if (done.insert(std::make_pair(dev, (const void*)k)).second) {
            (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, GR_LDS_MAX);
            (void)hipGetLastError();
        }
    }
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel((const void*)k, dim3((unsigned)grid), dim3(GR_THREADS), args, l.bytes, s);
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace qmm
