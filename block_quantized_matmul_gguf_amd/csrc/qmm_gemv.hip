// qmm_gemv.hip -- decode kernel (M <= 8) for y = x . W^T on GGUF blocks.
//
// The weight stream is the cost (the pages' CPU decode step is dominated by
// it: page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 修法, 7 ms
// Q8_0 vs 15 ms dequantized f32).  Layout of the work:
//   * the weight matrix is cut into units of 16 rows x one K split; the grid
//     is sized so every workgroup is resident at once, and each wave owns a
//     contiguous run of units, streaming them stage by stage with two stages
//     of 16-byte coalesced loads in flight (across unit boundaries), through a
//     private LDS stage from which every lane reads one row's bytes in the
//     matrix-core operand layout;
//   * all four waves of a workgroup share one K split, whose activation
//     operand the workgroup prepares once in LDS (mode a: f16 hi/lo split;
//     mode b: Q8_0 / Q8K quantization of each row);
//   * mode (a): v_mfma_f32_16x16x32_f16 with the weights as exact f16 integers
//     (q for Q8_0, the 4-bit q for Q4_K) against activation rows 0..7 = f16 hi
//     part and rows 8..15 = f16 lo part, block scales applied per block in f32;
//   * mode (b): v_mfma_i32_16x16x64_i8 over two 32-value blocks at once (A rows
//     0..7 carry the first block, 8..15 the second, zero elsewhere), giving the
//     int32 block sums; scaled in f32 (Q8_0: dw*dx*S; Q4_K: sub-block scales in
//     int32, then dx*(d*sumi - dmin*summins));
//   * with several K splits, partials go to a workspace and a small second
//     kernel sums them in a fixed order (deterministic; no cross-workgroup
//     fences).
#include <algorithm>
#include <mutex>

#include "qmm_act.h"

namespace qmm {

#ifndef QMM_NT_WEIGHTS
#define QMM_NT_WEIGHTS 1
#endif

constexpr int MAXP = 10;          // 16-byte staging pieces per lane and stage
constexpr int IMG_BYTES = 32768;  // activation operand of one K split
constexpr int SC_WORDS = 1024;    // per-split activation scales / sums
constexpr int MAX_RANGE = 4096;   // K values per split

struct GemvArgs {
    const uint8_t* w;
    int64_t row_bytes;
    int N, K, M;
    int units;      // weight units (32-blocks or 256-super-blocks) per row
    int ups;        // units per K split
    int ks;         // K splits
    int full_rows;  // 1: a stage is whole rows (ks == 1; the 16-row tile is contiguous)
    int su;         // units per stage otherwise
    int upw;        // row tiles per wave
    int tiles;      // ceil(N / 16)
    const float* x;
    float* part;
    float* y;
    int32_t* sums;
};

#define WAVE_SYNC()                                 \
    do {                                            \
        __atomic_signal_fence(__ATOMIC_SEQ_CST);    \
        __builtin_amdgcn_wave_barrier();            \
        __atomic_signal_fence(__ATOMIC_SEQ_CST);    \
    } while (0)

// Weight stream loads: a raw buffer descriptor per (tile, stage) whose record
// count ends at the last real row, so rows past N read as zeros (the range
// check is per dword and whole-row stages end on a dword boundary); non-
// temporal, since every weight byte is used once per run.  Every load path is
// branch-free, so the in-order load counter waits are exact.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
QMM_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
QMM_DEV float4 load_x16(rsrc_t r, uint32_t off)
{
    const f32x4_t v = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    return make_float4(v[0], v[1], v[2], v[3]);
}
QMM_DEV uint4 load_w16(rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, QMM_NT_WEIGHTS ? 2 : 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int FMT, int MODE, bool EMIT>
__global__ __launch_bounds__(256, 2) void gemv_kernel(GemvArgs a)
{
    constexpr int UB = FMT == FMT_Q8_0 ? 34 : 144;
    constexpr int QK = FMT == FMT_Q8_0 ? 32 : 256;
    // LDS sized per mode: the f16 hi/lo operand is 4 bytes per value and row,
    // the int8 one 1; scales [unit][8], Q4_K sums [sub-block or unit][8(x8)]
    constexpr int IMG = MODE == MODE_A ? IMG_BYTES : IMG_BYTES / 4;
    constexpr int SC0 = MODE == MODE_A ? 256 : (FMT == FMT_Q8_0 ? SC_WORDS : 128);
    constexpr int SC1 = FMT == FMT_Q4_K ? SC_WORDS : 4;
    __shared__ __align__(16) uint8_t s_img[IMG];
    __shared__ __align__(16) float s_sc0[SC0];
    __shared__ __align__(16) int32_t s_sc1[SC1];
    __shared__ __align__(16) uint8_t s_stage[4][GEMV_STAGE_BYTES];
    __shared__ float s_scale[GEMV_MAX_M], s_inv[GEMV_MAX_M];

    const int M = a.M, N = a.N;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, g = lane >> 4;
    const int split = blockIdx.x % a.ks;
    const int u_begin = split * a.ups;
    const int nu = min(u_begin + a.ups, a.units) - u_begin;

    // ---- this wave's units: row tiles t0 .. t0+ntile-1 of split `split` ----
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int t0 = ((blockIdx.x / a.ks) * 4 + wv) * a.upw;
    const int ntile = max(0, min(a.upw, a.tiles - t0));
    const int nstages = a.full_rows ? 1 : nu / a.su;  // su divides the split
    const int nq = ntile * nstages;                    // stages this wave streams
    const int SB = a.full_rows ? (int)a.row_bytes : a.su * UB;  // bytes per row and stage
    uint8_t* stg = s_stage[wave];
    uint4 pfA[MAXP], pfB[MAXP];

    // ---- x of this K split, loaded before the weight stream is queued ----
    // (loads retire in order: issued first, they are not stuck behind the weights)
    const rsrc_t xr = make_rsrc(a.x, (uint32_t)((int64_t)M * a.K * 4));
    const uint32_t xbase = (uint32_t)u_begin * QK * 4;
    float xv[32];
    int xc = -1;   // chunk of 32 values this thread prepares (mode a, Q8_0 mode b)
    float4 xq[8];  // Q8K: this lane's 4 values of up to 8 blocks of 256
    if (MODE == MODE_A || FMT == FMT_Q8_0) {
        const int n32 = nu * (QK / 32);
        const int cm = tid / n32, cu = tid - cm * n32;
        xc = tid < M * n32 ? tid : -1;
        const uint32_t off = xc >= 0 ? xbase + (uint32_t)(cm * a.K + 32 * cu) * 4 : 0x7ffffff0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 t = load_x16(xr, off + 16 * i);
            xv[4 * i] = t.x; xv[4 * i + 1] = t.y; xv[4 * i + 2] = t.z; xv[4 * i + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int b = wave + 4 * i;
            const int cm = b / nu, cu = b - cm * nu;
            const uint32_t off = b < M * nu ? xbase + (uint32_t)(cm * a.K + 256 * cu + 4 * lane) * 4 : 0x7ffffff0u;
            xq[i] = load_x16(xr, off);
        }
    }

    // ---- the weight stream: per-lane piece offsets, the same for every stage ----
    uint32_t voff[MAXP];
    {
        const int PR = SB >> 4;
        const uint32_t mg = (65536u + PR - 1) / PR;
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int p = lane + 64 * i;
            const int r = a.full_rows ? 0 : (int)(((uint32_t)p * mg) >> 16);
            const uint32_t off = a.full_rows ? 16u * p : (uint32_t)(r * a.row_bytes + 16 * (p - r * PR));
            voff[i] = p < SB ? off : 0x7ffffff0u;
        }
    }
    auto issue = [&](uint4 (&pf)[MAXP], int q) {  // stage q, or zeros past the last one
        const bool real = q < nq;
        const int qq = real ? q : 0;
        const int t = t0 + qq / nstages, s = qq - (qq / nstages) * nstages;
        const int n0 = 16 * t, rows = max(0, min(16, N - n0));
        const int64_t col = a.full_rows ? 0 : (int64_t)(u_begin + s * a.su) * UB;
        const uint8_t* base = a.w + (int64_t)n0 * a.row_bytes + col;
        const uint32_t nrec = real ? (uint32_t)((int64_t)rows * a.row_bytes - col) : 0u;
        const rsrc_t rs = make_rsrc(real ? base : a.w, nrec);
#pragma unroll
        for (int i = 0; i < MAXP; ++i) pf[i] = load_w16(rs, voff[i]);
    };
    issue(pfA, 0);
    issue(pfB, 1);

    // ---- the activation operand of this K split, once per workgroup ----
    // Mode (a): f16 hi/lo split of x (power-of-two scale per row and K split),
    // image rows 0..M-1 hi and M..2M-1 lo, k in the weight decoder's order.
    // Mode (b): each row quantized on its own per 32 (Q8_0) or 256 (Q8K) values,
    // int8 image rows 0..M-1 first block of a pair, M..2M-1 second block.
    if (MODE == MODE_A) {
        const int n32 = nu * (QK / 32);
        if (xc >= 0) {
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(xv[i]));
            s_sc0[xc] = am;
        }
        __syncthreads();
        if (tid < M) {
            float r = 0.0f;
            for (int c = 0; c < n32; ++c) r = fmaxf(r, s_sc0[tid * n32 + c]);
            const int e = split_exp(r);
            s_scale[tid] = ldexpf(1.0f, e);
            s_inv[tid] = ldexpf(1.0f, -e);
        }
        __syncthreads();
        if (xc >= 0) {
            const int cm = xc / n32, cu = xc - cm * n32;
            _Float16 hi[32], lo[32];
            const float sum = split_chunk(xv, s_scale[cm], hi, lo);
            half8_t* img = reinterpret_cast<half8_t*>(s_img);
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                half8_t vh, vl;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    int k;
                    if (FMT == FMT_Q8_0) k = (cu & 1) ? 8 * gg + t : q8_even_k(gg, t);
                    else k = 8 * gg + nib_perm(t);
                    vh[t] = hi[k];
                    vl[t] = lo[k];
                }
                img[(cu * 4 + gg) * 2 * M + cm] = vh;
                img[(cu * 4 + gg) * 2 * M + M + cm] = vl;
            }
            if (FMT == FMT_Q4_K) reinterpret_cast<float*>(s_sc1)[cu * 8 + cm] = sum;
        }
    } else if (FMT == FMT_Q8_0) {
        if (xc >= 0) {  // one 32-value block per thread
            const int cm = xc / nu, cu = xc - cm * nu;
            uint16_t dbits;
            float dval;
            int8_t q[32];
            q8_0_block(xv, dbits, dval, q);
            const int odd = cu & 1, row = odd ? M + cm : cm;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                int sv[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) sv[t] = q[odd ? 8 * gg + t : q8_even_k(gg, t)];
                reinterpret_cast<uint2*>(s_img)[((cu >> 1) * 4 + gg) * 2 * M + row] =
                    make_uint2(pack4(sv[0], sv[1], sv[2], sv[3]), pack4(sv[4], sv[5], sv[6], sv[7]));
            }
            s_sc0[cu * 8 + cm] = dval;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // one 256-value block per wave and step
            const int b = wave + 4 * i;
            if (b < M * nu) {
                const int cm = b / nu, cu = b - cm * nu;
                const float xs[4] = {xq[i].x, xq[i].y, xq[i].z, xq[i].w};
                float d;
                int q[4], s16;
                q8k_wave(xs, lane, d, q, s16);
                const int e = 4 * lane, c = e >> 6, w = e & 63, hf = w >> 5, gg = (w & 31) >> 3, tt = w & 7;
                const int row = hf ? M + cm : cm;
                *reinterpret_cast<uint32_t*>(s_img + ((((cu * 4 + c) * 4 + gg) * 2 * M + row) * 8 + tt)) =
                    pack4(q[0], q[1], q[2], q[3]);
                if (lane == 0) s_sc0[cu * 8 + cm] = d;
                const int pair = s16 + __shfl_down(s16, 4);
                if ((lane & 7) == 0) s_sc1[(cu * 8 + (lane >> 3)) * 8 + cm] = pair;
            }
        }
    }
    __syncthreads();

    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    // A-operand row of this lane: rows 0..7 -> image row m, rows 8..15 -> image row M+m
    const int arow = j < 8 ? j : M + (j - 8);
    const bool alive = (j & 7) < M;

    auto store = [&](uint4 (&pf)[MAXP]) {
        WAVE_SYNC();
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int p = lane + 64 * i;
            if (p < SB) reinterpret_cast<uint4*>(stg)[p] = pf[i];
        }
        WAVE_SYNC();
    };

    // one stage of one unit: rows n0..n0+15, stage s of the split
    auto compute = [&](int n0, int s) {
        const uint8_t* rowp = stg + j * SB;
        const int lu0 = a.full_rows ? 0 : s * a.su;  // first unit of the stage, relative to u_begin
        if (FMT == FMT_Q8_0) {
            const int npairs = SB / 68;
#pragma unroll 4
            for (int pp = 0; pp < npairs; ++pp) {
                const uint32_t* L = reinterpret_cast<const uint32_t*>(rowp + 68 * pp);
                const uint32_t dw0 = L[0], dw8 = L[8];
                const uint32_t le = L[1 + 2 * g], he_raw = L[2 + 2 * g];
                const uint32_t lo = L[9 + 2 * g], ho = L[10 + 2 * g];
                const uint32_t he = g == 3 ? __builtin_amdgcn_alignbyte(he_raw, dw0, 2) : he_raw;
                const int lb = lu0 + 2 * pp;  // even block, relative to u_begin
                if (MODE == MODE_A) {
                    uint32_t t0_, t1_, t2_, t3_;
                    i8x4_to_f16(le, t0_, t1_);
                    i8x4_to_f16(he, t2_, t3_);
                    const half8_t be = __builtin_bit_cast(half8_t, u32x4_t{t0_, t1_, t2_, t3_});
                    i8x4_to_f16(lo, t0_, t1_);
                    i8x4_to_f16(ho, t2_, t3_);
                    const half8_t bo = __builtin_bit_cast(half8_t, u32x4_t{t0_, t1_, t2_, t3_});
                    const half8_t* img = reinterpret_cast<const half8_t*>(s_img);
                    half8_t ae = {}, ao = {};
                    if (alive) {
                        ae = img[(lb * 4 + g) * 2 * M + arow];
                        ao = img[((lb + 1) * 4 + g) * 2 * M + arow];
                    }
                    const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
                    const f32x4_t ce = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, be, z, 0, 0, 0);
                    const f32x4_t co = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, bo, z, 0, 0, 0);
                    const float de = f16lo(dw0), dd = f16hi(dw8);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] += de * ce[r] + dd * co[r];
                } else {
                    const i32x4_t bq = {(int)le, (int)he, (int)lo, (int)ho};
                    uint2 av = make_uint2(0, 0);
                    if (alive) av = reinterpret_cast<const uint2*>(s_img)[((lb >> 1) * 4 + g) * 2 * M + arow];
                    const i32x4_t aq = j < 8 ? i32x4_t{(int)av.x, (int)av.y, 0, 0} : i32x4_t{0, 0, (int)av.x, (int)av.y};
                    const i32x4_t z = {0, 0, 0, 0};
                    const i32x4_t c = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq, bq, z, 0, 0, 0);
                    const int blk = lb + (g >> 1);
                    const float sw = g < 2 ? f16lo(dw0) : f16hi(dw8);
                    const f32x4_t dx = *reinterpret_cast<const f32x4_t*>(&s_sc0[blk * 8 + 4 * (g & 1)]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] += (sw * dx[r]) * (float)c[r];
                    if (EMIT) {
                        const int n = n0 + j;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int m = 4 * (g & 1) + r;
                            if (m < M && n < N) a.sums[((int64_t)m * N + n) * a.units + u_begin + blk] = c[r];
                        }
                    }
                }
            }
        } else {  // Q4_K super-blocks
            const int nsb = SB / 144;
#pragma unroll 2
            for (int uu = 0; uu < nsb; ++uu) {
                const uint8_t* sbp = rowp + 144 * uu;
                const u32x4_t hdr = *reinterpret_cast<const u32x4_t*>(sbp);
                const float d = f16lo(hdr[0]), dmin = f16hi(hdr[0]);
                int sc[8], mn[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) q4k_scale_min(hdr[1], hdr[2], hdr[3], q, sc[q], mn[q]);
                const int lu = lu0 + uu;  // super-block relative to u_begin
                if (MODE == MODE_A) {
                    const half8_t* img = reinterpret_cast<const half8_t*>(s_img);
                    const float* xs = reinterpret_cast<const float*>(s_sc1);
                    f32x4_t mins = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint2 qv = *reinterpret_cast<const uint2*>(sbp + 16 + 32 * c + 8 * g);
                        const half8_t b0 = nib8_to_f16(qv.x, qv.y, 0);
                        const half8_t b1 = nib8_to_f16(qv.x, qv.y, 4);
                        const int sub0 = lu * 8 + 2 * c;
                        half8_t a0 = {}, a1 = {};
                        if (alive) {
                            a0 = img[(sub0 * 4 + g) * 2 * M + arow];
                            a1 = img[((sub0 + 1) * 4 + g) * 2 * M + arow];
                        }
                        const f32x4_t z = {0.0f, 0.0f, 0.0f, 0.0f};
                        const f32x4_t c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, z, 0, 0, 0);
                        const f32x4_t c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, z, 0, 0, 0);
                        const float s0 = d * (float)sc[2 * c], s1 = d * (float)sc[2 * c + 1];
                        const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(&xs[sub0 * 8 + 4 * (g & 1)]);
                        const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(&xs[(sub0 + 1) * 8 + 4 * (g & 1)]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            acc[r] += s0 * c0[r] + s1 * c1[r];
                            mins[r] += (float)mn[2 * c] * x0[r] + (float)mn[2 * c + 1] * x1[r];
                        }
                    }
                    const float dm = g < 2 ? dmin : 0.0f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] -= dm * mins[r];
                } else {
                    i32x4_t sumi = {0, 0, 0, 0};
                    const int half = g >> 1;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint2 qv = *reinterpret_cast<const uint2*>(sbp + 16 + 32 * c + 8 * g);
                        const i32x4_t bq = {(int)(qv.x & 0x0f0f0f0fu), (int)(qv.y & 0x0f0f0f0fu),
                                            (int)((qv.x >> 4) & 0x0f0f0f0fu), (int)((qv.y >> 4) & 0x0f0f0f0fu)};
                        uint2 av = make_uint2(0, 0);
                        if (alive) av = reinterpret_cast<const uint2*>(s_img)[((lu * 4 + c) * 4 + g) * 2 * M + arow];
                        const i32x4_t aq = j < 8 ? i32x4_t{(int)av.x, (int)av.y, 0, 0} : i32x4_t{0, 0, (int)av.x, (int)av.y};
                        const i32x4_t z = {0, 0, 0, 0};
                        const i32x4_t cc = __builtin_amdgcn_mfma_i32_16x16x64_i8(aq, bq, z, 0, 0, 0);
                        const int scj = sc[2 * c + half];
#pragma unroll
                        for (int r = 0; r < 4; ++r) sumi[r] += scj * cc[r];
                        if (EMIT) {
                            const int n = n0 + j;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int m = 4 * (g & 1) + r;
                                if (m < M && n < N)
                                    a.sums[(((int64_t)m * N + n) * a.units + u_begin + lu) * 10 + 2 * c + half] = cc[r];
                            }
                        }
                    }
                    i32x4_t summ = {0, 0, 0, 0};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int jq = 2 * c + half;
                        const i32x4_t bsv = *reinterpret_cast<const i32x4_t*>(&s_sc1[(lu * 8 + jq) * 8 + 4 * (g & 1)]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) summ[r] += mn[jq] * bsv[r];
                    }
                    const f32x4_t dq = *reinterpret_cast<const f32x4_t*>(&s_sc0[lu * 8 + 4 * (g & 1)]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] += dq[r] * (d * (float)sumi[r] - dmin * (float)summ[r]);
                    if (EMIT) {
                        i32x4_t ti, tm;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            ti[r] = sumi[r] + __shfl_xor(sumi[r], 32);
                            tm[r] = summ[r] + __shfl_xor(summ[r], 32);
                        }
                        const int n = n0 + j;
                        if (g < 2) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int m = 4 * g + r;
                                if (m < M && n < N) {
                                    int32_t* o = a.sums + (((int64_t)m * N + n) * a.units + u_begin + lu) * 10;
                                    o[8] = ti[r];
                                    o[9] = tm[r];
                                }
                            }
                        }
                    }
                }
            }
        }
        if (s == nstages - 1 && !EMIT) {  // unit done: combine the two halves, write, reset
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += __shfl_xor(acc[r], 32);
            const int n = n0 + j;
            if (g < 2 && n < N) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 4 * g + r;
                    if (m < M) {
                        float v = acc[r];
                        if (MODE == MODE_A) v *= s_inv[m];
                        if (a.ks == 1) a.y[(int64_t)m * N + n] = v;
                        else a.part[((int64_t)split * GEMV_MAX_M + m) * N + n] = v;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = 0.0f;
        }
    };

    // two stages in flight: store stage q, queue stage q+2, compute stage q
    for (int q = 0; q < nq; q += 2) {
        store(pfA);
        issue(pfA, q + 2);
        compute(16 * (t0 + q / nstages), q - (q / nstages) * nstages);
        store(pfB);
        issue(pfB, q + 3);
        if (q + 1 < nq) compute(16 * (t0 + (q + 1) / nstages), (q + 1) - ((q + 1) / nstages) * nstages);
    }
}

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

// ------------------------------------------------------------- geometry ----

static int unit_values(int fmt) { return fmt == FMT_Q8_0 ? 32 : 256; }

bool gemv_supported(int fmt, int64_t K)
{
    if (fmt == FMT_Q4_K) return K % 256 == 0;
    if (K % 32) return false;
    const int64_t units = K / 32;
    const bool whole_rows = 16 * units * 34 <= GEMV_STAGE_BYTES && units % 2 == 0;
    return whole_rows || units % 8 == 0;
}

// Most K splits a run may use (sizes the split-K workspace): at least enough
// to keep every split within the LDS activation operand (1024 values for
// f32 activations at M = 8), at most one split per aligned unit group.
int gemv_max_splits(int fmt, int64_t K)
{
    const int64_t units = K / unit_values(fmt);
    if (fmt == FMT_Q8_0 && units % 8) return 1;
    const int64_t align = fmt == FMT_Q8_0 ? 8 : 1;
    const int64_t cap = std::max<int64_t>(GEMV_MAX_SPLITS, (K + 1023) / 1024);
    return (int)std::max<int64_t>(1, std::min<int64_t>(cap, units / align));
}

// K splits, units per wave and grid for one run: every workgroup resident at
// once (max_wgs = CUs x workgroups per CU), about one unit per wave when the
// matrix is large, and each K split at most min(4096, 8192/M) values, so one
// thread (one wave for Q8K) prepares at most one chunk of the activation
// operand and the operand fits in LDS.  The stage size divides every split.
GemvGeom gemv_geom(int fmt, int mode, int64_t N, int64_t K, int M, int max_wgs)
{
    (void)mode;
    GemvGeom g{};
    const int qk = unit_values(fmt);
    g.unit_bytes = fmt == FMT_Q8_0 ? 34 : 144;
    g.units = (int)(K / qk);
    g.row_bytes = (int64_t)g.units * g.unit_bytes;
    g.tiles = (int)((N + 15) / 16);
    const int range = std::min(MAX_RANGE, 8192 / M);
    const int max_units = std::max(1, range / qk);
    int ks = std::max((g.units + max_units - 1) / max_units, (4 * max_wgs) / g.tiles);
    ks = std::max(1, std::min(ks, gemv_max_splits(fmt, K)));
    if (fmt == FMT_Q8_0 && g.units % 8) {
        g.ks = 1;
        g.ups = g.units;
        g.full_rows = 1;
        g.su = g.units;
    } else {
        int ups = (g.units + ks - 1) / ks;
        if (fmt == FMT_Q8_0) ups = (ups + 7) / 8 * 8;
        while (ups > max_units && ups > (fmt == FMT_Q8_0 ? 8 : 1)) ups -= fmt == FMT_Q8_0 ? 8 : 1;
        g.ups = ups;
        g.ks = (g.units + ups - 1) / ups;
        const int last = g.units - (g.ks - 1) * ups;
        g.full_rows = fmt == FMT_Q8_0 && g.ks == 1 && 16 * g.row_bytes <= GEMV_STAGE_BYTES;
        if (g.full_rows) {
            g.su = g.units;
        } else {
            const int cand8[2] = {16, 8}, cand4[4] = {4, 3, 2, 1};
            const int* cand = fmt == FMT_Q8_0 ? cand8 : cand4;
            const int nc = fmt == FMT_Q8_0 ? 2 : 4;
            g.su = cand[nc - 1];
            for (int i = 0; i < nc; ++i)
                if (ups % cand[i] == 0 && last % cand[i] == 0) {
                    g.su = cand[i];
                    break;
                }
        }
    }
    const int64_t units_total = (int64_t)g.tiles * g.ks;
    g.upw = (int)std::max<int64_t>(1, (units_total + 4 * (int64_t)max_wgs - 1) / (4 * (int64_t)max_wgs));
    const int wgs_per_split = (int)((g.tiles + 4 * g.upw - 1) / (4 * g.upw));
    g.grid = wgs_per_split * g.ks;
    return g;
}

// ------------------------------------------------------------ launchers ----

template <int FMT, int MODE, bool EMIT>
static int resident_wgs()
{
    static int cached[64] = {0};
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemv_kernel<FMT, MODE, EMIT>, 256, 0) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
        cached[dev] = per_cu * cus;
    }
    return cached[dev];
}

int gemv_resident_wgs(int fmt, int mode, bool emit)
{
    if (fmt == FMT_Q8_0) {
        if (mode == MODE_A) return resident_wgs<FMT_Q8_0, MODE_A, false>();
        return emit ? resident_wgs<FMT_Q8_0, MODE_B, true>() : resident_wgs<FMT_Q8_0, MODE_B, false>();
    }
    if (mode == MODE_A) return resident_wgs<FMT_Q4_K, MODE_A, false>();
    return emit ? resident_wgs<FMT_Q4_K, MODE_B, true>() : resident_wgs<FMT_Q4_K, MODE_B, false>();
}

template <int FMT, int MODE, bool EMIT>
static void launch_one(const GemvArgs& a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((gemv_kernel<FMT, MODE, EMIT>), dim3((unsigned)grid), dim3(256), 0, s, a);
}

hipError_t launch_gemv(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, int M,
                       const GemvBufs& b, float* y, int32_t* sums, hipStream_t s)
{
    const bool emit = sums != nullptr;
    const GemvGeom g = gemv_geom(fmt, mode, N, K, M, gemv_resident_wgs(fmt, mode, emit));
    GemvArgs a{};
    a.w = (const uint8_t*)w;
    a.row_bytes = g.row_bytes;
    a.N = (int)N;
    a.K = (int)K;
    a.M = M;
    a.units = g.units;
    a.ups = g.ups;
    a.ks = g.ks;
    a.full_rows = g.full_rows;
    a.su = g.su;
    a.upw = g.upw;
    a.tiles = g.tiles;
    a.x = x;
    a.part = b.part;
    a.y = y;
    a.sums = sums;
    if (fmt == FMT_Q8_0) {
        if (mode == MODE_A) launch_one<FMT_Q8_0, MODE_A, false>(a, g.grid, s);
        else if (emit) launch_one<FMT_Q8_0, MODE_B, true>(a, g.grid, s);
        else launch_one<FMT_Q8_0, MODE_B, false>(a, g.grid, s);
    } else {
        if (mode == MODE_A) launch_one<FMT_Q4_K, MODE_A, false>(a, g.grid, s);
        else if (emit) launch_one<FMT_Q4_K, MODE_B, true>(a, g.grid, s);
        else launch_one<FMT_Q4_K, MODE_B, false>(a, g.grid, s);
    }
    if (!emit && g.ks > 1) {
        const int64_t total = (int64_t)M * N;
        hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, b.part, g.ks,
                           M, (int)N, y);
    }
    return hipGetLastError();
}

}  // namespace qmm
