// qmm_gemv.hip -- decode kernel (M <= 8) for y = x . W^T on GGUF blocks.
//
// The weight stream is the cost (the pages' CPU decode step is dominated by
// it: page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 修法, 7 ms
// Q8_0 vs 15 ms dequantized f32).  Layout of the work:
//   * a 256-thread workgroup owns 64 weight rows (four waves x 16 rows) and
//     one K range of at most 1024 values (grid.y splits K);
//   * each wave streams its 16 rows with coalesced 16-byte loads into a
//     private LDS stage (prefetched one stage ahead in registers), then every
//     lane reads the weight bytes of one row in the matrix-core operand layout;
//   * each workgroup prepares the activation operand of its K range in LDS
//     (mode a: f16 hi/lo split; mode b: Q8_0 / Q8K quantization of each row);
//   * mode (a): v_mfma_f32_16x16x32_f16 with the weights as exact f16 integers
//     (q for Q8_0, the 4-bit q for Q4_K) against activation rows 0..7 = f16 hi
//     part and rows 8..15 = f16 lo part, block scales applied per block in f32;
//   * mode (b): v_mfma_i32_16x16x64_i8 over two 32-value blocks at once (A rows
//     0..7 carry the first block, 8..15 the second, zero elsewhere), giving the
//     int32 block sums; scaled in f32 (Q8_0: dw*dx*S; Q4_K: sub-block scales in
//     int32, then dx*(d*sumi - dmin*summins));
//   * split-K partials go to a workspace and a small second kernel sums them
//     in a fixed order (deterministic; no cross-workgroup fences).
#include "qmm_act.h"

namespace qmm {

constexpr int MAXP = 10;  // 16-byte staging pieces per lane and stage

struct GemvArgs {
    const uint8_t* w;
    int64_t row_bytes;
    int N, K, M;
    int units, ups, full_rows, su, ks;
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

// Copy up to 16 bytes that end the weight buffer (the tail of a whole-row
// stage whose byte count is not a multiple of 16).
QMM_DEV uint4 load_tail(const uint8_t* p, int nbytes)
{
    uint32_t v[4] = {0, 0, 0, 0};
    for (int i = 0; i < nbytes; ++i) v[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int FMT, int MODE, bool EMIT>
__global__ __launch_bounds__(256, 2) void gemv_kernel(GemvArgs a)
{
    constexpr int UB = FMT == FMT_Q8_0 ? 34 : 144;
    // activation image bytes per weight unit (32-block or 256-super-block) and row M
    constexpr int IMG_BYTES = MODE == MODE_A ? 32768 : 8192;
    __shared__ __align__(16) uint8_t s_img[IMG_BYTES];
    __shared__ __align__(16) float s_sc0[256];
    __shared__ __align__(16) int32_t s_sc1[256];
    __shared__ __align__(16) uint8_t s_stage[4][GEMV_STAGE_BYTES];
    __shared__ float s_scale[GEMV_MAX_M], s_inv[GEMV_MAX_M];

    const int M = a.M, N = a.N;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, g = lane >> 4;
    const int split = blockIdx.y;
    const int u_begin = split * a.ups;
    const int u_end = min(u_begin + a.ups, a.units);
    const int nu = u_end - u_begin;

    // ---- build the activation operand of this K range in LDS ----
    // Mode (a): f16 hi/lo split of x (power-of-two scale per row and K range),
    // rows 0..M-1 hi and M..2M-1 lo, k in the weight decoder's order.
    // Mode (b): each row quantized on its own per 32 (Q8_0) or 256 (Q8K) values,
    // int8 image rows 0..M-1 first block of a pair, M..2M-1 second block.
    {
        constexpr int QK = FMT == FMT_Q8_0 ? 32 : 256;
        const float* xk = a.x + (int64_t)u_begin * QK;
        if (MODE == MODE_A) {
            const int n32 = nu * (QK / 32);
            const bool have = tid < M * n32;  // one 32-value chunk per thread (<= 256)
            const int cm = have ? tid / n32 : 0, cu = have ? tid - cm * n32 : 0;
            float v[32];
            if (have) {
                load32(xk + (int64_t)cm * a.K + 32 * cu, v);
                float am = 0.0f;
#pragma unroll
                for (int c = 0; c < 32; ++c) am = fmaxf(am, fabsf(v[c]));
                s_sc0[tid] = am;
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
            if (have) {
                _Float16 hi[32], lo[32];
                const float sum = split_chunk(v, s_scale[cm], hi, lo);
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
            if (tid < M * nu) {  // one 32-value block per thread
                const int cm = tid / nu, cu = tid - cm * nu;
                float v[32];
                load32(xk + (int64_t)cm * a.K + 32 * cu, v);
                uint16_t dbits;
                float dval;
                int8_t q[32];
                q8_0_block(v, dbits, dval, q);
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
            for (int b = wave; b < M * nu; b += 4) {  // one 256-value block per wave
                const int cm = b / nu, cu = b - cm * nu;
                const float4 xv = reinterpret_cast<const float4*>(xk + (int64_t)cm * a.K + 256 * cu)[lane];
                const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
                float d;
                int q[4], s16;
                q8k_wave(xs, lane, d, q, s16);
                const int e = 4 * lane, c = e >> 6, w = e & 63, hf = w >> 5, gg = (w & 31) >> 3, t0 = w & 7;
                const int row = hf ? M + cm : cm;
                *reinterpret_cast<uint32_t*>(s_img + ((((cu * 4 + c) * 4 + gg) * 2 * M + row) * 8 + t0)) =
                    pack4(q[0], q[1], q[2], q[3]);
                if (lane == 0) s_sc0[cu * 8 + cm] = d;
                const int pair = s16 + __shfl_down(s16, 4);
                if ((lane & 7) == 0) s_sc1[(cu * 8 + (lane >> 3)) * 8 + cm] = pair;
            }
        }
    }
    __syncthreads();

    const int n0 = blockIdx.x * GEMV_ROWS + wave * 16;
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    // A-operand row of this lane: rows 0..7 -> image row m, rows 8..15 -> image row M+m
    const int arow = j < 8 ? j : M + (j - 8);
    const bool alive = (j & 7) < M;

    if (n0 < N) {
        uint8_t* stg = s_stage[wave];
        const uint8_t* wt = a.w + (int64_t)n0 * a.row_bytes;
        const int nstages = a.full_rows ? 1 : (nu + a.su - 1) / a.su;
        const int64_t tile_valid = (int64_t)min(16, N - n0) * a.row_bytes;  // bytes of real rows
        uint4 pf[MAXP];

        // piece geometry of stage s: bytes per row SB, pieces P
        auto stage_sb = [&](int s) -> int {
            if (a.full_rows) return (int)a.row_bytes;
            return min(a.su, nu - s * a.su) * UB;
        };
        auto issue = [&](int s) {
            const int SB = stage_sb(s);
            const int P = SB;  // 16 rows * SB bytes / 16 bytes per piece
            if (a.full_rows) {
#pragma unroll
                for (int i = 0; i < MAXP; ++i) {
                    const int p = lane + 64 * i;
                    if (p < P) {
                        const int64_t off = 16 * (int64_t)p;
                        if (off + 16 <= tile_valid) pf[i] = *reinterpret_cast<const uint4*>(wt + off);
                        else if (off < tile_valid) pf[i] = load_tail(wt + off, (int)(tile_valid - off));
                    }
                }
            } else {
                const int PR = SB >> 4;
                const uint32_t mg = (65536u + PR - 1) / PR;
                const int64_t col = (int64_t)(u_begin + s * a.su) * UB;
#pragma unroll
                for (int i = 0; i < MAXP; ++i) {
                    const int p = lane + 64 * i;
                    const int r = (int)(((uint32_t)p * mg) >> 16);
                    if (p < P && n0 + r < N) {
                        const int jj = p - r * PR;
                        pf[i] = *reinterpret_cast<const uint4*>(wt + r * a.row_bytes + col + 16 * jj);
                    }
                }
            }
        };

        issue(0);
        for (int s = 0; s < nstages; ++s) {
            const int SB = stage_sb(s);
            WAVE_SYNC();
#pragma unroll
            for (int i = 0; i < MAXP; ++i) {
                const int p = lane + 64 * i;
                if (p < SB) reinterpret_cast<uint4*>(stg)[p] = pf[i];
            }
            WAVE_SYNC();
            if (s + 1 < nstages) issue(s + 1);
            const uint8_t* rowp = stg + j * SB;
            const int lu0 = a.full_rows ? 0 : s * a.su;  // first unit of the stage, relative to u_begin

            if (FMT == FMT_Q8_0) {
                const int npairs = SB / 68;
                for (int pp = 0; pp < npairs; ++pp) {
                    const uint32_t* L = reinterpret_cast<const uint32_t*>(rowp + 68 * pp);
                    const uint32_t dw0 = L[0], dw8 = L[8];
                    const uint32_t le = L[1 + 2 * g], he_raw = L[2 + 2 * g];
                    const uint32_t lo = L[9 + 2 * g], ho = L[10 + 2 * g];
                    const uint32_t he = g == 3 ? __builtin_amdgcn_alignbyte(he_raw, dw0, 2) : he_raw;
                    const int lb = lu0 + 2 * pp;  // even block, relative to u_begin
                    if (MODE == MODE_A) {
                        half8_t be, bo;
                        uint32_t t0, t1, t2, t3;
                        i8x4_to_f16(le, t0, t1);
                        i8x4_to_f16(he, t2, t3);
                        be = __builtin_bit_cast(half8_t, u32x4_t{t0, t1, t2, t3});
                        i8x4_to_f16(lo, t0, t1);
                        i8x4_to_f16(ho, t2, t3);
                        bo = __builtin_bit_cast(half8_t, u32x4_t{t0, t1, t2, t3});
                        const half8_t* img = reinterpret_cast<const half8_t*>(s_img);
                        half8_t ae = {}, ao = {};
                        if (alive) {
                            ae = img[((lb)*4 + g) * 2 * M + arow];
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
                                if (m < M && n < N)
                                    a.sums[((int64_t)m * N + n) * a.units + u_begin + blk] = c[r];
                            }
                        }
                    }
                }
            } else {  // Q4_K super-blocks
                const int nsb = SB / 144;
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
        }
    }

    if (EMIT) return;

    // ---- combine hi/lo (mode a) or even/odd-block (mode b) halves ----
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
}

// Split-K: y[m][n] = sum over K ranges of the partials, in range order.
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

GemvGeom gemv_geom(int fmt, int64_t K)
{
    GemvGeom g{};
    g.unit_bytes = fmt == FMT_Q8_0 ? 34 : 144;
    g.units = (int)(fmt == FMT_Q8_0 ? K / 32 : K / 256);
    g.row_bytes = (int64_t)g.units * g.unit_bytes;
    g.ks = (int)((K + GEMV_KRANGE - 1) / GEMV_KRANGE);
    if (fmt == FMT_Q8_0) {
        if (g.ks == 1 && 16 * g.row_bytes <= GEMV_STAGE_BYTES && g.units % 2 == 0) {
            g.full_rows = 1;
            g.ups = g.units;
            g.su = g.units;
        } else {
            g.full_rows = 0;
            g.ups = (g.units + g.ks - 1) / g.ks;
            g.ups = (g.ups + 7) / 8 * 8;
            g.ks = (g.units + g.ups - 1) / g.ups;
            g.su = 16;
        }
    } else {
        g.full_rows = 0;
        g.ups = (g.units + g.ks - 1) / g.ks;
        g.ks = (g.units + g.ups - 1) / g.ups;
        g.su = 4;
    }
    return g;
}

bool gemv_supported(int fmt, int64_t K)
{
    if (fmt == FMT_Q4_K) return K % 256 == 0;
    if (K % 32) return false;
    const GemvGeom g = gemv_geom(fmt, K);
    return g.full_rows || g.units % 8 == 0;
}

template <int FMT, int MODE, bool EMIT>
static void launch_one(const GemvArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.N + GEMV_ROWS - 1) / GEMV_ROWS), (unsigned)a.ks);
    hipLaunchKernelGGL((gemv_kernel<FMT, MODE, EMIT>), grid, dim3(256), 0, s, a);
}

hipError_t launch_gemv(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, int M,
                       const GemvGeom& g, const GemvBufs& b, float* y, int32_t* sums, hipStream_t s)
{
    GemvArgs a{};
    a.w = (const uint8_t*)w;
    a.row_bytes = g.row_bytes;
    a.N = (int)N;
    a.K = (int)K;
    a.M = M;
    a.units = g.units;
    a.ups = g.ups;
    a.full_rows = g.full_rows;
    a.su = g.su;
    a.ks = g.ks;
    a.x = x;
    a.part = b.part;
    a.y = y;
    a.sums = sums;
    const bool emit = sums != nullptr;
    if (fmt == FMT_Q8_0) {
        if (mode == MODE_A) launch_one<FMT_Q8_0, MODE_A, false>(a, s);
        else if (emit) launch_one<FMT_Q8_0, MODE_B, true>(a, s);
        else launch_one<FMT_Q8_0, MODE_B, false>(a, s);
    } else {
        if (mode == MODE_A) launch_one<FMT_Q4_K, MODE_A, false>(a, s);
        else if (emit) launch_one<FMT_Q4_K, MODE_B, true>(a, s);
        else launch_one<FMT_Q4_K, MODE_B, false>(a, s);
    }
    if (!emit && g.ks > 1) {
        const int64_t total = (int64_t)M * N;
        hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, b.part, g.ks,
                           M, (int)N, y);
    }
    return hipGetLastError();
}

}  // namespace qmm
