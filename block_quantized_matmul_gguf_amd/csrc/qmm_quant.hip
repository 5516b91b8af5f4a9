// qmm_quant.hip -- the standalone activation quantizer (canonical Q8_0 / Q8K
// blocks), the prefill kernels' activation preparation, and the weight
// quantizers.  The block arithmetic lives in qmm_act.h and is shared with the
// decode kernel's prologue.  Every activation row is quantized on its own
// (page "自己量化", section 动脑筋答案).
#include "qmm_act.h"

namespace qmm {

enum { LAY_AOS = 0, LAY_I8 = 3, LAY_F16 = 4 };

// Lanes sub = 0..7 of a group of eight hold values 4*sub .. 4*sub+3 of a
// 34-byte block; lane 0 also holds d.
QMM_DEV void store_q8_0_part(uint8_t* o, int sub, uint16_t dbits, const int q[4])
{
    uint16_t* h = reinterpret_cast<uint16_t*>(o);  // blocks are 2-byte aligned
    if (sub == 0) h[0] = dbits;
    h[1 + 2 * sub] = (uint16_t)((uint8_t)q[0] | ((uint16_t)(uint8_t)q[1] << 8));
    h[2 + 2 * sub] = (uint16_t)((uint8_t)q[2] | ((uint16_t)(uint8_t)q[3] << 8));
}

// Eight lanes per 32-value block, four values per lane, so that a wave reads
// (and writes) eight consecutive blocks of a row contiguously.  The block's
// max|x| is reduced over its eight lanes (a maximum: the same in any order)
// and the scale and values come from q8_0_scale / q8_0_q, as in every Q8_0
// quantizer.  LAY_AOS: canonical 34-byte blocks.  LAY_I8: the values as int8
// [M][K] plus f32 scales block-major [K/32][M] (and, for a traced run, the
// canonical blocks in `act` as well).
template <int LAY>
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const float* __restrict__ x, int M, int K,
                                                            uint8_t* __restrict__ out, float* __restrict__ sc,
                                                            uint8_t* __restrict__ act)
{
    const int nb = K / 32;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = t >> 3;
    const int sub = (int)(t & 7);
    if (blk >= (int64_t)M * nb) return;  // a block's eight lanes leave together
    const int m = (int)(blk / nb), b = (int)(blk % nb);
    const float4 v = *reinterpret_cast<const float4*>(x + (int64_t)m * K + 32 * b + 4 * sub);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    float id, dval;
    uint16_t dbits;
    q8_0_scale(amax, id, dbits, dval);
    const int q[4] = {q8_0_q(v.x, id), q8_0_q(v.y, id), q8_0_q(v.z, id), q8_0_q(v.w, id)};
    if (LAY == LAY_AOS) {
        store_q8_0_part(out + blk * 34, sub, dbits, q);
    } else if (LAY == LAY_I8) {
        if (act) store_q8_0_part(act + blk * 34, sub, dbits, q);
        *reinterpret_cast<uint32_t*>(out + (int64_t)m * K + 32 * b + 4 * sub) = pack4(q[0], q[1], q[2], q[3]);
        if (sub == 0) sc[(int64_t)b * M + m] = dval;
    }
}

// One wave per 256-value block, four blocks per workgroup.  LAY_AOS: canonical
// 292-byte blocks.  LAY_F16 (the f16 prefill kernel's operand): values as
// exact f16 [M][K], f32 scales block-major [K/256][M].  LAY_I8: values as int8
// [M][K], f32 scales block-major [K/256][M], and per block the eight sums of
// 32 consecutive values as f16 [K/256][M][16]: first each sum rounded down to
// a multiple of 64, then the remainders (0..63), all exact.
template <int LAY>
__global__ __launch_bounds__(256) void quantize_q8k_kernel(const float* __restrict__ x, int M, int K,
                                                           uint8_t* __restrict__ out, float* __restrict__ sc,
                                                           void* __restrict__ bs, uint8_t* __restrict__ act)
{
    const int nsb = K / 256;
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= (int64_t)M * nsb) return;  // the whole wave leaves together
    const int m = (int)(blk / nsb), sb = (int)(blk % nsb);
    const float4 xv = reinterpret_cast<const float4*>(x + (int64_t)m * K + 256 * sb)[lane];
    const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
    float d;
    int q[4], s16;
    q8k_wave(xs, lane, d, q, s16);
    if (LAY == LAY_AOS) {
        store_q8k_lane(out + blk * 292, lane, d, q, s16);
    } else if (LAY == LAY_F16) {
        if (act) store_q8k_lane(act + blk * 292, lane, d, q, s16);
        _Float16* o = reinterpret_cast<_Float16*>(out) + (int64_t)m * K + 256 * sb + 4 * lane;
        half2_t h0 = {(_Float16)(float)q[0], (_Float16)(float)q[1]}, h1 = {(_Float16)(float)q[2], (_Float16)(float)q[3]};
        *reinterpret_cast<u32x2_t*>(o) = u32x2_t{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
        if (lane == 0) sc[(int64_t)sb * M + m] = d;
    } else if (LAY == LAY_I8) {
        if (act) store_q8k_lane(act + blk * 292, lane, d, q, s16);
        const int pair = s16 + __shfl_down(s16, 4);  // lane 8j: bsums[2j] + bsums[2j+1]
        *reinterpret_cast<uint32_t*>(out + (int64_t)m * K + 256 * sb + 4 * lane) = pack4(q[0], q[1], q[2], q[3]);
        if (lane == 0) sc[(int64_t)sb * M + m] = d;
        if ((lane & 7) == 0) {
            _Float16* o = reinterpret_cast<_Float16*>(bs) + ((int64_t)sb * M + m) * 16 + (lane >> 3);
            const int hi = (pair >> 6) * 64;
            o[0] = (_Float16)(float)hi;
            o[8] = (_Float16)(float)(pair - hi);
        }
    }
}

// Mode (a) prefill preparation, one workgroup per row.  The row x is scaled
// by the power of two s that puts its largest magnitude in [2^14, 2^15) and
// split into f16 hi + lo; rs = 1/s.  Q4_K also gets the sums of x*s over every
// 32 values, divided by 32 so that they stay below 2^15, split the same way
// and laid out [M][K/256][8 hi, 8 lo].  Thread t takes the row's float4 chunks
// t, t + 256, ..., so every wave load reads (and every store writes) one
// contiguous run; a 32-value sum is formed by the eight threads holding it.
template <int FMT>
__global__ __launch_bounds__(256) void gemm_prep_kernel(const float* __restrict__ x, int M, int K,
                                                        _Float16* __restrict__ hi, _Float16* __restrict__ lo,
                                                        float* __restrict__ rs, _Float16* __restrict__ xs)
{
#pragma clang fp contract(off)
    __shared__ float red[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float4* v = reinterpret_cast<const float4*>(x + (int64_t)m * K);
    const int nc = K / 4;  // a multiple of 8: whole 32-value groups

    float am = 0.0f;
#pragma unroll 4
    for (int c = tid; c < nc; c += 256) {
        const float4 e = v[c];
        am = fmaxf(am, fmaxf(fmaxf(fabsf(e.x), fabsf(e.y)), fmaxf(fabsf(e.z), fabsf(e.w))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    if (lane == 0) red[wave] = am;
    __syncthreads();
    am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const int sexp = split_exp(am);
    const float s = ldexpf(1.0f, sexp);
    if (tid == 0) rs[m] = ldexpf(1.0f, -sexp);

    _Float16* oh = hi + (int64_t)m * K;
    _Float16* ol = lo + (int64_t)m * K;
    _Float16* ox = FMT == FMT_Q4_K ? xs + (int64_t)m * (K / 256) * 16 : nullptr;
    const int steps = (nc + 255) / 256;
    for (int i = 0; i < steps; ++i) {  // every thread takes each step (the sums below)
        const int c = tid + 256 * i;
        const bool ok = c < nc;  // the same for the eight threads of a 32-value group
        const float4 e = ok ? v[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float t[4];
        _Float16 h[4], l[4];
        split_one(e.x, s, h[0], l[0], t[0]);
        split_one(e.y, s, h[1], l[1], t[1]);
        split_one(e.z, s, h[2], l[2], t[2]);
        split_one(e.w, s, h[3], l[3], t[3]);
        if (ok) {
            reinterpret_cast<u32x2_t*>(oh)[c] = u32x2_t{__builtin_bit_cast(uint32_t, half2_t{h[0], h[1]}),
                                                        __builtin_bit_cast(uint32_t, half2_t{h[2], h[3]})};
            reinterpret_cast<u32x2_t*>(ol)[c] = u32x2_t{__builtin_bit_cast(uint32_t, half2_t{l[0], l[1]}),
                                                        __builtin_bit_cast(uint32_t, half2_t{l[2], l[3]})};
        }
        if constexpr (FMT == FMT_Q4_K) {
            float sum = ((t[0] + t[1]) + t[2]) + t[3];
            sum += __shfl_xor(sum, 1);
            sum += __shfl_xor(sum, 2);
            sum += __shfl_xor(sum, 4);
            if (ok && (lane & 7) == 0) {
                const int u = c >> 3;  // 32-value group of the row
                _Float16 sh, sl;
                float tt;
                split_one(sum, 0.03125f, sh, sl, tt);
                ox[16 * (u >> 3) + (u & 7)] = sh;
                ox[16 * (u >> 3) + 8 + (u & 7)] = sl;
            }
        }
    }
}

// Q4_K weights, one thread per 256-value super-block.  Per 32-value sub-block
// an affine fit lo = min(0, min x), hi = max x, scale = (hi-lo)/15, min = -lo;
// 6-bit sc_j, m_j quantize scale and min against the super-block maxima / 63
// (d = max scale/63, dmin = max min/63, stored as f16); the 4-bit values are
// re-quantized against the stored scales: q = clamp(round((x + dmin*m_j) /
// (d*sc_j)), 0, 15).  The pages name QTensor::quantize(&w, Q4K) but not its
// search (page "自己量化", section "3. 量化"); this is the plain min/max rule.
//
// SEARCH: each sub-block's scale and min come from a least-squares search
// instead.  For the sub-block's lo = min(0, min x), hi = max x, r = hi - lo,
// the codes q = clamp(round((x - lo) * c), 0, 15) are tried for the plain
// rule's c = 15 / r and for c = (140 + k) / (10 r), k = 0..20; each gets the
// least-squares line x ~ a q + b (b forced to 0, a refitted alone, when the
// fit gives b > 0: the format's offset -dmin*m is never positive; a <= 0 or
// all-equal codes skip the candidate), and the first of smallest squared error
// wins, the plain rule's (a = r/15, b = lo) competing first.  scale = a,
// min = -b; the super-block stage is the plain rule's.  Sums run in index
// order, one IEEE operation at a time, so the bytes are those of the oracle.
QMM_DEV void q4k_sub_range(const float* x, float& lo, float& hi)
{
    lo = 0.0f;
    hi = x[0];
    for (int l = 0; l < 32; ++l) {
        const float t = x[l];
        lo = t < lo ? t : lo;
        hi = t > hi ? t : hi;
    }
}

QMM_DEV void q4k_search_fit(const float* x, float& scale, float& minv)
{
#pragma clang fp contract(off)
    float lo, hi;
    q4k_sub_range(x, lo, hi);
    const float r = hi - lo;
    float best_a = r / 15.0f, best_b = lo;
    if (r == 0.0f) {
        scale = best_a;
        minv = -best_b;
        return;
    }
    float best_e = 0.0f;
    {
        const float c = 15.0f / r;
        for (int l = 0; l < 32; ++l) {
            int q = (int)roundf((x[l] - lo) * c);
            q = q < 0 ? 0 : (q > 15 ? 15 : q);
            const float t = best_a * (float)q + best_b - x[l];
            best_e = best_e + t * t;
        }
    }
    for (int k = 0; k <= 20; ++k) {
        const float c = (float)(140 + k) / (10.0f * r);
        int sq = 0, sqq = 0;
        float sx = 0.0f, sqx = 0.0f;
        for (int l = 0; l < 32; ++l) {
            int v = (int)roundf((x[l] - lo) * c);
            v = v < 0 ? 0 : (v > 15 ? 15 : v);
            sq += v;
            sqq += v * v;
            sx = sx + x[l];
            sqx = sqx + (float)v * x[l];
        }
        const int dd = 32 * sqq - sq * sq;
        if (dd == 0) continue;
        float a = (32.0f * sqx - (float)sq * sx) / (float)dd;
        float b = (sx - a * (float)sq) / 32.0f;
        if (b > 0.0f) {
            b = 0.0f;
            a = sqx / (float)sqq;
        }
        if (!(a > 0.0f)) continue;
        float e = 0.0f;
        for (int l = 0; l < 32; ++l) {
            int v = (int)roundf((x[l] - lo) * c);
            v = v < 0 ? 0 : (v > 15 ? 15 : v);
            const float t = a * (float)v + b - x[l];
            e = e + t * t;
        }
        if (e < best_e) {
            best_e = e;
            best_a = a;
            best_b = b;
        }
    }
    scale = best_a;
    minv = -best_b;
}

template <bool SEARCH>
__global__ __launch_bounds__(256) void quantize_q4_k_kernel(const float* __restrict__ w, int N, int K,
                                                            uint8_t* __restrict__ out)
{
#pragma clang fp contract(off)
    const int nsb = K / 256;
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= (int64_t)N * nsb) return;
    const float* v = w + (blk / nsb) * (int64_t)K + 256 * (blk % nsb);
    float scale[8], minv[8];
    float max_scale = 0.0f, max_min = 0.0f;
    for (int j = 0; j < 8; ++j) {
        if constexpr (SEARCH) {
            q4k_search_fit(v + 32 * j, scale[j], minv[j]);
        } else {
            float lo, hi;
            q4k_sub_range(v + 32 * j, lo, hi);
            scale[j] = (hi - lo) / 15.0f;
            minv[j] = -lo;
        }
        max_scale = scale[j] > max_scale ? scale[j] : max_scale;
        max_min = minv[j] > max_min ? minv[j] : max_min;
    }
    const float isc = max_scale > 0.0f ? 63.0f / max_scale : 0.0f;
    const float imn = max_min > 0.0f ? 63.0f / max_min : 0.0f;
    int sc[8], mn[8];
    for (int j = 0; j < 8; ++j) {
        const int a = (int)roundf(isc * scale[j]);
        const int c = (int)roundf(imn * minv[j]);
        sc[j] = a > 63 ? 63 : a;
        mn[j] = c > 63 ? 63 : c;
    }
    const uint16_t dh = f16bits(max_scale / 63.0f), mh = f16bits(max_min / 63.0f);
    const float dq = (float)__builtin_bit_cast(_Float16, dh);
    const float mq = (float)__builtin_bit_cast(_Float16, mh);
    uint32_t word[36];
    word[0] = (uint32_t)dh | ((uint32_t)mh << 16);
    for (int i = 1; i < 36; ++i) word[i] = 0;
    for (int j = 0; j < 4; ++j) {
        word[1] |= (uint32_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6)) << (8 * j);
        word[2] |= (uint32_t)((mn[j] & 63) | ((mn[j + 4] >> 4) << 6)) << (8 * j);
        word[3] |= (uint32_t)((sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)) << (8 * j);
    }
    for (int e = 0; e < 256; ++e) {
        const int j = e >> 5;
        const float d_eff = dq * (float)sc[j];
        const float m_eff = mq * (float)mn[j];
        int q = 0;
        if (d_eff != 0.0f) {
            q = (int)roundf((v[e] + m_eff) / d_eff);
            q = q < 0 ? 0 : (q > 15 ? 15 : q);
        }
        const int c = e >> 6, l = e & 63;
        const int byte = 16 + 32 * c + (l & 31);
        word[byte >> 2] |= (uint32_t)(q << (l < 32 ? 0 : 4)) << (8 * (byte & 3));
    }
    uint4* o = reinterpret_cast<uint4*>(out + blk * 144);
    for (int i = 0; i < 9; ++i) o[i] = make_uint4(word[4 * i], word[4 * i + 1], word[4 * i + 2], word[4 * i + 3]);
}

static unsigned nblocks(int64_t items, int per) { return (unsigned)((items + per - 1) / per); }

hipError_t launch_quantize_act(int act_fmt, const float* x, int64_t M, int64_t K, void* out, hipStream_t s)
{
    if (act_fmt == FMT_Q8_0) {
        hipLaunchKernelGGL(quantize_q8_0_kernel<LAY_AOS>, dim3(nblocks(M * (K / 32) * 8, 256)), dim3(256), 0, s,
                           x, (int)M, (int)K, (uint8_t*)out, (float*)nullptr, (uint8_t*)nullptr);
    } else {
        hipLaunchKernelGGL(quantize_q8k_kernel<LAY_AOS>, dim3(nblocks(M * (K / 256), 4)), dim3(256), 0, s,
                           x, (int)M, (int)K, (uint8_t*)out, (float*)nullptr, (void*)nullptr, (uint8_t*)nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_weights(int fmt, const float* w, int64_t N, int64_t K, void* out, hipStream_t s)
{
    if (fmt == FMT_Q8_0) return launch_quantize_act(FMT_Q8_0, w, N, K, out, s);
    hipLaunchKernelGGL(quantize_q4_k_kernel<false>, dim3(nblocks(N * (K / 256), 256)), dim3(256), 0, s,
                       w, (int)N, (int)K, (uint8_t*)out);
    return hipGetLastError();
}

hipError_t launch_quantize_q4_k_search(const float* w, int64_t N, int64_t K, void* out, hipStream_t s)
{
    hipLaunchKernelGGL(quantize_q4_k_kernel<true>, dim3(nblocks(N * (K / 256), 256)), dim3(256), 0, s,
                       w, (int)N, (int)K, (uint8_t*)out);
    return hipGetLastError();
}

// ---------------------------------------------------- odd block counts ----
// Rows of a 32-value format (Q8_0, Q4_0, Q5_0) with an odd number of blocks
// are run as rows one block longer: the weights copied with one all-zero block
// (d = 0) appended to every row, the activations with 32 zeros appended.  The
// extra block adds exact zeros in both modes (mode (b): an all-zero block
// quantizes to d = 0, q = 0).  One thread per 4 bytes of a padded row.

__global__ __launch_bounds__(256) void pad_rows_kernel(const uint8_t* __restrict__ src, int64_t rows, int src_bytes,
                                                       int dst_bytes, uint8_t* __restrict__ dst)
{
    const int per = dst_bytes / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= rows * per) return;
    const int64_t r = i / per;
    const int c = 4 * (int)(i - r * per);
    const uint8_t* sp = src + r * src_bytes;
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        if (c + b < src_bytes) v |= (uint32_t)sp[c + b] << (8 * b);
    *reinterpret_cast<uint32_t*>(dst + r * dst_bytes + c) = v;
}

__global__ __launch_bounds__(256) void pad_x_kernel(const float* __restrict__ x, int64_t M, int K, int Kp,
                                                    float* __restrict__ xp)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * Kp) return;
    const int64_t m = i / Kp;
    const int k = (int)(i - m * Kp);
    xp[i] = k < K ? x[m * K + k] : 0.0f;
}

// Keeps the first `keep` of every `from` items of `unit` bytes: the traced
// run's block sums and activation blocks of padded rows.  One thread per byte.
__global__ __launch_bounds__(256) void unpad_kernel(const uint8_t* __restrict__ src, int64_t groups, int from, int keep,
                                                    int unit, uint8_t* __restrict__ dst)
{
    const int per = keep * unit;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= groups * per) return;
    const int64_t g = i / per;
    dst[i] = src[g * from * unit + (i - g * per)];
}

hipError_t launch_pad(const void* w, int64_t N, int src_row_bytes, int dst_row_bytes, void* wpad, const float* x,
                      int64_t M, int64_t K, int64_t Kp, float* xpad, hipStream_t s)
{
    const int64_t wt = N * (dst_row_bytes / 4);
    hipLaunchKernelGGL(pad_rows_kernel, dim3(nblocks(wt, 256)), dim3(256), 0, s, (const uint8_t*)w, N, src_row_bytes,
                       dst_row_bytes, (uint8_t*)wpad);
    hipLaunchKernelGGL(pad_x_kernel, dim3(nblocks(M * Kp, 256)), dim3(256), 0, s, x, M, (int)K, (int)Kp, xpad);
    return hipGetLastError();
}

hipError_t launch_unpad(const void* src, int64_t groups, int from, int keep, int unit, void* dst, hipStream_t s)
{
    hipLaunchKernelGGL(unpad_kernel, dim3(nblocks(groups * keep * unit, 256)), dim3(256), 0, s,
                       (const uint8_t*)src, groups, from, keep, unit, (uint8_t*)dst);
    return hipGetLastError();
}

hipError_t launch_gemm_prep(int fmt, int mode, const float* x, int64_t M, int64_t K, const GemmBufs& b, hipStream_t s,
                            uint8_t* act)
{
    if (mode == MODE_B && fmt == FMT_Q6_K) {  // exact f16 values and block-major scales for the f16 kernel
        hipLaunchKernelGGL(quantize_q8k_kernel<LAY_F16>, dim3(nblocks(M * (K / 256), 4)), dim3(256), 0, s,
                           x, (int)M, (int)K, (uint8_t*)b.a0, b.sd, (void*)nullptr, act);
        return hipGetLastError();
    }
    if (mode == MODE_B) {  // int8 values, block scales (and Q8K sub-block sums) for the int8 kernel
        if (fmt == FMT_Q8_0)
            hipLaunchKernelGGL(quantize_q8_0_kernel<LAY_I8>, dim3(nblocks(M * (K / 32) * 8, 256)), dim3(256), 0, s,
                               x, (int)M, (int)K, (uint8_t*)b.a0, b.sd, act);
        else
            hipLaunchKernelGGL(quantize_q8k_kernel<LAY_I8>, dim3(nblocks(M * (K / 256), 4)), dim3(256), 0, s,
                               x, (int)M, (int)K, (uint8_t*)b.a0, b.sd, (void*)b.xs, act);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)M), block(256);
    if (fmt != FMT_Q4_K)  // Q8_0, Q6_K: the hi/lo split only
        hipLaunchKernelGGL(gemm_prep_kernel<FMT_Q8_0>, grid, block, 0, s, x, (int)M, (int)K, b.a0, b.a1, b.rs, b.xs);
    else
        hipLaunchKernelGGL(gemm_prep_kernel<FMT_Q4_K>, grid, block, 0, s, x, (int)M, (int)K, b.a0, b.a1, b.rs, b.xs);
    return hipGetLastError();
}

}  // namespace qmm
