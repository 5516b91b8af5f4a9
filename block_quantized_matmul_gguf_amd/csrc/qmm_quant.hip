// qmm_quant.hip -- activation quantizers, activation preparation for the
// decode (GEMV) and prefill (GEMM) kernels, and the weight quantizers.
//
// Q8_0 rule (page "自己量化", section 和下载的 Q8_0 逐字节比: the scale is
// max|x|/127): per 32 values d = amax/127 (f32), q = round-half-away(x * (1/d)),
// d stored as f16 (round to nearest even).  Q8K (the activation type of K-quant
// weights, page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处):
// per 256 values the signed element of largest |x| (first index on ties),
// iscale = -127/max, q = min(127, round(iscale*x)), d = 1/iscale, 16-value
// partial sums.  Every row is quantized on its own (page "自己量化", section
// 动脑筋答案).
#include "qmm_device.h"

namespace qmm {

enum { LAY_AOS = 0, LAY_GEMV = 1, LAY_GEMM = 2 };

// ----------------------------------------------------------------- Q8_0 ----

// One 32-value block: f16 scale bits, its f32 value, and the 32 int8 values.
QMM_DEV void q8_0_block(const float* __restrict__ v, uint16_t& dbits, float& dval, int8_t q[32])
{
#pragma clang fp contract(off)
    float a[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 t = reinterpret_cast<const float4*>(v)[i];
        a[4 * i] = t.x; a[4 * i + 1] = t.y; a[4 * i + 2] = t.z; a[4 * i + 3] = t.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float t = fabsf(a[j]);
        amax = t > amax ? t : amax;
    }
    const float d = amax / 127.0f;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    dbits = f16bits(d);
    dval = f16round(d);
#pragma unroll
    for (int j = 0; j < 32; ++j) q[j] = (int8_t)(int)roundf(a[j] * id);
}

QMM_DEV uint32_t pack4(int8_t a, int8_t b, int8_t c, int8_t d)
{
    return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
           ((uint32_t)(uint8_t)d << 24);
}

// One thread per block.  LAY_AOS: canonical 34-byte blocks.  LAY_GEMV: the
// decode kernel's int8 operand image plus scales [block][8].  LAY_GEMM: the
// values as f16 [M][K] plus scales [M][K/32].
template <int LAY>
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const float* __restrict__ x, int M, int K,
                                                            uint8_t* __restrict__ out, float* __restrict__ sc)
{
    const int nb = K / 32;
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= (int64_t)M * nb) return;
    const int m = (int)(blk / nb), b = (int)(blk % nb);
    uint16_t dbits;
    float dval;
    int8_t q[32];
    q8_0_block(x + (int64_t)m * K + 32 * b, dbits, dval, q);
    if (LAY == LAY_AOS) {
        uint16_t* o = reinterpret_cast<uint16_t*>(out + blk * 34);
        o[0] = dbits;
#pragma unroll
        for (int j = 0; j < 16; ++j) o[1 + j] = (uint16_t)((uint8_t)q[2 * j] | ((uint16_t)(uint8_t)q[2 * j + 1] << 8));
    } else if (LAY == LAY_GEMV) {
        // image[pair][g][row][8 bytes]; rows 0..M-1 even blocks, M..2M-1 odd blocks
        const int p = b >> 1, odd = b & 1;
        const int row = odd ? M + m : m;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int8_t s[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) s[t] = q[odd ? 8 * g + t : q8_even_k(g, t)];
            uint2 v = make_uint2(pack4(s[0], s[1], s[2], s[3]), pack4(s[4], s[5], s[6], s[7]));
            *reinterpret_cast<uint2*>(out + (((int64_t)p * 4 + g) * 2 * M + row) * 8) = v;
        }
        sc[b * 8 + m] = dval;
    } else {
        _Float16* o = reinterpret_cast<_Float16*>(out) + (int64_t)m * K + 32 * b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            half8_t h;
#pragma unroll
            for (int t = 0; t < 8; ++t) h[t] = (_Float16)(float)q[8 * i + t];
            reinterpret_cast<half8_t*>(o)[i] = h;
        }
        sc[(int64_t)m * nb + b] = dval;
    }
}

// ------------------------------------------------------------------ Q8K ----

// One wave per 256-value block, four blocks per 256-thread workgroup.
// LAY_AOS: canonical 292-byte blocks.  LAY_GEMV: int8 operand image
// [block][chunk c][g][row][8] (rows 0..M-1 sub-block 2c, M..2M-1 sub-block
// 2c+1), scales [block][8], bsum pairs [block][j][8].  LAY_GEMM: values as f16
// [M][K], scales [M][K/256], bsum pairs [M][K/32].
template <int LAY>
__global__ __launch_bounds__(256) void quantize_q8k_kernel(const float* __restrict__ x, int M, int K,
                                                           uint8_t* __restrict__ out, float* __restrict__ sc,
                                                           int32_t* __restrict__ bs)
{
#pragma clang fp contract(off)
    const int nsb = K / 256;
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= (int64_t)M * nsb) return;  // whole wave leaves together
    const int m = (int)(blk / nsb), sb = (int)(blk % nsb);
    const float4 xv = reinterpret_cast<const float4*>(x + (int64_t)m * K + 256 * sb)[lane];
    const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
    float best = -1.0f;
    int bi = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float a = fabsf(xs[u]);
        if (a > best) { best = a; bi = 4 * lane + u; }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    const float mine = xs[0] * (float)((bi & 3) == 0) + xs[1] * (float)((bi & 3) == 1) +
                       xs[2] * (float)((bi & 3) == 2) + xs[3] * (float)((bi & 3) == 3);
    const float mx = __shfl(mine, bi >> 2);
    int q[4] = {0, 0, 0, 0};
    float d = 0.0f;
    if (best != 0.0f) {
        const float iscale = -127.0f / mx;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = (int)roundf(iscale * xs[u]);
            q[u] = v < 127 ? v : 127;
        }
        d = 1.0f / iscale;
    }
    int s = q[0] + q[1] + q[2] + q[3];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);  // lanes 4i..4i+3 now hold bsums[i]
    const uint32_t packed = pack4((int8_t)q[0], (int8_t)q[1], (int8_t)q[2], (int8_t)q[3]);
    if (LAY == LAY_AOS) {
        uint8_t* o = out + blk * 292;
        if (lane == 0) *reinterpret_cast<float*>(o) = d;
        *reinterpret_cast<uint32_t*>(o + 4 + 4 * lane) = packed;
        if ((lane & 3) == 0) *reinterpret_cast<int16_t*>(o + 260 + 2 * (lane >> 2)) = (int16_t)s;
    } else {
        const int pair = s + __shfl_down(s, 4);  // lane 8j: bsums[2j] + bsums[2j+1]
        if (LAY == LAY_GEMV) {
            const int e = 4 * lane, c = e >> 6, w = e & 63, half = w >> 5, g = (w & 31) >> 3, t0 = w & 7;
            const int row = half ? M + m : m;
            *reinterpret_cast<uint32_t*>(out + ((((int64_t)sb * 4 + c) * 4 + g) * 2 * M + row) * 8 + t0) = packed;
            if (lane == 0) sc[sb * 8 + m] = d;
            if ((lane & 7) == 0) bs[(sb * 8 + (lane >> 3)) * 8 + m] = pair;
        } else {
            _Float16* o = reinterpret_cast<_Float16*>(out) + (int64_t)m * K + 256 * sb + 4 * lane;
            o[0] = (_Float16)(float)q[0]; o[1] = (_Float16)(float)q[1];
            o[2] = (_Float16)(float)q[2]; o[3] = (_Float16)(float)q[3];
            if (lane == 0) sc[(int64_t)m * nsb + sb] = d;
            if ((lane & 7) == 0) bs[(int64_t)m * (K / 32) + 8 * sb + (lane >> 3)] = pair;
        }
    }
}

// ------------------------------------------- mode (a): f16 hi/lo split ----

// One workgroup per activation row.  The row is scaled by a power of two s so
// that max|x*s| lies in [2^14, 2^15) (exact), then split x*s = hi + lo + r
// with hi = f16(x*s), lo = f16(x*s - hi), |r| <= 2^-22 |x*s| for normal lo.
// Weights enter the matrix cores as exact small integers, so products with
// hi and lo are exact and only f32 accumulation rounds.
// LAY_GEMV: image[unit32][g][row][8] f16 (rows 0..M-1 hi, M..2M-1 lo) in the
// k order of the weight decoder; sc0[m] = 1/s; Q4_K also sub-block sums of
// x*s [K/32][8].  LAY_GEMM: hi [M][K], lo [M][K], sc0[m], sums [M][K/32].
template <int LAY, int FMT>
__global__ __launch_bounds__(256) void split_x_kernel(const float* __restrict__ x, int M, int K,
                                                      _Float16* __restrict__ o0, _Float16* __restrict__ o1,
                                                      float* __restrict__ sc0, float* __restrict__ sums)
{
#pragma clang fp contract(off)
    __shared__ float red[4];
    const int m = blockIdx.x;
    const float* v = x + (int64_t)m * K;
    float am = 0.0f;
    for (int k = 4 * threadIdx.x; k < K; k += 1024) {
        const float4 t = *reinterpret_cast<const float4*>(v + k);
        am = fmaxf(am, fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w))));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int sexp = 0;
    if (am != 0.0f) {
        sexp = 14 - ilogbf(am);
        sexp = sexp > 126 ? 126 : sexp;
    }
    const float s = ldexpf(1.0f, sexp);
    if (threadIdx.x == 0) sc0[m] = ldexpf(1.0f, -sexp);
    const int n32 = K / 32;
    for (int u = threadIdx.x; u < n32; u += 256) {
        _Float16 hi[32], lo[32];
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 t = reinterpret_cast<const float4*>(v + 32 * u)[i];
            const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float xs = tv[c] * s;
                const _Float16 h = (_Float16)xs;
                hi[4 * i + c] = h;
                lo[4 * i + c] = (_Float16)(xs - (float)h);
                acc += xs;
            }
        }
        if (LAY == LAY_GEMV) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                half8_t vh, vl;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    int k;
                    if (FMT == FMT_Q8_0) k = (u & 1) ? 8 * g + t : q8_even_k(g, t);
                    else k = 8 * g + nib_perm(t);
                    vh[t] = hi[k];
                    vl[t] = lo[k];
                }
                half8_t* img = reinterpret_cast<half8_t*>(o0);
                img[((int64_t)u * 4 + g) * 2 * M + m] = vh;
                img[((int64_t)u * 4 + g) * 2 * M + M + m] = vl;
            }
            if (FMT == FMT_Q4_K) sums[u * 8 + m] = acc;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                half8_t vh, vl;
#pragma unroll
                for (int t = 0; t < 8; ++t) { vh[t] = hi[8 * i + t]; vl[t] = lo[8 * i + t]; }
                reinterpret_cast<half8_t*>(o0 + (int64_t)m * K + 32 * u)[i] = vh;
                reinterpret_cast<half8_t*>(o1 + (int64_t)m * K + 32 * u)[i] = vl;
            }
            if (FMT == FMT_Q4_K) sums[(int64_t)m * n32 + u] = acc;
        }
    }
}

// ---------------------------------------------------- Q4_K weights ----

// One thread per 256-value super-block.  Per 32-value sub-block an affine
// fit lo = min(0, min x), hi = max x, scale = (hi-lo)/15, min = -lo; the 6-bit
// sc_j, m_j quantize scale and min against the super-block maxima / 63
// (d = max scale/63, dmin = max min/63, stored as f16); the 4-bit values are
// re-quantized against the stored scales: q = clamp(round((x + dmin*m_j) /
// (d*sc_j)), 0, 15).  (The pages name QTensor::quantize(&w, Q4K) but not its
// search, page "自己量化", section "3. 量化"; this is the plain min/max rule.)
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
        float lo = 0.0f, hi = v[32 * j];
        for (int l = 0; l < 32; ++l) {
            const float t = v[32 * j + l];
            lo = t < lo ? t : lo;
            hi = t > hi ? t : hi;
        }
        scale[j] = (hi - lo) / 15.0f;
        minv[j] = -lo;
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
    uint8_t b[144];
    b[0] = (uint8_t)dh; b[1] = (uint8_t)(dh >> 8);
    b[2] = (uint8_t)mh; b[3] = (uint8_t)(mh >> 8);
    for (int j = 0; j < 4; ++j) {
        b[4 + j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        b[8 + j] = (uint8_t)((mn[j] & 63) | ((mn[j + 4] >> 4) << 6));
        b[12 + j] = (uint8_t)((sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4));
    }
    for (int i = 0; i < 128; ++i) b[16 + i] = 0;
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
        if (l < 32) b[16 + 32 * c + l] |= (uint8_t)q;
        else b[16 + 32 * c + l - 32] |= (uint8_t)(q << 4);
    }
    uint4* o = reinterpret_cast<uint4*>(out + blk * 144);
    for (int i = 0; i < 9; ++i) {
        uint4 t;
        t.x = b[16 * i] | (b[16 * i + 1] << 8) | (b[16 * i + 2] << 16) | ((uint32_t)b[16 * i + 3] << 24);
        t.y = b[16 * i + 4] | (b[16 * i + 5] << 8) | (b[16 * i + 6] << 16) | ((uint32_t)b[16 * i + 7] << 24);
        t.z = b[16 * i + 8] | (b[16 * i + 9] << 8) | (b[16 * i + 10] << 16) | ((uint32_t)b[16 * i + 11] << 24);
        t.w = b[16 * i + 12] | (b[16 * i + 13] << 8) | (b[16 * i + 14] << 16) | ((uint32_t)b[16 * i + 15] << 24);
        o[i] = t;
    }
}

// ------------------------------------------------------------ launchers ----

static unsigned nblocks(int64_t items, int per) { return (unsigned)((items + per - 1) / per); }

hipError_t launch_quantize_act(int act_fmt, const float* x, int64_t M, int64_t K, void* out, hipStream_t s)
{
    if (act_fmt == FMT_Q8_0) {
        hipLaunchKernelGGL(quantize_q8_0_kernel<LAY_AOS>, dim3(nblocks(M * (K / 32), 256)), dim3(256), 0, s,
                           x, (int)M, (int)K, (uint8_t*)out, (float*)nullptr);
    } else {
        hipLaunchKernelGGL(quantize_q8k_kernel<LAY_AOS>, dim3(nblocks(M * (K / 256), 4)), dim3(256), 0, s,
                           x, (int)M, (int)K, (uint8_t*)out, (float*)nullptr, (int32_t*)nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_weights(int fmt, const float* w, int64_t N, int64_t K, void* out, hipStream_t s)
{
    if (fmt == FMT_Q8_0) return launch_quantize_act(FMT_Q8_0, w, N, K, out, s);
    hipLaunchKernelGGL(quantize_q4_k_kernel, dim3(nblocks(N * (K / 256), 256)), dim3(256), 0, s,
                       w, (int)N, (int)K, (uint8_t*)out);
    return hipGetLastError();
}

hipError_t launch_gemv_prep(int fmt, int mode, const float* x, int M, int64_t K, const GemvBufs& b, hipStream_t s)
{
    if (mode == MODE_A) {
        if (fmt == FMT_Q8_0)
            hipLaunchKernelGGL((split_x_kernel<LAY_GEMV, FMT_Q8_0>), dim3(M), dim3(256), 0, s, x, M, (int)K,
                               (_Float16*)b.img, (_Float16*)nullptr, b.sc0, (float*)nullptr);
        else
            hipLaunchKernelGGL((split_x_kernel<LAY_GEMV, FMT_Q4_K>), dim3(M), dim3(256), 0, s, x, M, (int)K,
                               (_Float16*)b.img, (_Float16*)nullptr, b.sc0, (float*)b.sc1);
    } else if (fmt == FMT_Q8_0) {
        hipLaunchKernelGGL(quantize_q8_0_kernel<LAY_GEMV>, dim3(nblocks((int64_t)M * (K / 32), 256)), dim3(256), 0, s,
                           x, M, (int)K, (uint8_t*)b.img, b.sc0);
    } else {
        hipLaunchKernelGGL(quantize_q8k_kernel<LAY_GEMV>, dim3(nblocks((int64_t)M * (K / 256), 4)), dim3(256), 0, s,
                           x, M, (int)K, (uint8_t*)b.img, b.sc0, (int32_t*)b.sc1);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_prep(int fmt, int mode, const float* x, int64_t M, int64_t K, const GemmBufs& b, hipStream_t s)
{
    if (mode == MODE_A) {
        if (fmt == FMT_Q8_0)
            hipLaunchKernelGGL((split_x_kernel<LAY_GEMM, FMT_Q8_0>), dim3((unsigned)M), dim3(256), 0, s, x, (int)M,
                               (int)K, b.a0, b.a1, b.sc0, (float*)nullptr);
        else
            hipLaunchKernelGGL((split_x_kernel<LAY_GEMM, FMT_Q4_K>), dim3((unsigned)M), dim3(256), 0, s, x, (int)M,
                               (int)K, b.a0, b.a1, b.sc0, (float*)b.sc1);
    } else if (fmt == FMT_Q8_0) {
        hipLaunchKernelGGL(quantize_q8_0_kernel<LAY_GEMM>, dim3(nblocks(M * (K / 32), 256)), dim3(256), 0, s,
                           x, (int)M, (int)K, (uint8_t*)b.a0, b.sc0);
    } else {
        hipLaunchKernelGGL(quantize_q8k_kernel<LAY_GEMM>, dim3(nblocks(M * (K / 256), 4)), dim3(256), 0, s,
                           x, (int)M, (int)K, (uint8_t*)b.a0, b.sc0, (int32_t*)b.sc1);
    }
    return hipGetLastError();
}

}  // namespace qmm
