// qmm_act.h -- activation arithmetic shared by every kernel that quantizes or
// splits activations (the standalone quantizer, the prefill preparation and the
// decode kernel's prologue), so all of them produce identical values.
#pragma once
#include "qmm_device.h"

namespace qmm {

// Q8_0 scale of a block of 32 values from its max|x| (page "自己量化", section
// 和下载的 Q8_0 逐字节比: the scale is max|x|/127): d = amax/127 in f32, the
// quantizer multiplies by id = 1/d (0 for an all-zero block), d is stored as
// f16 (nearest even).  Every Q8_0 activation quantizer goes through this and
// q8_0_q, so all of them produce identical blocks.
QMM_DEV void q8_0_scale(float amax, float& id, uint16_t& dbits, float& dval)
{
#pragma clang fp contract(off)
    const float d = amax / 127.0f;
    id = d != 0.0f ? 1.0f / d : 0.0f;
    dbits = f16bits(d);
    dval = f16round(d);
}
// q = round-half-away(x * id) with the unrounded scale.
QMM_DEV int q8_0_q(float x, float id)
{
#pragma clang fp contract(off)
    return (int)roundf(x * id);
}

QMM_DEV void q8_0_block(const float a[32], uint16_t& dbits, float& dval, int8_t q[32])
{
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(a[j]));
    float id;
    q8_0_scale(amax, id, dbits, dval);
#pragma unroll
    for (int j = 0; j < 32; ++j) q[j] = (int8_t)q8_0_q(a[j], id);
}

// Q8K: the signed element of largest |x| picks the scale, the first index
// winning ties (the sign of the scale depends on which of +-max comes first).
// From that element mx (and its |mx| = best): iscale = -127/mx, d = 1/iscale;
// an all-zero block gives iscale = d = 0.
QMM_DEV void q8k_scale(float mx, float best, float& iscale, float& d)
{
#pragma clang fp contract(off)
    iscale = 0.0f;
    d = 0.0f;
    if (best != 0.0f) {
        iscale = -127.0f / mx;
        d = 1.0f / iscale;
    }
}
// The signed element of largest |x| of a 256-value block held by 16
// consecutive lanes in index order (each lane's elements precede the next
// lane's), each lane passing `best`, the largest |x| of its elements, and
// `bv`, the first of them with that magnitude.  The block's max |x| is
// reduced over the 16 lanes; the lowest lane whose `best` reaches it holds the
// first element with it (first index on ties).  Every lane of the 16 gets
// that element, and the max |x| in `amax`.
QMM_DEV float q8k_row16_max(float best, float bv, float& amax)
{
    float am = best;
    am = fmaxf(am, dpp_f<DPP_X1>(am));
    am = fmaxf(am, dpp_f<DPP_X2>(am));
    am = fmaxf(am, dpp_f<DPP_HMIRROR>(am));
    am = fmaxf(am, dpp_f<DPP_MIRROR>(am));
    const int lane = (int)__lane_id();
    const uint64_t hit = __ballot(best == am);
    const uint32_t row = (uint32_t)(hit >> (lane & 48)) & 0xffffu;  // never 0: some lane holds the max
    amax = am;
    return __shfl(bv, (lane & 48) + __builtin_ctz(row));
}

// q = min(127, round-half-away(iscale * x)).
QMM_DEV int q8k_q(float x, float iscale)
{
#pragma clang fp contract(off)
    const int v = (int)roundf(iscale * x);
    return v < 127 ? v : 127;
}

QMM_DEV void load32(const float* __restrict__ v, float a[32])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 t = reinterpret_cast<const float4*>(v)[i];
        a[4 * i] = t.x; a[4 * i + 1] = t.y; a[4 * i + 2] = t.z; a[4 * i + 3] = t.w;
    }
}

// Q8K block of 256 values held by one wave, four per lane (elements
// 4*lane..4*lane+3).  The signed element of largest |x| (first index on
// ties) sets iscale = -127/max; q = min(127, round-half-away(iscale*x));
// d = 1/iscale; an all-zero block gives d = 0, q = 0.  On return lanes
// 4i..4i+3 hold bsums[i] in s16.
QMM_DEV void q8k_wave(const float xs[4], int lane, float& d, int q[4], int& s16)
{
    // the lane's largest |x| and the first of its elements with it
    float best = -1.0f, bv = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const float a = fabsf(xs[u]);
        if (a > best) { best = a; bv = xs[u]; }
    }
    // the block's max |x|; the lowest lane reaching it holds the first index
    float am = best;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) am = fmaxf(am, __shfl_xor(am, off));
    const int owner = __builtin_ctzll(__ballot(best == am));  // the same in every lane
    const float mx = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), owner));
    best = am;
    float iscale;
    q8k_scale(mx, best, iscale, d);
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = q8k_q(xs[u], iscale);
    int s = q[0] + q[1] + q[2] + q[3];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s16 = s;
}

// Mode (a) activation split.  A row (or a row's K range) is scaled by the
// power of two s = 2^sexp that puts its max|x| in [2^14, 2^15) (exact), then
// x*s = hi + lo + r with hi = f16(x*s), lo = f16(x*s - hi): |r| <= 2^-22|x*s|
// while lo is a normal f16.  Weights enter the matrix cores as exact small
// integers, so their products with hi and lo are exact.
QMM_DEV int split_exp(float amax)
{
    if (amax == 0.0f) return 0;
    const int e = 14 - ilogbf(amax);
    return e > 126 ? 126 : e;
}

QMM_DEV void split_one(float x, float s, _Float16& hi, _Float16& lo, float& xs)
{
#pragma clang fp contract(off)
    xs = x * s;
    hi = (_Float16)xs;
    lo = (_Float16)(xs - (float)hi);
}

QMM_DEV float split_chunk(const float a[32], float s, _Float16 hi[32], _Float16 lo[32])
{
#pragma clang fp contract(off)
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        const float xs = a[c] * s;
        const _Float16 h = (_Float16)xs;
        hi[c] = h;
        lo[c] = (_Float16)(xs - (float)h);
        acc += xs;
    }
    return acc;  // sum of x*s over the chunk (the Q4_K mins term needs it)
}

QMM_DEV uint32_t pack4(int a, int b, int c, int d)
{
    return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
           ((uint32_t)(uint8_t)d << 24);
}

// Canonical activation blocks, as the standalone quantizer writes them (and
// the traced runs copy out of the kernels that quantize): Q8_0 34 bytes
// (2-byte aligned): f16 d, int8 q[32].
QMM_DEV void store_q8_0_block(uint8_t* o, uint16_t dbits, const int8_t q[32])
{
    uint16_t* h = reinterpret_cast<uint16_t*>(o);
    h[0] = dbits;
#pragma unroll
    for (int j = 0; j < 16; ++j) h[1 + j] = (uint16_t)((uint8_t)q[2 * j] | ((uint16_t)(uint8_t)q[2 * j + 1] << 8));
}
// Q8K 292 bytes (4-byte aligned): f32 d, int8 q[256], int16 bsums[16]; the
// part held by one lane of the wave that quantized the block (q8k_wave: values
// 4*lane..4*lane+3, lanes 4i hold bsums[i]).
QMM_DEV void store_q8k_lane(uint8_t* o, int lane, float d, const int q[4], int s16)
{
    if (lane == 0) *reinterpret_cast<float*>(o) = d;
    *reinterpret_cast<uint32_t*>(o + 4 + 4 * lane) = pack4(q[0], q[1], q[2], q[3]);
    if ((lane & 3) == 0) *reinterpret_cast<int16_t*>(o + 260 + 2 * (lane >> 2)) = (int16_t)s16;
}

}  // namespace qmm
