/*
 * qmm_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU reference for y = x . W^T with W held
 * as GGUF quantized blocks, in the two numerical forms the pages contrast:
 *
 *   mode (a)  f32 activations times weights dequantized from their blocks
 *             (the "Metal" form: page "同一个 GGUF，CPU 和 Metal 生成的文字不一样",
 *             section 出处);
 *   mode (b)  each activation row first quantized to Q8_0 (for Q8_0 weights) or
 *             Q8K (for K-quant weights), then integer block dot products scaled
 *             by the two block scales (the "CPU" form, same section; row-local
 *             quantization per page "自己量化", section 动脑筋答案).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header or table with the GPU path.
 *
 * Precision: mode (a) accumulates in double over weights dequantized exactly
 * (an f16 scale times a small integer is exact in double).  Mode (b) forms the
 * integer block sums in int64 and combines them with the scales in double.
 *
 * Block layouts (little-endian):
 *   Q8_0  34 B per 32 weights: f16 d, int8 q[32];  w_j = d*q_j.
 *   Q4_K 144 B per 256 weights: f16 d, f16 dmin, 12 B of 6-bit sub-block
 *         scales/mins, 128 B of 4-bit values; w = d*sc_j*q - dmin*m_j.
 *   Q8K  292 B per 256 activations: f32 d, int8 q[256], int16 bsums[16].
 *   Q4_0  18 B per 32 weights: f16 d, 16 B of 4-bit values; w = d*(q - 8).
 *   Q5_0  22 B per 32 weights: f16 d, 4 B of fifth bits, 16 B of 4-bit values;
 *         w = d*(q - 16).
 *   Q6_K 210 B per 256 weights: 128 B low 4 bits, 64 B high 2 bits, int8
 *         scales[16] (one per 16 values), f16 d; w = d*sc_j*(q - 32).
 * The byte sizes of Q8_0, Q4_K, Q4_0 and Q5_0 are fixed by the pages' byte
 * counts (page "自己量化", sections 和下载的 Q8_0 逐字节比 and 大小和误差);
 * Q6_K's is not.  The pages do not print the field order or any bit packing;
 * this file uses the public GGUF layout.  The packings are therefore pinned
 * only by hand-built blocks in the tests (parity of the packings unpinned by
 * the pages themselves).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC.
 * No fast-math: every float operation below is one IEEE-754 binary32 or
 * binary64 operation, rounded to nearest-even.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_Q4_0 2
#define ORC_Q5_0 6
#define ORC_Q8_0 8
#define ORC_Q4_K 12
#define ORC_Q6_K 14
#define ORC_Q8_K 15

#define Q8_0_QK 32
#define Q8_0_BYTES 34
#define QK_K 256
#define Q4_K_BYTES 144
#define Q8_K_BYTES 292
#define Q4_0_BYTES 18
#define Q5_0_BYTES 22
#define Q6_K_BYTES 210

/* ---------------------------------------------------------------- f16 ---- */

/* binary32 -> binary16, round to nearest, ties to even, subnormals kept. */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);   /* NaN */
    if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  /* >= 65520 -> inf */
    if (a >= 0x38800000u) {                                   /* f16 normal range */
        uint32_t mant = a & 0x7fffffu;
        uint32_t exp = (a >> 23) - 127u + 15u;
        uint32_t h = (exp << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;
        return (uint16_t)(sign | h);
    }
    int e = (int)(a >> 23) - 127;
    if (e < -25) return sign;                                 /* below half of 2^-24 */
    uint32_t full = (a & 0x7fffffu) | 0x800000u;              /* |f| = full * 2^(e-23) */
    int shift = -(e + 1);                                     /* 14 .. 24 */
    uint32_t m = full >> shift;
    uint32_t rem = full & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (m & 1u))) m += 1u;
    return (uint16_t)(sign | m);
}

double orc_f16_to_f64(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m | 0x400), e - 25);
    return s ? -v : v;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static float rdf32(const uint8_t* p) { float f; memcpy(&f, p, 4); return f; }
static void wrf32(uint8_t* p, float f) { memcpy(p, &f, 4); }

/* round half away from zero ("round"); ties-to-even when even != 0 */
static int round_q(float t, int even) { return even ? (int)rintf(t) : (int)roundf(t); }

/* ---------------------------------------------------------- quantizers -- */

/*
 * Q8_0, 32 values per block.  Scale = max|x| / 127 ("no freedom", page
 * "自己量化", section 和下载的 Q8_0 逐字节比); q = round(x / d) evaluated as
 * x * (1/d) with the unrounded f32 d; d is stored rounded to f16.
 * variant bit0: use x / d instead of x * (1/d); bit1: round ties to even.
 * The same rule quantizes weights and (mode b) activation rows.
 */
void orc_quantize_q8_0_v(const float* x, int64_t rows, int64_t K, uint8_t* out, int variant)
{
    const int64_t nb = K / Q8_0_QK;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* v = x + r * K + b * Q8_0_QK;
            uint8_t* blk = out + (r * nb + b) * Q8_0_BYTES;
            float amax = 0.0f;
            for (int j = 0; j < Q8_0_QK; ++j) {
                float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            float d = amax / 127.0f;
            float id = d != 0.0f ? 1.0f / d : 0.0f;
            wr16(blk, orc_f32_to_f16(d));
            for (int j = 0; j < Q8_0_QK; ++j) {
                float t;
                if (variant & 1) t = d != 0.0f ? v[j] / d : 0.0f;
                else t = v[j] * id;
                blk[2 + j] = (uint8_t)(int8_t)round_q(t, variant & 2);
            }
        }
    }
}

void orc_quantize_q8_0(const float* x, int64_t rows, int64_t K, uint8_t* out)
{
    orc_quantize_q8_0_v(x, rows, K, out, 0);
}

/*
 * Q8K, 256 values per block (the activation type paired with K-quant weights,
 * page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处).  The pages
 * name only "per 256"; the rule here: take the element of largest |x| (first
 * index on ties) with its sign, iscale = -127/max, q = min(127, round(iscale*x)),
 * d = 1/iscale, bsums[i] = sum of q over 16-element group i.
 * variant bit0: iscale = -128/max; bit1: round ties to even.
 */
void orc_quantize_q8k_v(const float* x, int64_t rows, int64_t K, uint8_t* out, int variant)
{
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* v = x + r * K + b * QK_K;
            uint8_t* blk = out + (r * nb + b) * Q8_K_BYTES;
            int8_t* qs = (int8_t*)(blk + 4);
            float amax = 0.0f, mx = 0.0f;
            for (int j = 0; j < QK_K; ++j) {
                float a = fabsf(v[j]);
                if (a > amax) { amax = a; mx = v[j]; }
            }
            if (amax == 0.0f) {
                memset(blk, 0, Q8_K_BYTES);
                continue;
            }
            float iscale = ((variant & 1) ? -128.0f : -127.0f) / mx;
            for (int j = 0; j < QK_K; ++j) {
                int q = round_q(iscale * v[j], variant & 2);
                if (q > 127) q = 127;
                qs[j] = (int8_t)q;
            }
            for (int i = 0; i < 16; ++i) {
                int s = 0;
                for (int l = 0; l < 16; ++l) s += qs[16 * i + l];
                wr16(blk + 260 + 2 * i, (uint16_t)(int16_t)s);
            }
            wrf32(blk, 1.0f / iscale);
        }
    }
}

void orc_quantize_q8k(const float* x, int64_t rows, int64_t K, uint8_t* out)
{
    orc_quantize_q8k_v(x, rows, K, out, 0);
}

/* Q4_K 6-bit scale/min of sub-block j from the 12 packed bytes s[]. */
static void q4k_scale_min(const uint8_t* s, int j, int* sc, int* m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 0x0f) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* 4-bit value of element e (0..255) of a Q4_K super-block's 128 value bytes. */
static int q4k_nibble(const uint8_t* qs, int e)
{
    int c = e / 64, l = e % 64;
    uint8_t byte = qs[32 * c + (l % 32)];
    return l < 32 ? (byte & 0x0f) : (byte >> 4);
}

/*
 * Q4_K weights for synthetic tests (the pages name QTensor::quantize(&w, Q4K)
 * but not its search, page "自己量化", section 3. 量化).  Plainest rule:
 * per 32-element sub-block an affine min/max fit, its scale and min quantized
 * to 6 bits against the super-block maximum / 63, then the 4-bit values
 * re-quantized against the stored f16 scales.
 */
/* The super-block stage shared by both Q4_K rules: given each sub-block's
 * scale and min (>= 0), d = max scale / 63 and dmin = max min / 63 (stored as
 * f16), 6-bit sc_j and m_j against those maxima, then every value requantized
 * against the stored effective scale and min. */
static void q4k_pack(const float* v, const float scale[8], const float minv[8], uint8_t* blk)
{
    float max_scale = 0.0f, max_min = 0.0f;
    for (int j = 0; j < 8; ++j) {
        if (scale[j] > max_scale) max_scale = scale[j];
        if (minv[j] > max_min) max_min = minv[j];
    }
    int sc[8], mn[8];
    float isc = max_scale > 0.0f ? 63.0f / max_scale : 0.0f;
    float imn = max_min > 0.0f ? 63.0f / max_min : 0.0f;
    for (int j = 0; j < 8; ++j) {
        int a = (int)roundf(isc * scale[j]);
        int c = (int)roundf(imn * minv[j]);
        sc[j] = a > 63 ? 63 : a;
        mn[j] = c > 63 ? 63 : c;
    }
    uint16_t dh = orc_f32_to_f16(max_scale / 63.0f);
    uint16_t mh = orc_f32_to_f16(max_min / 63.0f);
    wr16(blk, dh);
    wr16(blk + 2, mh);
    uint8_t* s = blk + 4;
    for (int j = 0; j < 4; ++j) {
        s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
        s[j + 4] = (uint8_t)((mn[j] & 63) | ((mn[j + 4] >> 4) << 6));
        s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4));
    }
    float dq = (float)orc_f16_to_f64(dh);
    float mq = (float)orc_f16_to_f64(mh);
    uint8_t* qs = blk + 16;
    memset(qs, 0, 128);
    for (int e = 0; e < QK_K; ++e) {
        int j = e / 32;
        float d_eff = dq * (float)sc[j];
        float m_eff = mq * (float)mn[j];
        int q = 0;
        if (d_eff != 0.0f) {
            q = (int)roundf((v[e] + m_eff) / d_eff);
            if (q < 0) q = 0;
            if (q > 15) q = 15;
        }
        int c = e / 64, l = e % 64;
        if (l < 32) qs[32 * c + l] |= (uint8_t)q;
        else qs[32 * c + (l - 32)] |= (uint8_t)(q << 4);
    }
}

/* lo = min(0, min x), hi = max x over a 32-value sub-block */
static void sub_range(const float* x, float* lo, float* hi)
{
    *lo = 0.0f;
    *hi = x[0];
    for (int l = 0; l < 32; ++l) {
        if (x[l] < *lo) *lo = x[l];
        if (x[l] > *hi) *hi = x[l];
    }
}

void orc_quantize_q4_k(const float* w, int64_t rows, int64_t K, uint8_t* out)
{
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* v = w + r * K + b * QK_K;
            float scale[8], minv[8];
            for (int j = 0; j < 8; ++j) {
                float lo, hi;
                sub_range(v + 32 * j, &lo, &hi);
                scale[j] = (hi - lo) / 15.0f;
                minv[j] = -lo;
            }
            q4k_pack(v, scale, minv, out + (r * nb + b) * Q4_K_BYTES);
        }
    }
}

/*
 * Q4_K weights with a search for each sub-block's scale and min (the page
 * "自己量化", section "3. 量化", names QTensor::quantize(&w, Q4K) but not its
 * search; this is a plain least-squares search written from the definition
 * of the format).  For a sub-block x[0..31] with lo = min(0, min x), hi =
 * max x, r = hi - lo:
 *   candidate codes q_l = clamp(round((x_l - lo) * c), 0, 15) for the plain
 *   rule's c = 15 / r and for c = (140 + k) / (10 r), k = 0..20 (steps of
 *   0.1 around 15 codes per range);
 *   for each, the least-squares line x ~ a q + b over the 32 values (b forced
 *   to 0 by refitting a alone when the fit gives b > 0: the format's offset
 *   is -dmin*m <= 0), a candidate with a <= 0 or all codes equal skipped;
 *   kept: the first candidate of smallest squared error sum (a q + b - x)^2,
 *   the plain rule's (a = r/15, b = lo) competing first.
 * Then scale = a, min = -b, and the super-block stage of the plain rule.
 * All sums run in index order in f32, one IEEE operation at a time.
 */
static void q4k_search_fit(const float* x, float* scale, float* minv)
{
    float lo, hi;
    sub_range(x, &lo, &hi);
    const float r = hi - lo;
    float best_a = r / 15.0f, best_b = lo;
    if (r == 0.0f) {
        *scale = best_a;
        *minv = -best_b;
        return;
    }
    float best_e = 0.0f;
    {
        const float c = 15.0f / r;
        for (int l = 0; l < 32; ++l) {
            int q = (int)roundf((x[l] - lo) * c);
            q = q < 0 ? 0 : q > 15 ? 15 : q;
            const float t = best_a * (float)q + best_b - x[l];
            best_e = best_e + t * t;
        }
    }
    for (int k = 0; k <= 20; ++k) {
        const float c = (float)(140 + k) / (10.0f * r);
        int q[32], sq = 0, sqq = 0;
        float sx = 0.0f, sqx = 0.0f;
        for (int l = 0; l < 32; ++l) {
            int v = (int)roundf((x[l] - lo) * c);
            v = v < 0 ? 0 : v > 15 ? 15 : v;
            q[l] = v;
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
            const float t = a * (float)q[l] + b - x[l];
            e = e + t * t;
        }
        if (e < best_e) {
            best_e = e;
            best_a = a;
            best_b = b;
        }
    }
    *scale = best_a;
    *minv = -best_b;
}

void orc_quantize_q4_k_search(const float* w, int64_t rows, int64_t K, uint8_t* out)
{
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* v = w + r * K + b * QK_K;
            float scale[8], minv[8];
            for (int j = 0; j < 8; ++j) q4k_search_fit(v + 32 * j, &scale[j], &minv[j]);
            q4k_pack(v, scale, minv, out + (r * nb + b) * Q4_K_BYTES);
        }
    }
}

/* The signed element of largest |x| among n (first index on ties); 0 if all 0. */
static float signed_absmax(const float* v, int n)
{
    float amax = 0.0f, mx = 0.0f;
    for (int j = 0; j < n; ++j) {
        float a = fabsf(v[j]);
        if (a > amax) { amax = a; mx = v[j]; }
    }
    return mx;
}

/*
 * Q4_0 (offset 8) and Q5_0 (offset 16) weights, 32 values per block, for
 * synthetic inputs: the page "自己量化" (section 3. 量化) names
 * QTensor::quantize to Q4_0, and to Q5_0 for rows K-quants cannot take, but
 * not the rule.  Rule used: the signed element of largest |x| maps to the
 * most negative code, d = max / -offset, q = floor(x * (1/d) + offset + 1/2)
 * capped at 2*offset - 1 (the public GGUF reference rule); d stored as f16.
 * Element j < 16 is the low nibble of value byte j, element j + 16 its high
 * nibble; Q5_0 keeps bit 4 of element j in bit j of a little-endian u32.
 */
static void quantize_q4_q5_0(const float* w, int64_t rows, int64_t K, uint8_t* out, int five)
{
    const int64_t nb = K / 32;
    const int bytes = five ? Q5_0_BYTES : Q4_0_BYTES;
    const float off = five ? 16.0f : 8.0f;
    const int qmax = five ? 31 : 15;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* v = w + r * K + b * 32;
            uint8_t* blk = out + (r * nb + b) * bytes;
            float mx = signed_absmax(v, 32);
            float d = mx / -off;
            float id = d != 0.0f ? 1.0f / d : 0.0f;
            wr16(blk, orc_f32_to_f16(d));
            uint8_t* qs = blk + (five ? 6 : 2);
            uint32_t qh = 0;
            memset(qs, 0, 16);
            for (int j = 0; j < 32; ++j) {
                float t = v[j] * id;
                t = t + (off + 0.5f);
                int q = (int)t; /* t > 0 here, so truncation is floor */
                if (q > qmax) q = qmax;
                qs[j % 16] |= (uint8_t)((q & 15) << (j < 16 ? 0 : 4));
                qh |= (uint32_t)((q >> 4) & 1) << j;
            }
            if (five) {
                blk[2] = (uint8_t)qh;
                blk[3] = (uint8_t)(qh >> 8);
                blk[4] = (uint8_t)(qh >> 16);
                blk[5] = (uint8_t)(qh >> 24);
            }
        }
    }
}

void orc_quantize_q4_0(const float* w, int64_t rows, int64_t K, uint8_t* out)
{
    quantize_q4_q5_0(w, rows, K, out, 0);
}

void orc_quantize_q5_0(const float* w, int64_t rows, int64_t K, uint8_t* out)
{
    quantize_q4_q5_0(w, rows, K, out, 1);
}

/* Byte offsets of element e (0..255) of a Q6_K super-block: the low-bits
 * byte (nibble *nib: 0 low, 1 high) and the high-bits byte (bit pair *pair). */
static void q6k_where(int e, int* lo_byte, int* nib, int* hi_byte, int* pair)
{
    int half = e / 128, el = e % 128, g = el / 32, l = el % 32;
    *lo_byte = 64 * half + 32 * (g & 1) + l;
    *nib = g >> 1;
    *hi_byte = 128 + 32 * half + l;
    *pair = g;
}

/* 6-bit value (0..63) of element e of a Q6_K super-block. */
static int q6k_value(const uint8_t* blk, int e)
{
    int lb, nib, hb, pair;
    q6k_where(e, &lb, &nib, &hb, &pair);
    int lo = nib ? (blk[lb] >> 4) : (blk[lb] & 15);
    int hi = (blk[hb] >> (2 * pair)) & 3;
    return lo | (hi << 4);
}

/*
 * Q6_K weights for synthetic inputs (the pages name Q6K tensors of a
 * downloaded file, page "自己量化", section 和下载的 Q8_0 逐字节比, but no
 * quantizer).  Plain rule: per 16-value sub-block j the signed element of
 * largest |x| gives s_j = max / -32; over the super-block the signed s_j of
 * largest |s_j| gives d = s / -128; sc_j = min(127, round(s_j / d)); each
 * value q = clamp(round(x / (d*sc_j)), -32, 31) + 32 against the stored f16 d
 * (q = 32 where d*sc_j is 0).
 */
void orc_quantize_q6_k(const float* w, int64_t rows, int64_t K, uint8_t* out)
{
    const int64_t nb = K / QK_K;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const float* v = w + r * K + b * QK_K;
            uint8_t* blk = out + (r * nb + b) * Q6_K_BYTES;
            float s[16];
            for (int j = 0; j < 16; ++j) s[j] = signed_absmax(v + 16 * j, 16) / -32.0f;
            float smax = signed_absmax(s, 16);
            float d = smax / -128.0f;
            uint16_t dh = orc_f32_to_f16(d);
            float dq = (float)orc_f16_to_f64(dh);
            memset(blk, 0, Q6_K_BYTES);
            int sc[16];
            for (int j = 0; j < 16; ++j) {
                int c = d != 0.0f ? (int)roundf(s[j] / d) : 0;
                sc[j] = c > 127 ? 127 : c;
                blk[192 + j] = (uint8_t)(int8_t)sc[j];
            }
            wr16(blk + 208, dh);
            for (int e = 0; e < QK_K; ++e) {
                float de = dq * (float)sc[e / 16];
                int q = 0;
                if (de != 0.0f) {
                    q = (int)roundf(v[e] / de);
                    if (q < -32) q = -32;
                    if (q > 31) q = 31;
                }
                q += 32;
                int lb, nib, hb, pair;
                q6k_where(e, &lb, &nib, &hb, &pair);
                blk[lb] |= (uint8_t)((q & 15) << (4 * nib));
                blk[hb] |= (uint8_t)((q >> 4) << (2 * pair));
            }
        }
    }
}

/* 5-bit value (0..31) of element j of a Q5_0 block, 4-bit of a Q4_0 block. */
static int q5_0_value(const uint8_t* blk, int j)
{
    uint32_t qh = (uint32_t)blk[2] | ((uint32_t)blk[3] << 8) | ((uint32_t)blk[4] << 16) | ((uint32_t)blk[5] << 24);
    int lo = j < 16 ? (blk[6 + j] & 15) : (blk[6 + j - 16] >> 4);
    return lo | (int)(((qh >> j) & 1u) << 4);
}

static int q4_0_value(const uint8_t* blk, int j)
{
    return j < 16 ? (blk[2 + j] & 15) : (blk[2 + j - 16] >> 4);
}

/* ------------------------------------------------------------ decoders -- */

static int64_t row_bytes(int fmt, int64_t K)
{
    if (fmt == ORC_Q8_0) return (K / Q8_0_QK) * Q8_0_BYTES;
    if (fmt == ORC_Q4_K) return (K / QK_K) * Q4_K_BYTES;
    if (fmt == ORC_Q8_K) return (K / QK_K) * Q8_K_BYTES;
    if (fmt == ORC_Q4_0) return (K / 32) * Q4_0_BYTES;
    if (fmt == ORC_Q5_0) return (K / 32) * Q5_0_BYTES;
    if (fmt == ORC_Q6_K) return (K / QK_K) * Q6_K_BYTES;
    return -1;
}

int64_t orc_row_bytes(int fmt, int64_t K) { return row_bytes(fmt, K); }

/* Dequantize one row of K values (exact in double). */
static void dequant_row(int fmt, const uint8_t* row, int64_t K, double* out)
{
    if (fmt == ORC_Q8_0) {
        for (int64_t b = 0; b < K / Q8_0_QK; ++b) {
            const uint8_t* blk = row + b * Q8_0_BYTES;
            double d = orc_f16_to_f64(rd16(blk));
            for (int j = 0; j < Q8_0_QK; ++j) out[b * Q8_0_QK + j] = d * (double)(int8_t)blk[2 + j];
        }
    } else if (fmt == ORC_Q4_K) {
        for (int64_t b = 0; b < K / QK_K; ++b) {
            const uint8_t* blk = row + b * Q4_K_BYTES;
            double d = orc_f16_to_f64(rd16(blk));
            double dmin = orc_f16_to_f64(rd16(blk + 2));
            for (int e = 0; e < QK_K; ++e) {
                int sc, m;
                q4k_scale_min(blk + 4, e / 32, &sc, &m);
                out[b * QK_K + e] = d * sc * q4k_nibble(blk + 16, e) - dmin * m;
            }
        }
    } else if (fmt == ORC_Q8_K) {
        for (int64_t b = 0; b < K / QK_K; ++b) {
            const uint8_t* blk = row + b * Q8_K_BYTES;
            double d = (double)rdf32(blk);
            for (int j = 0; j < QK_K; ++j) out[b * QK_K + j] = d * (double)(int8_t)blk[4 + j];
        }
    } else if (fmt == ORC_Q4_0 || fmt == ORC_Q5_0) {
        const int five = fmt == ORC_Q5_0, bytes = five ? Q5_0_BYTES : Q4_0_BYTES;
        for (int64_t b = 0; b < K / 32; ++b) {
            const uint8_t* blk = row + b * bytes;
            double d = orc_f16_to_f64(rd16(blk));
            for (int j = 0; j < 32; ++j)
                out[b * 32 + j] = d * (double)(five ? q5_0_value(blk, j) - 16 : q4_0_value(blk, j) - 8);
        }
    } else if (fmt == ORC_Q6_K) {
        for (int64_t b = 0; b < K / QK_K; ++b) {
            const uint8_t* blk = row + b * Q6_K_BYTES;
            double d = orc_f16_to_f64(rd16(blk + 208));
            for (int e = 0; e < QK_K; ++e)
                out[b * QK_K + e] = d * (double)(int8_t)blk[192 + e / 16] * (double)(q6k_value(blk, e) - 32);
        }
    }
}

void orc_dequantize(int fmt, const uint8_t* blocks, int64_t rows, int64_t K, double* out)
{
    const int64_t rb = row_bytes(fmt, K);
    for (int64_t r = 0; r < rows; ++r) dequant_row(fmt, blocks + r * rb, K, out + r * K);
}

/* ------------------------------------------------------------- mode (a) -- */

/*
 * y[m][n] = sum_k x[m][k] * w^[n][k] in double, with w^ the exactly
 * dequantized weight; absacc[m][n] = sum_k |x[m][k] * w^[n][k]| (the tolerance
 * base).  This is the plain matmul the pages' Metal and dequantize-all runs
 * agree on up to summation order (page "同一个 GGUF，CPU 和 Metal 生成的文字不一样",
 * section 出处, the -deq comparison).
 */
void orc_matmul_a(int fmt, const uint8_t* w, int64_t N, int64_t K,
                  const float* x, int64_t M, double* y, double* absacc)
{
    const int64_t rb = row_bytes(fmt, K);
#pragma omp parallel
    {
        double* wr = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            dequant_row(fmt, w + n * rb, K, wr);
            for (int64_t m = 0; m < M; ++m) {
                double s = 0.0, a = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double p = (double)x[m * K + k] * wr[k];
                    s += p;
                    a += fabs(p);
                }
                y[m * N + n] = s;
                if (absacc) absacc[m * N + n] = a;
            }
        }
        free(wr);
    }
}

/* ------------------------------------------------------------- mode (b) -- */

/* Q8_0, Q4_0 and Q5_0 weights take Q8_0 activations, K-quants Q8K (page
 * "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处). */
static int act_format(int wfmt)
{
    return (wfmt == ORC_Q8_0 || wfmt == ORC_Q4_0 || wfmt == ORC_Q5_0) ? ORC_Q8_0 : ORC_Q8_K;
}

static void quantize_act(int wfmt, const float* x, int64_t M, int64_t K, uint8_t* xq)
{
    if (act_format(wfmt) == ORC_Q8_0) orc_quantize_q8_0(x, M, K, xq);
    else orc_quantize_q8k(x, M, K, xq);
}

/* Signed integer weight value of element j of a 32-value block (Q8_0, Q4_0, Q5_0). */
static int int_weight32(int fmt, const uint8_t* blk, int j)
{
    if (fmt == ORC_Q8_0) return (int8_t)blk[2 + j];
    if (fmt == ORC_Q4_0) return q4_0_value(blk, j) - 8;
    return q5_0_value(blk, j) - 16;
}

static int64_t weight_block_bytes(int fmt)
{
    return fmt == ORC_Q8_0 ? Q8_0_BYTES : fmt == ORC_Q4_0 ? Q4_0_BYTES : fmt == ORC_Q5_0 ? Q5_0_BYTES
         : fmt == ORC_Q4_K ? Q4_K_BYTES : Q6_K_BYTES;
}

/*
 * Integer block sums of one weight row against one quantized activation row.
 * Q8_0, Q4_0, Q5_0: S[b] = sum_{j<32} qw*qx with qw the signed weight value
 * (q - 8 for Q4_0, q - 16 for Q5_0).  Q4_K: per super-block i, 10 values:
 * S_0..S_7 (per 32), sumi = sum_j sc_j*S_j, summins = sum_j m_j*(bsums[2j]+bsums[2j+1]).
 * Q6_K: per super-block 17 values: S_0..S_15 (per 16, weights q - 32) and
 * sumi = sum_j sc_j*S_j.
 */
static void row_block_sums(int fmt, const uint8_t* wrow, const uint8_t* xrow, int64_t K, int64_t* out)
{
    if (fmt == ORC_Q8_0 || fmt == ORC_Q4_0 || fmt == ORC_Q5_0) {
        const int64_t wb = weight_block_bytes(fmt);
        for (int64_t b = 0; b < K / Q8_0_QK; ++b) {
            const uint8_t* blk = wrow + b * wb;
            const int8_t* qx = (const int8_t*)(xrow + b * Q8_0_BYTES + 2);
            int64_t s = 0;
            for (int j = 0; j < Q8_0_QK; ++j) s += (int64_t)int_weight32(fmt, blk, j) * qx[j];
            out[b] = s;
        }
    } else if (fmt == ORC_Q6_K) {
        for (int64_t i = 0; i < K / QK_K; ++i) {
            const uint8_t* wb = wrow + i * Q6_K_BYTES;
            const int8_t* q8 = (const int8_t*)(xrow + i * Q8_K_BYTES + 4);
            int64_t* o = out + i * 17;
            int64_t sumi = 0;
            for (int j = 0; j < 16; ++j) {
                int64_t s = 0;
                for (int l = 0; l < 16; ++l) s += (int64_t)(q6k_value(wb, 16 * j + l) - 32) * q8[16 * j + l];
                o[j] = s;
                sumi += (int64_t)(int8_t)wb[192 + j] * s;
            }
            o[16] = sumi;
        }
    } else {
        for (int64_t i = 0; i < K / QK_K; ++i) {
            const uint8_t* wb = wrow + i * Q4_K_BYTES;
            const uint8_t* xb = xrow + i * Q8_K_BYTES;
            const int8_t* q8 = (const int8_t*)(xb + 4);
            int64_t* o = out + i * 10;
            int64_t sumi = 0, summins = 0;
            for (int j = 0; j < 8; ++j) {
                int sc, m;
                q4k_scale_min(wb + 4, j, &sc, &m);
                int64_t s = 0;
                for (int l = 0; l < 32; ++l) s += (int64_t)q4k_nibble(wb + 16, 32 * j + l) * q8[32 * j + l];
                o[j] = s;
                sumi += (int64_t)sc * s;
                int16_t b0 = (int16_t)rd16(xb + 260 + 2 * (2 * j));
                int16_t b1 = (int16_t)rd16(xb + 260 + 2 * (2 * j + 1));
                summins += (int64_t)m * ((int64_t)b0 + b1);
            }
            o[8] = sumi;
            o[9] = summins;
        }
    }
}

static int64_t sums_per_row(int fmt, int64_t K)
{
    if (fmt == ORC_Q8_0 || fmt == ORC_Q4_0 || fmt == ORC_Q5_0) return K / Q8_0_QK;
    return (K / QK_K) * (fmt == ORC_Q6_K ? 17 : 10);
}

int64_t orc_sums_per_row(int fmt, int64_t K) { return sums_per_row(fmt, K); }

/* sums[(m*N + n)*sums_per_row + t] for every activation row m and weight row n. */
void orc_block_sums(int fmt, const uint8_t* w, int64_t N, int64_t K,
                    const float* x, int64_t M, int64_t* sums)
{
    const int afmt = act_format(fmt);
    const int64_t rb = row_bytes(fmt, K), xb = row_bytes(afmt, K), spr = sums_per_row(fmt, K);
    uint8_t* xq = (uint8_t*)malloc((size_t)(M * xb));
    quantize_act(fmt, x, M, K, xq);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m)
            row_block_sums(fmt, w + n * rb, xq + m * xb, K, sums + (m * N + n) * spr);
    free(xq);
}

/*
 * Mode (b): quantize each activation row (Q8_0 with Q8_0, Q4_0 and Q5_0
 * weights, Q8K with K-quant weights), form the integer block sums, then
 *   Q8_0, Q4_0, Q5_0: y = sum_b dw_b * dx_b * S_b
 *   Q4_K: y = sum_i dx_i * (d_i * sumi_i - dmin_i * summins_i)
 *   Q6_K: y = sum_i dx_i * d_i * sumi_i
 * in double.  absacc = sum_k |w^_k * x~_k| with x~ the dequantized quantized
 * activation (the quantities actually multiplied).
 */
void orc_matmul_b(int fmt, const uint8_t* w, int64_t N, int64_t K,
                  const float* x, int64_t M, double* y, double* absacc)
{
    const int afmt = act_format(fmt);
    const int64_t rb = row_bytes(fmt, K), xb = row_bytes(afmt, K), spr = sums_per_row(fmt, K);
    uint8_t* xq = (uint8_t*)malloc((size_t)(M * xb));
    double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
    quantize_act(fmt, x, M, K, xq);
    orc_dequantize(afmt, xq, M, K, xd);
#pragma omp parallel
    {
        int64_t* s = (int64_t*)malloc(sizeof(int64_t) * (size_t)spr);
        double* wr = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* wrow = w + n * rb;
            if (absacc) dequant_row(fmt, wrow, K, wr);
            for (int64_t m = 0; m < M; ++m) {
                const uint8_t* xrow = xq + m * xb;
                row_block_sums(fmt, wrow, xrow, K, s);
                double acc = 0.0;
                if (fmt == ORC_Q8_0 || fmt == ORC_Q4_0 || fmt == ORC_Q5_0) {
                    const int64_t wb = weight_block_bytes(fmt);
                    for (int64_t b = 0; b < K / Q8_0_QK; ++b) {
                        double dw = orc_f16_to_f64(rd16(wrow + b * wb));
                        double dx = orc_f16_to_f64(rd16(xrow + b * Q8_0_BYTES));
                        acc += dw * dx * (double)s[b];
                    }
                } else if (fmt == ORC_Q6_K) {
                    for (int64_t i = 0; i < K / QK_K; ++i) {
                        double d = orc_f16_to_f64(rd16(wrow + i * Q6_K_BYTES + 208));
                        double dx = (double)rdf32(xrow + i * Q8_K_BYTES);
                        acc += dx * d * (double)s[i * 17 + 16];
                    }
                } else {
                    for (int64_t i = 0; i < K / QK_K; ++i) {
                        double d = orc_f16_to_f64(rd16(wrow + i * Q4_K_BYTES));
                        double dmin = orc_f16_to_f64(rd16(wrow + i * Q4_K_BYTES + 2));
                        double dx = (double)rdf32(xrow + i * Q8_K_BYTES);
                        acc += dx * (d * (double)s[i * 10 + 8] - dmin * (double)s[i * 10 + 9]);
                    }
                }
                y[m * N + n] = acc;
                if (absacc) {
                    double a = 0.0;
                    for (int64_t k = 0; k < K; ++k) a += fabs(wr[k] * xd[m * K + k]);
                    absacc[m * N + n] = a;
                }
            }
        }
        free(s);
        free(wr);
    }
    free(xq);
    free(xd);
}

/* ---------------------------------------------------------------- misc -- */

int orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}
