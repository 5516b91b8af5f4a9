// qmm_ext.hip -- Q4_0, Q5_0 and Q6_K weights: decode (M <= 8) kernels for both
// numerical forms, their activation preparation, the Q4_0/Q5_0 -> Q8_0
// transcode that lets the prefill take the Q8_0 kernels, dequantize-all and
// the weight quantizers.
//
// Formats (page "自己量化": Q4_0 18 B and Q5_0 22 B per 32 values by the byte
// counts of sections 和下载的 Q8_0 逐字节比 and 大小和误差; Q6_K, which the same
// page names among the downloaded file's tensors, 210 B per 256; field order
// and packing are the public GGUF layout, which the pages do not print):
//   Q4_0  f16 d, 16 B of nibbles (element j < 16 low nibble of byte j, element
//         j + 16 its high nibble); w = d*(q - 8).
//   Q5_0  f16 d, u32 of fifth bits (bit j for element j), 16 B of nibbles as
//         Q4_0; w = d*(q - 16).
//   Q6_K  ql[128], qh[64], int8 scales[16], f16 d; element e of half n = e/128,
//         group g = (e%128)/32, l = e%32: low 4 bits in ql[64n + 32(g&1) + l]
//         (high nibble for g >= 2), high 2 bits = bit pair g of qh[32n + l];
//         w = d*sc[e/16]*(q - 32).
// Mode (b) pairs Q4_0 and Q5_0 with Q8_0 activations and Q6_K with Q8K (page
// "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处).
#include <algorithm>
#include <mutex>
#include <set>
#include <utility>

#include "qmm_act.h"

namespace qmm {

template <int FMT>
struct Ext;
template <>
struct Ext<FMT_Q4_0> {
    static constexpr int BYTES = 18, OFF = 8, UNIT = 64;  // a unit is a 4-byte-aligned pair of blocks
};
template <>
struct Ext<FMT_Q5_0> {
    static constexpr int BYTES = 22, OFF = 16, UNIT = 64;
};
template <>
struct Ext<FMT_Q6_K> {
    static constexpr int BYTES = 210, OFF = 32, UNIT = 32;  // a unit is a 32-value piece of a super-block
};

// sum over a block of (code - off) * x, the codes converted exactly.
template <int NT>
QMM_DEV float dot_codes_f32(const uint32_t* v, const float* x, float off)
{
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int c = 0; c < 4; ++c) s = fmaf((float)((v[t] >> (8 * c)) & 0xffu) - off, x[4 * t + c], s);
    }
    return s;
}

template <int NT>
QMM_DEV int dot_codes_i8(const uint32_t* v, const uint32_t* xq)
{
    int s = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) s = __builtin_amdgcn_sdot4((int)v[t], (int)xq[t], s, false);
    return s;
}

QMM_DEV void load_x(const float* p, int n, float* out)
{
    for (int i = 0; i < n / 4; ++i) {
        const float4 t = reinterpret_cast<const float4*>(p)[i];
        out[4 * i] = t.x; out[4 * i + 1] = t.y; out[4 * i + 2] = t.z; out[4 * i + 3] = t.w;
    }
}

QMM_DEV void load_q(const int8_t* p, uint32_t out[8])
{
    const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// ------------------------------------------------------- decode kernel ----

constexpr int EXT_GROUP_MAX = 4;  // problems per launch of a grouped run

struct ExtArgs {
    // problems sharing K, mode and the activations, their rows end to end:
    // problem p holds rows row0[p] .. row0[p+1]-1 of the N, weights w[p],
    // outputs y[p] [M][row0[p+1]-row0[p]]
    const uint8_t* w[EXT_GROUP_MAX];
    float* y[EXT_GROUP_MAX];
    int row0[EXT_GROUP_MAX + 1];  // N <= 2^30
    int groups;
    int64_t row_bytes;
    const float* x;    // f32 activations [M][K]
    const int8_t* xq;  // mode (b): quantized activations int8 [M][K] (null: quantized in the kernel)
    const float* xd;   //   their scales [M][K/32] (Q8_0) or [M][K/256] (Q8K)
    const int32_t* xs; //   sums of their values [M][K/32] (Q8_0) or [M][K/16] (Q8K bsums)
    int32_t* sums;     // traced runs (HOOK instances, mode (b)): the integer block sums, written beside y
    uint8_t* act;      //   and the canonical quantized activation blocks, where the kernel quantizes them
    int nxblk;         //   activation blocks per row (K/32 or K/256)
    int N, K, M, m0;   // N: rows of all problems; this launch: activation rows m0 + MT*blockIdx.y .. + MT - 1 of M
    int units;         // units per row
    int lpr_log2;      // log2 of the lanes per row
};

// Activations staged in LDS: per activation row, one slot per unit holding
// the unit's values (f32 in mode (a), int8 in mode (b)) plus 16 bytes of
// padding, so that the 16-byte reads of 16 lanes at consecutive units fall in
// distinct banks.
template <int FMT, int MODE>
QMM_DEV constexpr int xl_stride() { return Ext<FMT>::UNIT * (MODE == MODE_A ? 4 : 1) + 16; }

// Rows of activations [mb, mb + rows) as the kernel reads them: from LDS
// (XL) or from global memory.
template <int FMT, int MODE, bool XL>
QMM_DEV const uint8_t* x_unit(const ExtArgs& a, const uint8_t* xl, int m, int mm, int u)
{
    if constexpr (XL) return xl + ((int64_t)m * a.units + u) * xl_stride<FMT, MODE>();
    if constexpr (MODE == MODE_A) return reinterpret_cast<const uint8_t*>(a.x + (int64_t)mm * a.K + Ext<FMT>::UNIT * u);
    return reinterpret_cast<const uint8_t*>(a.xq + (int64_t)mm * a.K + Ext<FMT>::UNIT * u);
}

// The weight bytes of one unit as loaded (raw dwords), then decoded.
template <int FMT>
struct Raw {
    // a 4-byte-aligned pair of blocks
    static constexpr int ND = FMT == FMT_Q4_0 ? 9 : 11;
    uint32_t r[ND];
    QMM_DEV void load(const uint8_t* row, int u)
    {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(row + (int64_t)u * (2 * Ext<FMT>::BYTES));
#pragma unroll
        for (int i = 0; i < ND; ++i) r[i] = q[i];
    }
};
template <>
struct Raw<FMT_Q6_K> {
    // piece pc of super-block i: the dwords under its 32 low-bit bytes and 32
    // high-bit bytes (one more when the super-block starts at 2 mod 4), the
    // dword holding its two scales and the one holding d.  Q6_K super-blocks
    // (210 B) are only 2-byte aligned; every load is a 4-byte-aligned dword
    // that holds at least one byte of the super-block, so no access leaves the
    // pages the weight buffer occupies.
    uint32_t lo[9], hi[9], scw, dw, sh;
    QMM_DEV void load(const uint8_t* row, int u)
    {
        const int i = u >> 3, pc = u & 7, nn = pc >> 2, g = pc & 3;
        const uint8_t* s = row + (int64_t)i * 210;
        sh = (uint32_t)((uintptr_t)s & 3);
        // rounded down by pointer arithmetic (an integer round trip would
        // lose the global address space and give flat loads)
        const uint32_t* pl = reinterpret_cast<const uint32_t*>(s + 64 * nn + 32 * (g & 1) - sh);
        const uint32_t* ph = reinterpret_cast<const uint32_t*>(s + 128 + 32 * nn - sh);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            lo[t] = pl[t];
            hi[t] = ph[t];
        }
        // the ninth dwords: the last two bytes when the super-block starts at
        // 2 mod 4, else the bytes that follow inside the super-block (the
        // high bits after the low bits, the scales after the high bits)
        lo[8] = pl[8];
        hi[8] = ph[8];
        scw = *reinterpret_cast<const uint32_t*>(s + 192 + 2 * pc - ((sh + 2 * pc) & 3));
        dw = *reinterpret_cast<const uint32_t*>(s + 208 - sh);
    }
};

// Codes (0..63, v[t] = elements 4t..4t+3 of the piece), the two sub-block
// scales and d of Q6_K piece pc (values 32pc..32pc+31 of its super-block).
QMM_DEV void q6k_decode(const Raw<FMT_Q6_K>& w, int pc, uint32_t v[8], int& sc0, int& sc1, float& d)
{
    const int g = pc & 3, ls = 4 * (g >> 1), hs = 2 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t l = __builtin_amdgcn_alignbyte(w.lo[t + 1], w.lo[t], w.sh);
        const uint32_t h = __builtin_amdgcn_alignbyte(w.hi[t + 1], w.hi[t], w.sh);
        v[t] = ((l >> ls) & 0x0f0f0f0fu) | (((h >> hs) & 0x03030303u) << 4);
    }
    const uint32_t scb = w.scw >> (8 * ((w.sh + 2 * pc) & 3));
    sc0 = (int)(int8_t)(scb & 0xffu);
    sc1 = (int)(int8_t)((scb >> 8) & 0xffu);
    d = (float)__builtin_bit_cast(_Float16, (uint16_t)((w.dw >> (8 * w.sh)) & 0xffffu));
}

// Codes and scales of a pair of Q4_0 / Q5_0 blocks from its raw dwords.
template <int FMT>
QMM_DEV void pair_decode(const Raw<FMT>& w, uint32_t v[2][8], float d[2])
{
    pair_codes<FMT>(w.r, v, d);
}

// Mode (b) LDS layout after the activation slots of MT rows: the block
// scales [MT][K/32 or K/256] (f32), then the value sums [MT][K/32 or K/16].
template <int FMT, int MODE, int MT>
QMM_DEV int xl_extra_off(const ExtArgs& a) { return MT * a.units * xl_stride<FMT, MODE>(); }
template <int FMT>
QMM_DEV int xd_per_row(int K) { return FMT == FMT_Q6_K ? K / 256 : K / 32; }
template <int FMT>
QMM_DEV int xs_per_row(int K) { return FMT == FMT_Q6_K ? K / 16 : K / 32; }

// The problem of global row n (0 <= n < N) and the row within it: a chain of
// selects over the few problems, no indexed access to the argument arrays.
QMM_DEV int ext_problem(const ExtArgs& a, int n)
{
    int p = 0;
#pragma unroll
    for (int q = 1; q < EXT_GROUP_MAX; ++q) p = (q < a.groups && n >= a.row0[q]) ? q : p;
    return p;
}
template <typename T>
QMM_DEV T ext_pick(T const (&arr)[EXT_GROUP_MAX], int p)
{
    T v = arr[0];
#pragma unroll
    for (int q = 1; q < EXT_GROUP_MAX; ++q) v = p == q ? arr[q] : v;
    return v;
}
QMM_DEV int ext_row0(const ExtArgs& a, int p)  // 0 <= p <= groups
{
    int v = a.row0[0];
#pragma unroll
    for (int q = 1; q <= EXT_GROUP_MAX; ++q) v = p == q ? a.row0[q] : v;
    return v;
}

// The arithmetic of one unit u of row n against activation rows mb ..
// mb + mrows - 1: into acc, or (block-sums hook) into a.sums.
template <int FMT, int MODE, int MT, bool XL, bool HOOK>
QMM_DEV void unit_math(const ExtArgs& a, const uint8_t* xl, const Raw<FMT>& w, int u, int64_t n, int mb, int mrows,
                       int spr, float acc[MT])
{
    using F = Ext<FMT>;
    auto xl_scales = [&](const ExtArgs& aa, const uint8_t* p) {
        return reinterpret_cast<const float*>(p + xl_extra_off<FMT, MODE, MT>(aa));
    };
    auto xl_sums = [&](const ExtArgs& aa, const uint8_t* p) {
        return reinterpret_cast<const int32_t*>(p + xl_extra_off<FMT, MODE, MT>(aa)) + MT * xd_per_row<FMT>(aa.K);
    };
    if constexpr (FMT == FMT_Q6_K) {
        const int i = u >> 3, pc = u & 7;
        uint32_t v[8];
        int sc0, sc1;
        float d;
        q6k_decode(w, pc, v, sc0, sc1, d);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (MT > 1 && m >= mrows) break;  // a one-row instance always has its row
            const int mm = mb + m;
            const uint8_t* xp = x_unit<FMT, MODE, XL>(a, xl, m, mm, u);
            if constexpr (MODE == MODE_A) {
                float x[32];
                load_x(reinterpret_cast<const float*>(xp), 32, x);
                const float s0 = dot_codes_f32<4>(v, x, 32.0f);
                const float s1 = dot_codes_f32<4>(v + 4, x + 16, 32.0f);
                acc[m] = fmaf(d, (float)sc0 * s0 + (float)sc1 * s1, acc[m]);
                if (MT > 1) asm volatile("" ::: "memory");  // one row's activations live at a time
            } else {
                uint32_t xq[8];
                load_q(reinterpret_cast<const int8_t*>(xp), xq);
                const int32_t* bs = (XL ? xl_sums(a, xl) + (int64_t)m * (a.K / 16) : a.xs + (int64_t)mm * (a.K / 16)) + 2 * u;
                const int S0 = dot_codes_i8<4>(v, xq) - 32 * bs[0];
                const int S1 = dot_codes_i8<4>(v + 4, xq + 4) - 32 * bs[1];
                const int part = sc0 * S0 + sc1 * S1;
                if constexpr (HOOK) {
                    int32_t* o = a.sums + ((int64_t)mm * a.N + n) * spr + 17 * i;
                    o[2 * pc] = S0;
                    o[2 * pc + 1] = S1;
                    int t = part;  // sumi: the eight pieces of the super-block are lanes 8k..8k+7
                    t += __shfl_xor(t, 1);
                    t += __shfl_xor(t, 2);
                    t += __shfl_xor(t, 4);
                    if (pc == 0) o[16] = t;
                }
                const float dx = XL ? xl_scales(a, xl)[(int64_t)m * (a.K / 256) + i] : a.xd[(int64_t)mm * (a.K / 256) + i];
                acc[m] = fmaf(d * dx, (float)part, acc[m]);
            }
        }
    } else {
        uint32_t v[2][8];
        float d[2];
        pair_decode<FMT>(w, v, d);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (MT > 1 && m >= mrows) break;  // a one-row instance always has its row
            const int mm = mb + m;
            const uint8_t* xp = x_unit<FMT, MODE, XL>(a, xl, m, mm, u);
            if constexpr (MODE == MODE_A) {
                float x[32];
                load_x(reinterpret_cast<const float*>(xp), 32, x);
                const float s0 = dot_codes_f32<8>(v[0], x, (float)F::OFF);
                load_x(reinterpret_cast<const float*>(xp) + 32, 32, x);
                const float s1 = dot_codes_f32<8>(v[1], x, (float)F::OFF);
                acc[m] = fmaf(d[0], s0, fmaf(d[1], s1, acc[m]));
                if (MT > 1) asm volatile("" ::: "memory");  // one row's activations live at a time
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int b = 2 * u + h;
                    uint32_t xq[8];
                    load_q(reinterpret_cast<const int8_t*>(xp) + 32 * h, xq);
                    const int32_t sx = XL ? xl_sums(a, xl)[(int64_t)m * (a.K / 32) + b] : a.xs[(int64_t)mm * (a.K / 32) + b];
                    const int S = dot_codes_i8<8>(v[h], xq) - F::OFF * sx;
                    if constexpr (HOOK) a.sums[((int64_t)mm * a.N + n) * spr + b] = S;
                    const float dx = XL ? xl_scales(a, xl)[(int64_t)m * (a.K / 32) + b] : a.xd[(int64_t)mm * (a.K / 32) + b];
                    acc[m] = fmaf(d[h] * dx, (float)S, acc[m]);
                }
            }
        }
    }
}

// Each wave takes 64/L rows at a time (L = lanes per row, a power of two
// covering the row's units up to 64) and strides over the row groups; each
// lane walks units lane, lane + L, ... of its row, and the row sums meet by
// butterfly inside the L lanes.  Activation rows mb .. mb + MT - 1, staged in
// LDS once per workgroup when XL.  HOOK (mode (b), the traced run): the same
// run, which also writes the integer block sums it forms and, where it
// quantizes the activations itself, those blocks; y may then be null.
constexpr int EXT_WAVES = 8, EXT_THREADS = 64 * EXT_WAVES;  // decode workgroup: eight waves share the staged activations

template <int FMT, int MODE, int MT, bool XL, bool HOOK, bool GRP>
__global__ __launch_bounds__(EXT_THREADS) void ext_gemv_kernel(ExtArgs a)
{
    using F = Ext<FMT>;
    extern __shared__ __align__(16) uint8_t xl[];
    const int lane = threadIdx.x & 63;
    const int L = 1 << a.lpr_log2;
    const int sub = lane & (L - 1);
    const int spr = FMT == FMT_Q6_K ? (a.K / 256) * 17 : a.K / 32;  // block sums per (m, n)
    const int mb = a.m0 + (int)blockIdx.y * MT;                       // first activation row here
    const int mrows = min(MT, a.M - mb);

    if constexpr (XL && MODE == MODE_A) {
        // f32 activations copied into their slots
        constexpr int ub = F::UNIT * 4, st = xl_stride<FMT, MODE>();
        const int per_row = a.units * (ub / 16);
        for (int c = threadIdx.x; c < mrows * per_row; c += EXT_THREADS) {
            const int m = c / per_row, cc = c % per_row;
            const int u = cc / (ub / 16), w = cc % (ub / 16);
            const float4 t = *reinterpret_cast<const float4*>(a.x + (int64_t)(mb + m) * a.K + 4 * (int64_t)cc);
            *reinterpret_cast<float4*>(xl + ((int64_t)m * a.units + u) * st + 16 * w) = t;
        }
        __syncthreads();
    }
    if constexpr (XL && MODE == MODE_B) {
        constexpr int st = xl_stride<FMT, MODE>();
        const int nd = xd_per_row<FMT>(a.K);
        float* ld = reinterpret_cast<float*>(xl + xl_extra_off<FMT, MODE, MT>(a));
        int32_t* ls = reinterpret_cast<int32_t*>(ld + MT * nd);
        if (a.xq) {
            // quantized by the separate launch: copied into their slots
            constexpr int ub = F::UNIT;
            const int per_row = a.units * (ub / 16), ns = xs_per_row<FMT>(a.K);
            for (int c = threadIdx.x; c < mrows * per_row; c += EXT_THREADS) {
                const int m = c / per_row, cc = c % per_row;
                const int u = cc / (ub / 16), w = cc % (ub / 16);
                const uint4 t = *reinterpret_cast<const uint4*>(a.xq + (int64_t)(mb + m) * a.K + 16 * (int64_t)cc);
                *reinterpret_cast<uint4*>(xl + ((int64_t)m * a.units + u) * st + 16 * w) = t;
            }
            for (int c = threadIdx.x; c < mrows * nd; c += EXT_THREADS) ld[c] = a.xd[(int64_t)mb * nd + c];
            for (int c = threadIdx.x; c < mrows * ns; c += EXT_THREADS) ls[c] = a.xs[(int64_t)mb * ns + c];
        } else if constexpr (FMT == FMT_Q6_K) {
            // quantized here, with the arithmetic of the standalone quantizer
            // (so bit-identical to it).  Q8K: one wave per 256 values.
            // Q8K: one wave per 256 values, four per lane
            const int lane_ = threadIdx.x & 63, nsb = a.K / 256;
            for (int blk = threadIdx.x >> 6; blk < mrows * nsb; blk += EXT_WAVES) {
                const int m = blk / nsb, sb = blk % nsb;
                const float4 xv = reinterpret_cast<const float4*>(a.x + (int64_t)(mb + m) * a.K + 256 * sb)[lane_];
                const float v[4] = {xv.x, xv.y, xv.z, xv.w};
                float d;
                int q[4], s16;
                q8k_wave(v, lane_, d, q, s16);
                if (HOOK && a.act && blockIdx.x == 0)
                    store_q8k_lane(a.act + ((int64_t)(mb + m) * a.nxblk + sb) * 292, lane_, d, q, s16);
                const int u = 8 * sb + (lane_ >> 3);  // the 32-value unit of elements 4*lane..4*lane+3
                *reinterpret_cast<uint32_t*>(xl + ((int64_t)m * a.units + u) * st + 4 * (lane_ & 7)) =
                    pack4(q[0], q[1], q[2], q[3]);
                if (lane_ == 0) ld[m * nd + sb] = d;
                if ((lane_ & 3) == 0) ls[m * (a.K / 16) + 16 * sb + (lane_ >> 2)] = s16;
            }
        } else {
            // quantized here; Q8_0: one thread per 32 values
            for (int blk = threadIdx.x; blk < mrows * nd; blk += EXT_THREADS) {
                const int m = blk / nd, b = blk % nd;
                float v[32];
                load32(a.x + (int64_t)(mb + m) * a.K + 32 * b, v);
                uint16_t dbits;
                float dval;
                int8_t q[32];
                q8_0_block(v, dbits, dval, q);
                if (HOOK && a.act && blockIdx.x == 0) store_q8_0_block(a.act + ((int64_t)(mb + m) * a.nxblk + b) * 34, dbits, q);
                int sum = 0;
#pragma unroll
                for (int j = 0; j < 32; ++j) sum += q[j];
                uint4* o = reinterpret_cast<uint4*>(xl + ((int64_t)m * a.units + (b >> 1)) * st + 32 * (b & 1));
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    o[i] = make_uint4(pack4(q[16 * i], q[16 * i + 1], q[16 * i + 2], q[16 * i + 3]),
                                      pack4(q[16 * i + 4], q[16 * i + 5], q[16 * i + 6], q[16 * i + 7]),
                                      pack4(q[16 * i + 8], q[16 * i + 9], q[16 * i + 10], q[16 * i + 11]),
                                      pack4(q[16 * i + 12], q[16 * i + 13], q[16 * i + 14], q[16 * i + 15]));
                ld[m * nd + b] = dval;
                ls[m * nd + b] = sum;
            }
        }
        __syncthreads();
    }

    const int rpw = 64 >> a.lpr_log2;
    const int64_t groups = ((int64_t)a.N + rpw - 1) / rpw;
    for (int64_t g = (int64_t)blockIdx.x * EXT_WAVES + (threadIdx.x >> 6); g < groups; g += (int64_t)gridDim.x * EXT_WAVES) {
        const int64_t n = g * rpw + (lane >> a.lpr_log2);
        const bool live = n < a.N;
        // GRP: the row's problem (a single-problem launch skips the lookup)
        const int p = GRP ? ext_problem(a, live ? (int)n : 0) : 0;
        const int ln = (live ? (int)n : 0) - (GRP ? ext_row0(a, p) : 0);  // row within its problem
        const uint8_t* row = (GRP ? ext_pick(a.w, p) : a.w[0]) + (int64_t)ln * a.row_bytes;

        float acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
        Raw<FMT> r;
#pragma unroll 1
        for (int u = sub; live && u < a.units; u += L) {
            r.load(row, u);
            unit_math<FMT, MODE, MT, XL, HOOK>(a, xl, r, u, n, mb, mrows, spr, acc);
        }
        if (HOOK && a.y[0] == nullptr) continue;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float t = acc[m];
            for (int off = L >> 1; off > 0; off >>= 1) t += __shfl_xor(t, off);
            if (live && sub == 0 && m < mrows) {
                if constexpr (GRP) ext_pick(a.y, p)[(int64_t)(mb + m) * (ext_row0(a, p + 1) - ext_row0(a, p)) + ln] = t;
                else a.y[0][(int64_t)(mb + m) * a.N + ln] = t;
            }
        }
    }
}

// ------------------------------------------- mode (b) activation prep ------

// Q8_0 activations for Q4_0 / Q5_0 weights, one thread per 32 values: the
// values int8 [M][K], the f16-rounded scale [M][K/32] and the sum of the
// values [M][K/32] (which carries the weight offset).
__global__ __launch_bounds__(256) void ext_prep_q8_0_kernel(const float* __restrict__ x, int M, int K,
                                                            int8_t* __restrict__ xq, float* __restrict__ xd,
                                                            int32_t* __restrict__ xs, uint8_t* __restrict__ act)
{
    const int nb = K / 32;
    const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (blk >= (int64_t)M * nb) return;
    const int m = (int)(blk / nb), b = (int)(blk % nb);
    float v[32];
    load32(x + (int64_t)m * K + 32 * b, v);
    uint16_t dbits;
    float dval;
    int8_t q[32];
    q8_0_block(v, dbits, dval, q);
    if (act) store_q8_0_block(act + blk * 34, dbits, q);  // traced runs
    int s = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) s += q[j];
    uint4* o = reinterpret_cast<uint4*>(xq + (int64_t)m * K + 32 * b);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        o[i] = make_uint4(pack4(q[16 * i], q[16 * i + 1], q[16 * i + 2], q[16 * i + 3]),
                          pack4(q[16 * i + 4], q[16 * i + 5], q[16 * i + 6], q[16 * i + 7]),
                          pack4(q[16 * i + 8], q[16 * i + 9], q[16 * i + 10], q[16 * i + 11]),
                          pack4(q[16 * i + 12], q[16 * i + 13], q[16 * i + 14], q[16 * i + 15]));
    xd[blk] = dval;
    xs[blk] = s;
}

// Q8K activations for Q6_K weights, one wave per 256 values: int8 [M][K],
// d [M][K/256], bsums [M][K/16].
__global__ __launch_bounds__(256) void ext_prep_q8k_kernel(const float* __restrict__ x, int M, int K,
                                                           int8_t* __restrict__ xq, float* __restrict__ xd,
                                                           int32_t* __restrict__ xs, uint8_t* __restrict__ act)
{
    const int nsb = K / 256;
    const int lane = threadIdx.x & 63;
    const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= (int64_t)M * nsb) return;  // the whole wave leaves together
    const int m = (int)(blk / nsb), sb = (int)(blk % nsb);
    const float4 xv = reinterpret_cast<const float4*>(x + (int64_t)m * K + 256 * sb)[lane];
    const float v[4] = {xv.x, xv.y, xv.z, xv.w};
    float d;
    int q[4], s16;
    q8k_wave(v, lane, d, q, s16);
    if (act) store_q8k_lane(act + blk * 292, lane, d, q, s16);  // traced runs
    *reinterpret_cast<uint32_t*>(xq + (int64_t)m * K + 256 * sb + 4 * lane) = pack4(q[0], q[1], q[2], q[3]);
    if (lane == 0) xd[blk] = d;
    if ((lane & 3) == 0) xs[blk * 16 + (lane >> 2)] = s16;
}

// --------------------------------------------------- Q4_0/Q5_0 -> Q8_0 -----

// One thread per block: Q8_0 block with the same d and q' = q - offset, whose
// dequantized values d*q' equal the source's exactly (the prefill then runs
// the Q8_0 kernels, whose block sums are the same integers).
template <int FMT>
__global__ __launch_bounds__(256) void ext_to_q8_0_kernel(const uint8_t* __restrict__ w, int64_t blocks,
                                                          uint8_t* __restrict__ out)
{
    using F = Ext<FMT>;
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= blocks) return;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(w + b * F::BYTES);
    uint32_t qs[4], qh = 0;
    const int qo = FMT == FMT_Q5_0 ? 3 : 1;  // u16 index of the nibbles
#pragma unroll
    for (int t = 0; t < 4; ++t) qs[t] = (uint32_t)src[qo + 2 * t] | ((uint32_t)src[qo + 2 * t + 1] << 16);
    if (FMT == FMT_Q5_0) qh = (uint32_t)src[1] | ((uint32_t)src[2] << 16);
    uint32_t v[8];
    block_codes<FMT>(qs, qh, v);
    uint16_t* o = reinterpret_cast<uint16_t*>(out + b * 34);
    o[0] = src[0];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        // bytes minus the offset (no borrow: each byte is >= 0 before and the
        // result is taken per byte)
        uint32_t r = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) r |= (uint32_t)(uint8_t)((int)((v[t] >> (8 * c)) & 0xffu) - F::OFF) << (8 * c);
        o[1 + 2 * t] = (uint16_t)(r & 0xffffu);
        o[2 + 2 * t] = (uint16_t)(r >> 16);
    }
}

// ------------------------------------------------------- dequantize -------

// One thread per 32 values: f32 [N][K], each value d*(q - 8), d*(q - 16) or
// (d*sc)*(q - 32) rounded once (d*sc is exact in f32).
template <int FMT>
__global__ __launch_bounds__(256) void ext_dequant_kernel(const uint8_t* __restrict__ w, int64_t N, int K,
                                                          int64_t row_bytes, float* __restrict__ out)
{
    const int n32 = K / 32;
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= N * n32) return;
    const int64_t n = u / n32;
    const int p = (int)(u % n32);
    const uint8_t* row = w + n * row_bytes;
    float val[32];
    Raw<FMT> raw;
    if constexpr (FMT == FMT_Q6_K) {
        uint32_t v[8];
        int sc0, sc1;
        float d;
        raw.load(row, p);
        q6k_decode(raw, p & 7, v, sc0, sc1, d);
        const float e0 = d * (float)sc0, e1 = d * (float)sc1;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                val[4 * t + c] = (t < 4 ? e0 : e1) * ((float)((v[t] >> (8 * c)) & 0xffu) - 32.0f);
    } else {
        using F = Ext<FMT>;
        uint32_t v[2][8];
        float d[2];
        raw.load(row, p >> 1);
        pair_decode<FMT>(raw, v, d);
        const int h = p & 1;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c) val[4 * t + c] = d[h] * ((float)((v[h][t] >> (8 * c)) & 0xffu) - (float)F::OFF);
    }
    float4* o = reinterpret_cast<float4*>(out + n * K + 32 * p);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = make_float4(val[4 * i], val[4 * i + 1], val[4 * i + 2], val[4 * i + 3]);
}

// ------------------------------------------------- weight quantizers ------

// The value itself, hidden from the optimizer: keeps max * (-1/8) and its
// f16 conversion two roundings (the compiler would otherwise fuse them into one
// mixed-precision fma with a +0 addend, which turns the -0 scale of an
// all-zero block into +0).
QMM_DEV float opaque(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Q4_0 / Q5_0, one thread per 32 values (the pages name QTensor::quantize to
// Q4_0 and its Q5_0 fallback, page "自己量化", section 3. 量化, not the rule):
// the signed element of largest |x| (first index on ties) takes the most
// negative code, d = max / -offset, q = floor(x*(1/d) + offset + 1/2) capped
// at 2*offset - 1, d stored as f16.
template <int FMT>
__global__ __launch_bounds__(256) void ext_quantize_q4_q5_kernel(const float* __restrict__ w, int64_t blocks,
                                                                 uint8_t* __restrict__ out)
{
#pragma clang fp contract(off)
    using F = Ext<FMT>;
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= blocks) return;
    float v[32];
    load32(w + b * 32, v);
    float amax = 0.0f, mx = 0.0f;
    for (int j = 0; j < 32; ++j) {
        const float t = fabsf(v[j]);
        if (t > amax) { amax = t; mx = v[j]; }
    }
    const float d = mx / -(float)F::OFF;
    const float id = d != 0.0f ? 1.0f / d : 0.0f;
    uint32_t qs[4] = {0u, 0u, 0u, 0u}, qh = 0u;
    for (int j = 0; j < 32; ++j) {
        float t = v[j] * id;
        t = t + ((float)F::OFF + 0.5f);
        int q = (int)t;
        q = q > 2 * F::OFF - 1 ? 2 * F::OFF - 1 : q;
        const int byte = j & 15;
        qs[byte >> 2] |= (uint32_t)(q & 15) << (8 * (byte & 3) + (j < 16 ? 0 : 4));
        qh |= (uint32_t)((q >> 4) & 1) << j;
    }
    uint16_t* o = reinterpret_cast<uint16_t*>(out + b * F::BYTES);
    o[0] = f16bits(opaque(d));
    int at = 1;
    if (FMT == FMT_Q5_0) {
        o[1] = (uint16_t)(qh & 0xffffu);
        o[2] = (uint16_t)(qh >> 16);
        at = 3;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        o[at + 2 * t] = (uint16_t)(qs[t] & 0xffffu);
        o[at + 2 * t + 1] = (uint16_t)(qs[t] >> 16);
    }
}

// Q6_K, one thread per 256 values (no quantizer is described on the pages):
// per 16 values s_j = (signed max) / -32; d = (signed s_j of largest |s_j|) /
// -128; sc_j = min(127, round(s_j / d)); q = clamp(round(x / (d*sc_j)), -32,
// 31) + 32 against the stored f16 d (q = 32 where d*sc_j is 0).
__global__ __launch_bounds__(256) void ext_quantize_q6_k_kernel(const float* __restrict__ w, int64_t blocks,
                                                                uint8_t* __restrict__ out)
{
#pragma clang fp contract(off)
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= blocks) return;
    const float* v = w + b * 256;
    float s[16];
    float smx = 0.0f, sam = 0.0f;
    for (int j = 0; j < 16; ++j) {
        float am = 0.0f, mx = 0.0f;
        for (int l = 0; l < 16; ++l) {
            const float t = fabsf(v[16 * j + l]);
            if (t > am) { am = t; mx = v[16 * j + l]; }
        }
        s[j] = mx / -32.0f;
        if (fabsf(s[j]) > sam) { sam = fabsf(s[j]); smx = s[j]; }
    }
    const float d = smx / -128.0f;
    const uint16_t dh = f16bits(opaque(d));
    const float dq = (float)__builtin_bit_cast(_Float16, dh);
    uint32_t word[53];
    for (int i = 0; i < 53; ++i) word[i] = 0u;
    int sc[16];
    for (int j = 0; j < 16; ++j) {
        const int c = d != 0.0f ? (int)roundf(s[j] / d) : 0;
        sc[j] = c > 127 ? 127 : c;
        word[(192 + j) >> 2] |= (uint32_t)(uint8_t)(int8_t)sc[j] << (8 * ((192 + j) & 3));
    }
    word[52] |= (uint32_t)dh;  // bytes 208..209
    for (int e = 0; e < 256; ++e) {
        const float de = dq * (float)sc[e >> 4];
        int q = 0;
        if (de != 0.0f) {
            q = (int)roundf(v[e] / de);
            q = q < -32 ? -32 : (q > 31 ? 31 : q);
        }
        q += 32;
        const int half = e >> 7, el = e & 127, g = el >> 5, l = el & 31;
        const int lb = 64 * half + 32 * (g & 1) + l, hb = 128 + 32 * half + l;
        word[lb >> 2] |= (uint32_t)((q & 15) << (4 * (g >> 1))) << (8 * (lb & 3));
        word[hb >> 2] |= (uint32_t)((q >> 4) << (2 * g)) << (8 * (hb & 3));
    }
    uint16_t* o = reinterpret_cast<uint16_t*>(out + b * 210);
    for (int i = 0; i < 105; ++i) o[i] = (uint16_t)(word[i >> 1] >> (16 * (i & 1)));
}

// ----------------------------------------------------------- launchers ----

static unsigned ext_blocks(int64_t items, int per) { return (unsigned)((items + per - 1) / per); }

bool is_ext_format(int fmt) { return fmt == FMT_Q4_0 || fmt == FMT_Q5_0 || fmt == FMT_Q6_K; }

int64_t ext_block_bytes(int fmt) { return fmt == FMT_Q4_0 ? 18 : fmt == FMT_Q5_0 ? 22 : 210; }

constexpr int EXT_XL_MAX = 160 * 1024;  // LDS of a compute unit; above it the kernel reads activations from global memory

// Dynamic LDS above the default 64 KB: the kernel's limit raised once per
// device (host-side, before any capture of a run).
static void ext_allow_lds(const void* kernel)
{
    static std::set<std::pair<int, const void*>> done;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (done.insert(std::make_pair(dev, kernel)).second) {
        (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, EXT_XL_MAX);
        (void)hipGetLastError();
    }
}

template <int FMT, int MODE, int MT, bool HOOK, bool GRP>
static void launch_staged(const ExtArgs& a, dim3 grid, dim3 block, int lds, hipStream_t s)
{
    if (lds > 64 * 1024) ext_allow_lds(reinterpret_cast<const void*>(&ext_gemv_kernel<FMT, MODE, MT, true, HOOK, GRP>));
    hipLaunchKernelGGL((ext_gemv_kernel<FMT, MODE, MT, true, HOOK, GRP>), grid, block, lds, s, a);
}

// Grouped launches (a.groups > 1) always stage their activations (the host
// groups only runs that do).
template <int FMT, int MODE, int MT>
static void launch_one(bool xl, const ExtArgs& a, unsigned gx, unsigned gy, int lds, hipStream_t s)
{
    const dim3 grid(gx, gy), block(EXT_THREADS);
    if constexpr (MODE == MODE_B) {
        if (a.sums) {  // the traced run: the same staging choice as the plain run
            if (xl) launch_staged<FMT, MODE, MT, true, false>(a, grid, block, lds, s);
            else hipLaunchKernelGGL((ext_gemv_kernel<FMT, MODE, MT, false, true, false>), grid, block, 0, s, a);
            return;
        }
    }
    if (a.groups > 1) launch_staged<FMT, MODE, MT, false, true>(a, grid, block, lds, s);
    else if (xl) launch_staged<FMT, MODE, MT, false, false>(a, grid, block, lds, s);
    else hipLaunchKernelGGL((ext_gemv_kernel<FMT, MODE, MT, false, false, false>), grid, block, 0, s, a);
}

template <int FMT, int MODE>
static void launch_mt(int mt, bool xl, const ExtArgs& a, unsigned gx, unsigned gy, int lds, hipStream_t s)
{
    if (mt == 1) {
        launch_one<FMT, MODE, 1>(xl, a, gx, gy, lds, s);
        return;
    }
    if constexpr (MODE == MODE_B) {
        if (mt == 2) return launch_one<FMT, MODE, 2>(xl, a, gx, gy, lds, s);
        if (mt == 4) return launch_one<FMT, MODE, 4>(xl, a, gx, gy, lds, s);
    }
    launch_one<FMT, MODE, 8>(xl, a, gx, gy, lds, s);
}

// LDS bytes of the staged activations: MT rows of units * stride, and in
// mode (b) the rows' block scales and value sums.
static int ext_xl_bytes(int fmt, int mode, int units, int K, int mt)
{
    const int unit = fmt == FMT_Q6_K ? 32 : 64;
    int bytes = mt * units * (unit * (mode == MODE_A ? 4 : 1) + 16);
    if (mode == MODE_B) bytes += 4 * mt * (fmt == FMT_Q6_K ? K / 256 + K / 16 : 2 * (K / 32));
    return bytes;
}

// Activation rows per launch row: mode (a) keeps the one- and eight-row
// instances (the two- and four-row ones hold every decoded value and
// activation at once and need over 200 registers).
static int ext_mt(int mode, int M) { return M == 1 ? 1 : mode == MODE_A ? 8 : M == 2 ? 2 : M <= 4 ? 4 : 8; }

// Whether a run stages its activations in LDS (and, in mode (b), quantizes
// them there): unless they exceed the LDS.
static bool ext_staged(int fmt, int mode, int units, int K, int mt)
{
    return ext_xl_bytes(fmt, mode, units, K, mt) <= EXT_XL_MAX;
}

// The decode kernel over activation rows m0.. in one launch per 65535 * MT rows.
static hipError_t ext_gemv(int fmt, int mode, ExtArgs a, hipStream_t s)
{
    const int mt = ext_mt(mode, a.M);
    const int lds = ext_xl_bytes(fmt, mode, a.units, a.K, mt);
    const bool xl = ext_staged(fmt, mode, a.units, a.K, mt);
    int lg = 0;
    while ((1 << lg) < a.units && lg < 6) ++lg;
    a.lpr_log2 = lg;
    // workgroups: enough to cover the row groups once, at most what the
    // compute units hold at once by LDS (so that each workgroup's staged
    // activations serve several rows)
    const int64_t groups = ((int64_t)a.N + (64 >> lg) - 1) / (64 >> lg);
    const int slot = mt * a.units * ((fmt == FMT_Q6_K ? 32 : 64) * (mode == MODE_A ? 4 : 1) + 16);
    const int per_cu = xl ? std::max(1, std::min(4, (160 * 1024) / slot)) : 4;
    const int64_t cap = (int64_t)device_cus() * per_cu;
    const unsigned gx = (unsigned)std::min<int64_t>((groups + EXT_WAVES - 1) / EXT_WAVES, cap);
    const int64_t chunk = 65535ll * mt;
    for (int64_t m0 = 0; m0 < a.M; m0 += chunk) {
        a.m0 = (int)m0;
        const unsigned gy = (unsigned)std::min<int64_t>(65535, (a.M - m0 + mt - 1) / mt);
        if (fmt == FMT_Q4_0) {
            if (mode == MODE_A) launch_mt<FMT_Q4_0, MODE_A>(mt, xl, a, gx, gy, lds, s);
            else launch_mt<FMT_Q4_0, MODE_B>(mt, xl, a, gx, gy, lds, s);
        } else if (fmt == FMT_Q5_0) {
            if (mode == MODE_A) launch_mt<FMT_Q5_0, MODE_A>(mt, xl, a, gx, gy, lds, s);
            else launch_mt<FMT_Q5_0, MODE_B>(mt, xl, a, gx, gy, lds, s);
        } else {
            if (mode == MODE_A) launch_mt<FMT_Q6_K, MODE_A>(mt, xl, a, gx, gy, lds, s);
            else launch_mt<FMT_Q6_K, MODE_B>(mt, xl, a, gx, gy, lds, s);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_ext_prep(int fmt, const float* x, int64_t M, int64_t K, const ExtBufs& b, hipStream_t s,
                           uint8_t* act)
{
    if (fmt == FMT_Q6_K)
        hipLaunchKernelGGL(ext_prep_q8k_kernel, dim3(ext_blocks(M * (K / 256), 4)), dim3(256), 0, s, x, (int)M, (int)K,
                           b.xq, b.xd, b.xs, act);
    else
        hipLaunchKernelGGL(ext_prep_q8_0_kernel, dim3(ext_blocks(M * (K / 32), 256)), dim3(256), 0, s, x, (int)M,
                           (int)K, b.xq, b.xd, b.xs, act);
    return hipGetLastError();
}

hipError_t launch_ext_run(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, int64_t M,
                          const ExtBufs& b, float* y, hipStream_t s, const Trace* tr)
{
    if (tr && mode != MODE_B) return hipErrorInvalidValue;
    // mode (b) with one or two activation rows staged in LDS quantizes them
    // inside the decode kernel (a.xq null); otherwise a separate launch
    // writes them to the workspace first (with more rows every workgroup
    // quantizing them all costs more than that launch)
    ExtArgs a{};
    a.w[0] = (const uint8_t*)w;
    a.y[0] = y;
    a.row0[0] = 0;
    for (int p = 1; p <= EXT_GROUP_MAX; ++p) a.row0[p] = (int)N;
    a.groups = 1;
    a.row_bytes = fmt == FMT_Q6_K ? (K / 256) * 210 : (K / 32) * ext_block_bytes(fmt);
    a.x = x;
    a.xq = b.xq;
    a.xd = b.xd;
    a.xs = b.xs;
    a.sums = tr ? tr->sums : nullptr;
    a.act = tr ? tr->act : nullptr;
    a.nxblk = fmt == FMT_Q6_K ? (int)(K / 256) : (int)(K / 32);
    a.N = (int)N;
    a.K = (int)K;
    a.M = (int)M;
    a.units = fmt == FMT_Q6_K ? (int)(K / 32) : (int)(K / 64);
    if (mode == MODE_B) {
        const int mt = ext_mt(mode, (int)M);
        if (mt <= 2 && ext_staged(fmt, mode, a.units, (int)K, mt)) {
            a.xq = nullptr;
        } else {
            const hipError_t e = launch_ext_prep(fmt, x, M, K, b, s, a.act);
            if (e != hipSuccess) return e;
        }
    }
    return ext_gemv(fmt, mode, a, s);
}

int ext_group_max() { return EXT_GROUP_MAX; }

bool ext_group_supported(int fmt, int mode, int64_t K, int64_t M)
{
    if (mode != MODE_A && mode != MODE_B) return false;
    if (M < 1 || M > GEMV_MAX_M) return false;
    const int units = fmt == FMT_Q6_K ? (int)(K / 32) : (int)(K / 64);
    return ext_staged(fmt, mode, units, (int)K, ext_mt(mode, (int)M));
}

// Up to EXT_GROUP_MAX problems sharing K, mode and x in one launch (their
// rows end to end); each row's arithmetic is that of a separate run.  b: the
// workspace of the first problem's plan (the activations are shared).
hipError_t launch_ext_group(int fmt, int mode, int count, const void* const* w, const int64_t* Ns, float* const* y,
                            const float* x, int64_t K, int64_t M, const ExtBufs& b, hipStream_t s)
{
    ExtArgs a{};
    int64_t rows = 0;
    for (int p = 0; p < count; ++p) {
        a.w[p] = (const uint8_t*)w[p];
        a.y[p] = y[p];
        a.row0[p] = (int)rows;
        rows += Ns[p];
    }
    for (int p = count; p <= EXT_GROUP_MAX; ++p) a.row0[p] = (int)rows;
    for (int p = count; p < EXT_GROUP_MAX; ++p) {
        a.w[p] = a.w[0];
        a.y[p] = a.y[0];
    }
    a.groups = count;
    a.row_bytes = fmt == FMT_Q6_K ? (K / 256) * 210 : (K / 32) * ext_block_bytes(fmt);
    a.x = x;
    a.xq = b.xq;
    a.xd = b.xd;
    a.xs = b.xs;
    a.sums = nullptr;
    a.N = (int)rows;
    a.K = (int)K;
    a.M = (int)M;
    a.units = fmt == FMT_Q6_K ? (int)(K / 32) : (int)(K / 64);
    if (mode == MODE_B) {
        const int mt = ext_mt(mode, (int)M);
        if (mt <= 2 && ext_staged(fmt, mode, a.units, (int)K, mt)) {
            a.xq = nullptr;
        } else {
            const hipError_t e = launch_ext_prep(fmt, x, M, K, b, s, nullptr);
            if (e != hipSuccess) return e;
        }
    }
    return ext_gemv(fmt, mode, a, s);
}

hipError_t launch_ext_to_q8_0(int fmt, const void* w, int64_t N, int64_t K, void* out, hipStream_t s)
{
    const int64_t blocks = N * (K / 32);
    if (fmt == FMT_Q4_0)
        hipLaunchKernelGGL(ext_to_q8_0_kernel<FMT_Q4_0>, dim3(ext_blocks(blocks, 256)), dim3(256), 0, s,
                           (const uint8_t*)w, blocks, (uint8_t*)out);
    else
        hipLaunchKernelGGL(ext_to_q8_0_kernel<FMT_Q5_0>, dim3(ext_blocks(blocks, 256)), dim3(256), 0, s,
                           (const uint8_t*)w, blocks, (uint8_t*)out);
    return hipGetLastError();
}

// Q4_0 / Q5_0 rows with an odd number of blocks (2-byte aligned blocks): one
// thread per block, bytes read one at a time; w = d * (q - offset) exactly.
template <int FMT>
__global__ __launch_bounds__(256) void ext_dequant_block_kernel(const uint8_t* __restrict__ w, int64_t blocks,
                                                                float* __restrict__ out)
{
    constexpr int BB = FMT == FMT_Q4_0 ? 18 : 22, OFF = FMT == FMT_Q4_0 ? 8 : 16;
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= blocks) return;
    const uint8_t* p = w + b * BB;
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(p[0] | (p[1] << 8)));
    uint32_t qh = 0;
    if constexpr (FMT == FMT_Q5_0) qh = p[2] | (p[3] << 8) | (p[4] << 16) | ((uint32_t)p[5] << 24);
    const uint8_t* qs = p + BB - 16;
    float v[32];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        int lo = qs[j] & 15, hi = qs[j] >> 4;
        if constexpr (FMT == FMT_Q5_0) {
            lo |= ((qh >> j) & 1) << 4;
            hi |= ((qh >> (j + 16)) & 1) << 4;
        }
        v[j] = d * (float)(lo - OFF);
        v[j + 16] = d * (float)(hi - OFF);
    }
    float* o = out + 32 * b;
#pragma unroll
    for (int j = 0; j < 32; ++j) o[j] = v[j];
}

hipError_t launch_ext_dequantize(int fmt, const void* w, int64_t N, int64_t K, float* out, hipStream_t s)
{
    const unsigned grid = ext_blocks(N * (K / 32), 256);
    const int64_t rb = fmt == FMT_Q6_K ? (K / 256) * 210 : (K / 32) * ext_block_bytes(fmt);
    if (fmt != FMT_Q6_K && K % 64) {  // odd block count: block by block
        if (fmt == FMT_Q4_0)
            hipLaunchKernelGGL(ext_dequant_block_kernel<FMT_Q4_0>, dim3(grid), dim3(256), 0, s, (const uint8_t*)w,
                               N * (K / 32), out);
        else
            hipLaunchKernelGGL(ext_dequant_block_kernel<FMT_Q5_0>, dim3(grid), dim3(256), 0, s, (const uint8_t*)w,
                               N * (K / 32), out);
        return hipGetLastError();
    }
    if (fmt == FMT_Q4_0)
        hipLaunchKernelGGL(ext_dequant_kernel<FMT_Q4_0>, dim3(grid), dim3(256), 0, s, (const uint8_t*)w, N, (int)K, rb, out);
    else if (fmt == FMT_Q5_0)
        hipLaunchKernelGGL(ext_dequant_kernel<FMT_Q5_0>, dim3(grid), dim3(256), 0, s, (const uint8_t*)w, N, (int)K, rb, out);
    else
        hipLaunchKernelGGL(ext_dequant_kernel<FMT_Q6_K>, dim3(grid), dim3(256), 0, s, (const uint8_t*)w, N, (int)K, rb, out);
    return hipGetLastError();
}

hipError_t launch_ext_quantize_weights(int fmt, const float* w, int64_t N, int64_t K, void* out, hipStream_t s)
{
    if (fmt == FMT_Q6_K) {
        const int64_t blocks = N * (K / 256);
        hipLaunchKernelGGL(ext_quantize_q6_k_kernel, dim3(ext_blocks(blocks, 256)), dim3(256), 0, s, w, blocks,
                           (uint8_t*)out);
    } else {
        const int64_t blocks = N * (K / 32);
        if (fmt == FMT_Q4_0)
            hipLaunchKernelGGL(ext_quantize_q4_q5_kernel<FMT_Q4_0>, dim3(ext_blocks(blocks, 256)), dim3(256), 0, s, w,
                               blocks, (uint8_t*)out);
        else
            hipLaunchKernelGGL(ext_quantize_q4_q5_kernel<FMT_Q5_0>, dim3(ext_blocks(blocks, 256)), dim3(256), 0, s, w,
                               blocks, (uint8_t*)out);
    }
    return hipGetLastError();
}

}  // namespace qmm
