// qmm_gemm.hip -- prefill kernel (M > 8) for y = x . W^T on GGUF blocks on
// the f16 matrix cores: Q8_0 and Q4_K in mode (a), f32 activations (their
// mode (b) runs on the int8 matrix cores, qmm_gemm_q.hip), and Q6_K in both
// modes.
//
// The activation row, scaled by the power of two s that puts its largest
// value in [2^14, 2^15), enters as an exact f16 pair hi + lo of x*s (page
// "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处: the Metal path
// keeps the activations in f32 and dequantizes the weights in the kernel).
// The weights enter as exact f16 integers (Q8_0: q; Q4_K: sc_j*q <= 945).
// Two v_mfma_f32_16x16x32_f16 passes (hi, lo) per 32 values give sum q*x*s;
// the weight scales follow in f32:
//   Q8_0: acc += d * C after every 32-value block;
//   Q4_K: acc += d * C - dmin * Cmin after every super-block, where
//         Cmin = sum_j m_j * (s * sum of x over sub-block j) is one more MFMA
//         whose 32-deep operands hold the eight sub-block sums' hi parts and
//         lo parts against m_j twice.
// y = acc / s.
//
// Q6_K (210 bytes per 256 values: w = d * sc * (q - 32), sc an int8 per 16
// values).  Mode (a): the weights enter as the exact f16 values q - 32 and the
// scale is applied per 16 values: v_mfma_f32_32x32x16_f16 takes one 16-value
// sub-block (K = 16) of a 32 x 32 tile, two of them (hi, lo) give its sum C,
// and acc += (d * sc) * C in f32 (d * sc is exact in f32).  Mode (b) keeps the
// scales in the operand, where sc * (q - 32) reaches 4096 and is not exact in
// f16: each 16-value scale is split as sc = 16 * sc_hi + sc_lo (sc_hi = sc >>
// 4, sc_lo = sc & 15) and the weights enter as two exact f16 operands, 16 *
// sc_hi * (q - 32) (multiples of 16, at most 4096) and sc_lo * (q - 32) (at
// most 480 in magnitude): their products with x sum to x * sc * (q - 32)
// exactly.
// Mode (b) (page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处:
// the activations quantized to Q8K, integer dots, then the scales): the
// activation operand is the int8 values themselves (exact in f16), one pass;
// the two weight operands keep separate accumulators, each an exact integer in
// f32 over a whole super-block (the first a multiple of 16 below 2^27, the
// second below 2^24), so their sum is sumi = sum_j sc_j * S_j of the page's
// integer form; then acc += (d_x * d) * sumi.
//
// A 256-thread workgroup owns a (32*TM) x (32*TN) output tile, four waves in
// 2 x 2, each (16*TM) x (16*TN) as TM x TN MFMA tiles.  K advances 64 values
// per stage through two LDS buffers: while a stage computes, the next stage's
// activation pairs and raw weight bytes are in flight to registers; after the
// compute they are decoded (weights to exact f16) into the other buffer, and
// one barrier per stage hands it over.
#include <map>
#include <mutex>
#include <set>
#include <type_traits>
#include <utility>

#include "qmm_device.h"

namespace qmm {

struct GemmArgs {
    PrefillGroup g;      // the problems: weights, outputs (EMIT instances: may be null), rows
    int64_t row_bytes;
    int K, M;
    int nm;              // row blocks of the output (tiles along M)
    int remap;           // 1: give each XCD a contiguous run of tiles
    const _Float16* hi;  // mode (a): hi part of x*s [M][K]; mode (b): the quantized values as f16 [M][K]
    const _Float16* lo;  // mode (a): lo part
    const float* rs;     // mode (a): 1/s per row
    const _Float16* xs;  // Q4_K: [M][K/256][16] sub-block sums * s / 32, hi then lo
    const float* dx;     // mode (b): activation block scales, block-major [K/256][M]
    int32_t* sums;       // EMIT (Q6_K mode (b)): per super-block 17 values, sumi last (the per-16 sums not formed)
};

// LDS rows hold 64 values (128 bytes) as 8 chunks of 16 bytes; chunk c of row
// r sits in slot c ^ (r & 7), so that the 16-byte MFMA operand reads and the
// 16-byte staging writes hit distinct banks.
constexpr int G_ROW = 128;
QMM_DEV uint32_t swz(int row, int chunk) { return (uint32_t)(row * G_ROW + ((chunk ^ (row & 7)) << 4)); }

// WM x WN waves, each owning TM x TN tiles of 16 x 16 outputs.
template <int FMT, int MODE, int WM, int WN, int TM, int TN>
struct GemmCfg {
    static constexpr int NT = 64 * WM * WN;
    static constexpr int BM = 16 * TM * WM, BN = 16 * TN * WN;
    static constexpr int NA = MODE == MODE_A ? 2 : 1;          // activation operands: hi, lo / the values
    // Q6_K mode (a) runs on 32 x 32 x 16 MFMAs (K = one 16-value sub-block):
    // one weight operand (q - 32) and the sub-block scale d * sc in f32
    static constexpr bool Q6A = FMT == FMT_Q6_K && MODE == MODE_A;
    static constexpr int NB = FMT == FMT_Q6_K && MODE == MODE_B ? 2 : 1;  // weight operands (Q6_K (b): the split scale)
    static constexpr int A_HALF = BM * G_ROW;  // one activation operand of one stage, bytes
    static constexpr int A_BYTES = NA * A_HALF;
    static constexpr int B_PART = BN * G_ROW;  // one weight operand of one stage
    static constexpr int B_BYTES = NB * B_PART;
    static constexpr int OFF_B = 2 * A_BYTES;
    static constexpr int OFF_S = OFF_B + 2 * B_BYTES;
    // Q8_0: block scales [2 stages][2 blocks][BN] f32.
    // Q4_K, by super-block parity: {d, dmin, -, -} [2][BN] (16 B each), 32*m_j
    // [2][BN][8] f16, activation sub-block sums [2][BM][16] f16.
    // Q6_K mode (b), by super-block parity: {d, -, -, -} [2][BN], d_x [2][BM] f32.
    // Q6_K mode (a): d * sc of the stage's four sub-blocks [2 stages][BN][4] f32.
    static constexpr int OFF_DD = OFF_S;
    static constexpr int OFF_MJ = OFF_DD + 2 * BN * 16;
    static constexpr int OFF_X = OFF_MJ + 2 * BN * 16;
    static constexpr int OFF_DXB = OFF_DD + 2 * BN * 16;  // Q6_K mode (b)
    static constexpr int OFF_SC = OFF_S;                  // Q6_K mode (a)
    static constexpr int BYTES = FMT == FMT_Q8_0 ? OFF_S + 2 * 2 * BN * 4
                               : FMT == FMT_Q4_K ? OFF_X + 2 * BM * 32
                               : MODE == MODE_A  ? OFF_SC + 2 * BN * 16
                                                 : OFF_DXB + 2 * BM * 4;
    static constexpr int AU = 8 * NA * BM / NT;        // 16-byte activation chunks per thread per stage
    static constexpr int BU = (2 * BN + NT - 1) / NT;  // weight units (row, half) per thread per stage
    static constexpr int XU = (2 * BM + NT - 1) / NT;  // Q4_K sub-block-sum chunks per thread
    static_assert((8 * BM) % NT == 0, "activation chunks must split evenly between the operands");
    static_assert(MODE == MODE_A || FMT == FMT_Q6_K, "mode (b) of Q8_0 and Q4_K runs on the int8 kernel");
    static_assert(!Q6A || (TM % 2 == 0 && TN % 2 == 0), "32 x 32 tiles");
};

template <int FMT, int MODE, int WM, int WN, int TM, int TN, bool EMIT>
__global__ __launch_bounds__(64 * WM * WN, WM * WN / 4) void gemm_kernel(GemmArgs a)
{
    using C = GemmCfg<FMT, MODE, WM, WN, TM, TN>;
    constexpr int NT = C::NT, BM = C::BM, BN = C::BN, AU = C::AU, BU = C::BU, XU = C::XU;
    constexpr bool Q8 = FMT == FMT_Q8_0, Q6 = FMT == FMT_Q6_K, MB = MODE == MODE_B;
    static_assert(!EMIT || (Q6 && MB), "the traced f16 prefill is Q6_K mode (b)");
    extern __shared__ __align__(16) uint8_t lds[];

    const int M = a.M, K = a.K;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int t = blockIdx.x;
    if (a.remap) {
        const int per = (int)gridDim.x >> 3;
        t = (t & 7) * per + (t >> 3);
    }
    // this tile's problem (grouped launches) and its place in it
    const uint8_t* W;
    float* Y;
    int N, tile0;
    pg_locate(a.g, t / a.nm, W, Y, N, tile0);
    const int m0 = (t % a.nm) * BM, n0 = (t / a.nm - tile0) * BN;
    const int wm = (wave % WM) * 16 * TM, wn = (wave / WM) * 16 * TN;
    const int nst = K / 64;
    const int li = lane & 15, kg = lane >> 4;

    // Resources over this workgroup's rows: loads past the last row return zeros.
    const int64_t rb = a.row_bytes;
    const rsrc_t rhi = make_rsrc(a.hi + (int64_t)m0 * K, clamp_u32((int64_t)(M - m0) * K * 2));
    // (mode (b) has one activation operand: no lo part, an empty resource)
    const rsrc_t rlo = make_rsrc(MB ? a.hi : a.lo + (int64_t)m0 * K, MB ? 0u : clamp_u32((int64_t)(M - m0) * K * 2));
    // Q6_K rows (210 bytes per super-block) may start 2 bytes into a dword: the
    // resource starts at the dword at or below the tile's first row (w0 bytes
    // before it) and ends at the dword holding its last byte (a dword holding a
    // byte of the buffer lies in the buffer's pages)
    const uint32_t w0 = Q6 ? (uint32_t)(((uintptr_t)W + (uint64_t)n0 * rb) & 3u) : 0u;
    const rsrc_t rw = make_rsrc(W + (int64_t)n0 * rb - w0,
                                clamp_u32(Q6 ? ((int64_t)(N - n0) * rb + w0 + 3) & ~3ll : (int64_t)(N - n0) * rb));
    const rsrc_t rx = make_rsrc(FMT != FMT_Q4_K ? a.hi : a.xs + (int64_t)m0 * (K / 256) * 16,
                                clamp_u32((int64_t)(M - m0) * (K / 256) * 32));
    // mode (b): the rows' activation scale of a super-block (block-major, this tile's rows)
    const int drow = tid & (BM - 1);
    auto rdx_of = [&](int sb) { return make_rsrc(a.dx + (int64_t)sb * M + m0, clamp_u32((int64_t)(M - m0) * 4)); };

    // ---- per-thread staging roles, fixed for the whole K loop ----
    // activation chunk idx over [hi, lo][BM rows][8 chunks] (mode b: the values only)
    uint32_t ag[AU], as_[AU];
#pragma unroll
    for (int i = 0; i < AU; ++i) {
        const int idx = (tid + NT * i) % (8 * BM), row = idx >> 3, ch = idx & 7;
        ag[i] = (uint32_t)(row * K * 2 + ch * 16);
        as_[i] = (uint32_t)((i < AU / C::NA ? 0 : C::A_HALF) + swz(row, ch));
    }
    // weight unit (row, half): Q8_0 half = block of the stage, Q4_K half = low
    // or high nibbles (values 0-31 or 32-63 of the stage).  Each unit writes
    // chunks 4*half .. 4*half+3 of its row.  Threads past 2*BN units repeat
    // earlier units (same values to the same places).
    uint32_t bg[BU], bsel[BU], bsh[BU], brow[BU], bst[BU][4];
#pragma unroll
    for (int i = 0; i < BU; ++i) {
        const int u = (tid + NT * i) % (2 * BN), row = u >> 1, sub = u & 1;
        bg[i] = (uint32_t)(Q8 ? row * rb + 32 * sub : w0 + row * rb);
        bsel[i] = sub ? 0x07060504u : 0x05040302u;  // Q8_0: byte selector of the block's values
        bsh[i] = (uint32_t)sub;
        brow[i] = (uint32_t)row;
#pragma unroll
        for (int e = 0; e < 4; ++e) bst[i][e] = swz(row, 4 * sub + e);
    }
    uint32_t xg[XU], xs_[XU];
#pragma unroll
    for (int i = 0; i < XU; ++i) {
        const int u = (tid + NT * i) % (2 * BM);
        xg[i] = (uint32_t)((u >> 1) * (K / 256) * 32 + 16 * (u & 1));
        xs_[i] = (uint32_t)((u >> 1) * 32 + 16 * (u & 1));
    }
    // MFMA operand reads: row wm + 16 i + li (A) or wn + 16 j + li (B), chunk 4 s + kg
    uint32_t afr[2], bfr[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        afr[s] = swz(wm + li, 4 * s + kg);
        bfr[s] = swz(wn + li, 4 * s + kg);
    }

    // ---- staging registers, two sets (stage parity); mode (a) of Q8_0 and Q4_K
    // keeps one set (the next stage is loaded once the current registers are in
    // LDS): fewer registers (Q4_K spilled with two) and measured faster ----
    constexpr bool Q4 = FMT == FMT_Q4_K;
    constexpr bool ONESET = (Q4 || Q8) && !MB;
    constexpr int NSET = ONESET ? 1 : 2;
    uint4 ra[NSET][AU];
    uint32_t rq8[NSET][Q8 ? BU : 1][9];
    uint4 rhd[NSET][Q4 ? BU : 1], rqa[NSET][Q4 ? BU : 1], rqb[NSET][Q4 ? BU : 1];
    uint4 rxv[XU];
    // Q6_K: per unit the 32 bytes of low bits and of high bits and the stage's
    // four scales, each read as whole dwords from the 4-byte-aligned address at
    // or below the field (super-blocks are only 2-byte aligned), and the dword
    // holding d; rsh: the unit's byte offset within those dwords (0 or 2)
    uint32_t rql[2][Q6 ? BU : 1][9], rqh[2][Q6 ? BU : 1][9], rsc[2][Q6 ? BU : 1][2], rdd[2][Q6 ? BU : 1],
        rsh[2][Q6 ? BU : 1];
    float rdxv[2];

    auto load = [&](int st, auto setc, auto csc) {
        constexpr int SET = ONESET ? 0 : decltype(setc)::value;
        constexpr int CS = decltype(csc)::value;  // stage within the super-block (Q4_K)
#pragma unroll
        for (int i = 0; i < AU; ++i)
            ra[SET][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(i < AU / C::NA ? rhi : rlo, ag[i], 128 * st, 0));
        if constexpr (Q8) {
#pragma unroll
            for (int i = 0; i < BU; ++i) {
                const u32x4_t v0 = __builtin_amdgcn_raw_buffer_load_b128(rw, bg[i], 68 * st, 0);
                const u32x4_t v1 = __builtin_amdgcn_raw_buffer_load_b128(rw, bg[i] + 16, 68 * st, 0);
                const uint32_t v2 = __builtin_amdgcn_raw_buffer_load_b32(rw, bg[i] + 32, 68 * st, 0);
#pragma unroll
                for (int k = 0; k < 4; ++k) { rq8[SET][i][k] = v0[k]; rq8[SET][i][4 + k] = v1[k]; }
                rq8[SET][i][8] = v2;
            }
        } else if constexpr (Q6) {
            const int sb = st >> 2;
            auto ld9 = [&](uint32_t off, uint32_t (&r)[9]) {
                const u32x4_t v0 = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
                const u32x4_t v1 = __builtin_amdgcn_raw_buffer_load_b128(rw, off + 16, 0, 0);
#pragma unroll
                for (int k = 0; k < 4; ++k) { r[k] = v0[k]; r[4 + k] = v1[k]; }
                r[8] = __builtin_amdgcn_raw_buffer_load_b32(rw, off + 32, 0, 0);
            };
#pragma unroll
            for (int i = 0; i < BU; ++i) {
                const uint32_t base = bg[i] + 210u * (uint32_t)sb;  // this row's super-block
                const uint32_t sh = base & 3u, al = base - sh;
                rsh[SET][i] = sh;
                ld9(al + 64 * (CS >> 1) + 32 * bsh[i], rql[SET][i]);  // low bits of values 64*CS + 32*half ..
                ld9(al + 128 + 32 * (CS >> 1), rqh[SET][i]);          // their high bits
                rsc[SET][i][0] = __builtin_amdgcn_raw_buffer_load_b32(rw, al + 192 + 4 * CS, 0, 0);
                rsc[SET][i][1] = __builtin_amdgcn_raw_buffer_load_b32(rw, al + 196 + 4 * CS, 0, 0);
                rdd[SET][i] = __builtin_amdgcn_raw_buffer_load_b32(rw, al + 208, 0, 0);
            }
            if constexpr (MB) {
                if (CS == 0 && tid < BM)
                    rdxv[SET] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdx_of(sb), (uint32_t)(4 * drow), 0, 0));
            }
        } else {
            const int sb = st >> 2;
#pragma unroll
            for (int i = 0; i < BU; ++i) {
                rhd[SET][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, bg[i], 144 * sb, 0));
                rqa[SET][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, bg[i] + 16 + 32 * CS, 144 * sb, 0));
                rqb[SET][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, bg[i] + 32 + 32 * CS, 144 * sb, 0));
            }
            if (CS == 0) {
#pragma unroll
                for (int i = 0; i < XU; ++i)
                    rxv[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, xg[i], 32 * sb, 0));
            }
        }
    };

    // ---- staging items: registers of one set -> LDS buffer P ----
    // Items: activation chunks, then per weight unit four 8-value chunks and
    // its scales.  `item` runs one of them; the compute loop spreads them over
    // its MFMA groups.
    constexpr int NI = AU + BU * 5 + (Q4 ? XU : 0) + (Q6 && MB ? 1 : 0);
    half2_t qs_s[BU], qs_b[BU];  // Q4_K: sc and -1024*sc of the unit's sub-block
    auto item = [&](int w, int st, auto setc, auto pc, auto csc) {
        constexpr int SET = ONESET ? 0 : decltype(setc)::value;
        constexpr int P = decltype(pc)::value;
        constexpr int CS = decltype(csc)::value;
        if (w < AU) {
            *reinterpret_cast<uint4*>(lds + P * C::A_BYTES + as_[w]) = ra[SET][w];
            return;
        }
        w -= AU;
        if (w < 5 * BU) {
            const int i = w / 5, e = w % 5;
            uint8_t* bbase = lds + C::OFF_B + P * C::B_BYTES;
            if constexpr (Q8) {
                if (e < 4) {
                    uint32_t h[4];
                    i8x4_to_f16(__builtin_amdgcn_perm(rq8[SET][i][2 * e + 1], rq8[SET][i][2 * e], bsel[i]), h[0], h[1]);
                    i8x4_to_f16(__builtin_amdgcn_perm(rq8[SET][i][2 * e + 2], rq8[SET][i][2 * e + 1], bsel[i]), h[2], h[3]);
                    *reinterpret_cast<uint4*>(bbase + bst[i][e]) = make_uint4(h[0], h[1], h[2], h[3]);
                } else {
                    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(rq8[SET][i][0] >> (16 * bsh[i])));
                    reinterpret_cast<float*>(lds + C::OFF_S)[(P * 2 + bsh[i]) * BN + brow[i]] = d;
                }
            } else if constexpr (Q6) {
                const uint32_t sh = rsh[SET][i];
                if (e < 4) {
                    // values 8e .. 8e+7 of the unit's 32: their low bits are nibble CS & 1 of
                    // bytes 8e .. 8e+7 of the low-bit run, their high bits bit pair
                    // 2 (CS & 1) + half of the same bytes of the high-bit run
                    const uint32_t* ql = rql[SET][i];
                    const uint32_t* qh = rqh[SET][i];
                    const uint32_t l0 = __builtin_amdgcn_alignbyte(ql[2 * e + 1], ql[2 * e], sh);
                    const uint32_t l1 = __builtin_amdgcn_alignbyte(ql[2 * e + 2], ql[2 * e + 1], sh);
                    const uint32_t h0 = __builtin_amdgcn_alignbyte(qh[2 * e + 1], qh[2 * e], sh);
                    const uint32_t h1 = __builtin_amdgcn_alignbyte(qh[2 * e + 2], qh[2 * e + 1], sh);
                    constexpr int LSH = 4 * (CS & 1);
                    const uint32_t hsh = 2 * (2 * (CS & 1) + bsh[i]);
                    const uint32_t c0 = ((l0 >> LSH) & 0x0f0f0f0fu) | (((h0 >> hsh) & 0x03030303u) << 4);
                    const uint32_t c1 = ((l1 >> LSH) & 0x0f0f0f0fu) | (((h1 >> hsh) & 0x03030303u) << 4);
                    // the codes as exact f16 q - 32 (bit pattern 0x64XX is 1024 + XX)
                    const half2_t bias = {(_Float16)-1056.0f, (_Float16)-1056.0f};
                    half2_t v[4];
                    v[0] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c0, 0x05010400u)) + bias;
                    v[1] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c0, 0x07030602u)) + bias;
                    v[2] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c1, 0x05010400u)) + bias;
                    v[3] = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c1, 0x07030602u)) + bias;
                    // their scale, byte 2 half + e/2 of the stage's four
                    const uint32_t scw = __builtin_amdgcn_alignbyte(rsc[SET][i][1], rsc[SET][i][0], sh);
                    const int sc = (int)(int8_t)(scw >> (8 * (2 * bsh[i] + (e >> 1))));
                    if constexpr (!MB) {
                        // mode (a): the values q - 32 as they are, and d * sc (exact in f32) once per sub-block
                        *reinterpret_cast<uint4*>(bbase + bst[i][e]) =
                            make_uint4(__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                                       __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3]));
                        if ((e & 1) == 0) {
                            const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(rdd[SET][i] >> (8 * sh)));
                            reinterpret_cast<float*>(lds + C::OFF_SC)[(P * BN + brow[i]) * 4 + 2 * bsh[i] + (e >> 1)] = d * (float)sc;
                        }
                        return;
                    }
                    // mode (b): split as 16 sc_hi + sc_lo
                    const _Float16 fh = (_Float16)(float)(16 * (sc >> 4)), fl = (_Float16)(float)(sc & 15);
                    const half2_t sh2 = {fh, fh}, sl2 = {fl, fl};
                    uint32_t p0[4], p1[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        p0[k] = __builtin_bit_cast(uint32_t, v[k] * sh2);
                        p1[k] = __builtin_bit_cast(uint32_t, v[k] * sl2);
                    }
                    *reinterpret_cast<uint4*>(bbase + bst[i][e]) = make_uint4(p0[0], p0[1], p0[2], p0[3]);
                    *reinterpret_cast<uint4*>(bbase + C::B_PART + bst[i][e]) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
                } else if (MB && CS == 0 && bsh[i] == 0) {  // mode (b): d of the row's super-block (bytes 208, 209)
                    const int sp = (st >> 2) & 1;
                    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(rdd[SET][i] >> (8 * sh)));
                    reinterpret_cast<float*>(lds + C::OFF_DD)[(sp * BN + brow[i]) * 4] = d;
                }
            } else {
                const uint4 hd = rhd[SET][i];
                if (e == 0) {
                    int sc0, mn0, sc1, mn1;
                    q4k_scale_min(hd.y, hd.z, hd.w, 2 * CS, sc0, mn0);
                    q4k_scale_min(hd.y, hd.z, hd.w, 2 * CS + 1, sc1, mn1);
                    const int sc = bsh[i] ? sc1 : sc0;
                    const _Float16 f = (_Float16)(float)sc, g = (_Float16)(-1024.0f * (float)sc);
                    qs_s[i] = half2_t{f, f};
                    qs_b[i] = half2_t{g, g};
                }
                if (e < 4) {
                    // values 8e .. 8e+7 of the half: bytes 8e .. 8e+7 of the 32 stage bytes
                    const uint32_t d0 = e < 2 ? (e == 0 ? rqa[SET][i].x : rqa[SET][i].z) : (e == 2 ? rqb[SET][i].x : rqb[SET][i].z);
                    const uint32_t d1 = e < 2 ? (e == 0 ? rqa[SET][i].y : rqa[SET][i].w) : (e == 2 ? rqb[SET][i].y : rqb[SET][i].w);
                    const uint32_t n0_ = (d0 >> (4 * bsh[i])) & 0x0f0f0f0fu, n1_ = (d1 >> (4 * bsh[i])) & 0x0f0f0f0fu;
                    uint32_t h[4];
                    h[0] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, n0_, 0x05010400u)), qs_s[i], qs_b[i]));
                    h[1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, n0_, 0x07030602u)), qs_s[i], qs_b[i]));
                    h[2] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, n1_, 0x05010400u)), qs_s[i], qs_b[i]));
                    h[3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, n1_, 0x07030602u)), qs_s[i], qs_b[i]));
                    *reinterpret_cast<uint4*>(bbase + bst[i][e]) = make_uint4(h[0], h[1], h[2], h[3]);
                } else if (CS == 0) {
                    // the (row, 0) unit stores {d, dmin}, the (row, 1) unit the mins 32*m_j
                    const int sp = (st >> 2) & 1;
                    uint32_t mj[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        int s_, ma, mb;
                        q4k_scale_min(hd.y, hd.z, hd.w, 2 * j, s_, ma);
                        q4k_scale_min(hd.y, hd.z, hd.w, 2 * j + 1, s_, mb);
                        mj[j] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)(float)(32 * ma), (_Float16)(float)(32 * mb)});
                    }
                    const uint4 v = bsh[i] ? make_uint4(mj[0], mj[1], mj[2], mj[3])
                                           : make_uint4(__float_as_uint(f16lo(hd.x)), __float_as_uint(f16hi(hd.x)), 0u, 0u);
                    *reinterpret_cast<uint4*>(lds + (bsh[i] ? C::OFF_MJ : C::OFF_DD) + (sp * BN + brow[i]) * 16) = v;
                }
            }
            return;
        }
        w -= 5 * BU;
        if constexpr (Q4) {
            if (CS == 0 && w < XU) {
                const int sp = (st >> 2) & 1;
                *reinterpret_cast<uint4*>(lds + C::OFF_X + sp * BM * 32 + xs_[w]) = rxv[w];
            }
        }
        if constexpr (Q6 && MB) {  // the rows' activation scale of the super-block
            if (CS == 0 && tid < BM) reinterpret_cast<float*>(lds + C::OFF_DXB)[((st >> 2) & 1) * BM + drow] = rdxv[SET];
        }
    };

    // csb: the super-block's sums before its scales (Q4_K, Q6_K); Q6_K mode
    // (b) keeps the second weight operand's sums apart in csb2 (both exact)
    // acc32: Q6_K mode (a), TM/2 x TN/2 tiles of 32 x 32 outputs
    constexpr bool Q6A = C::Q6A;
    constexpr int TM2 = Q6A ? TM / 2 : 1, TN2 = Q6A ? TN / 2 : 1;
    f32x4_t acc[Q6A ? 1 : TM][Q6A ? 1 : TN], csb[Q8 || Q6A ? 1 : TM][Q8 || Q6A ? 1 : TN],
        csb2[Q6 && MB ? TM : 1][Q6 && MB ? TN : 1];
    f32x16_t acc32[TM2][TN2];
    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x16_t zero16 = {};
#pragma unroll
    for (int i = 0; i < (Q6A ? 1 : TM); ++i)
#pragma unroll
        for (int j = 0; j < (Q6A ? 1 : TN); ++j) acc[i][j] = zero;
#pragma unroll
    for (int i = 0; i < TM2; ++i)
#pragma unroll
        for (int j = 0; j < TN2; ++j) acc32[i][j] = zero16;
    const int l32 = lane & 31, hl = lane >> 5;  // 32 x 32 operands: row l32, k-half hl

    // ---- one stage: MFMAs out of buffer P, interleaved with staging stage st+1
    // (register set SET ^ 1) into buffer P ^ 1 when STORE ----
    auto iter = [&](int st, auto pc, auto csc, auto ldc, auto stc) {
        constexpr int P = decltype(pc)::value;
        constexpr int CS = decltype(csc)::value;
        constexpr bool LOAD = decltype(ldc)::value, STORE = decltype(stc)::value;
        using IP = std::integral_constant<int, P>;
        using IQ = std::integral_constant<int, P ^ 1>;
        using ICS1 = std::integral_constant<int, (CS + 1) & 3>;
        using ICS2 = std::integral_constant<int, (CS + 2) & 3>;
        if (LOAD && !ONESET) load(st + 2, IP{}, ICS2{});
        const uint8_t* sa = lds + P * C::A_BYTES;
        const uint8_t* sbb = lds + C::OFF_B + P * C::B_BYTES;
        if constexpr (Q6A) {
            // four 16-value sub-blocks per stage: per 32 x 32 tile two MFMAs (hi, lo)
            // on the exact f16 values q - 32, then acc += (d * sc) * C in f32
            const float* scs = reinterpret_cast<const float*>(lds + C::OFF_SC) + P * BN * 4;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                half8_t ah[TM2], al[TM2];
#pragma unroll
                for (int i = 0; i < TM2; ++i) {
                    const uint32_t o = swz(wm + 32 * i + l32, 2 * u + hl);
                    ah[i] = *reinterpret_cast<const half8_t*>(sa + o);
                    al[i] = *reinterpret_cast<const half8_t*>(sa + C::A_HALF + o);
                }
#pragma unroll
                for (int j = 0; j < TN2; ++j) {
                    const int nl = wn + 32 * j + l32;
                    const half8_t bw = *reinterpret_cast<const half8_t*>(sbb + swz(nl, 2 * u + hl));
                    const float sc = scs[nl * 4 + u];
#pragma unroll
                    for (int i = 0; i < TM2; ++i) {
                        f32x16_t c = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[i], bw, zero16, 0, 0, 0);
                        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[i], bw, c, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc32[i][j][r] = __builtin_fmaf(sc, c[r], acc32[i][j][r]);
                    }
                    if (STORE) {
                        constexpr int R = 4 * TN2;
                        const int rg = u * TN2 + j;
#pragma unroll
                        for (int w = 0; w < NI; ++w)
                            if ((w * R) / NI == rg) item(w, st + 1, IQ{}, IQ{}, ICS1{});
                    }
                }
            }
            __syncthreads();
            return;
        }
        f32x4_t cvp[TM];
        float dwp = 0.0f;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            half8_t ah[TM], al[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                ah[i] = *reinterpret_cast<const half8_t*>(sa + afr[s] + 16 * G_ROW * i);
                if constexpr (!MB) al[i] = *reinterpret_cast<const half8_t*>(sa + C::A_HALF + afr[s] + 16 * G_ROW * i);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const half8_t bw = *reinterpret_cast<const half8_t*>(sbb + bfr[s] + 16 * G_ROW * j);
                if constexpr (Q6) {
                    const half8_t bw1 = *reinterpret_cast<const half8_t*>(sbb + C::B_PART + bfr[s] + 16 * G_ROW * j);
                    const bool first = CS == 0 && s == 0;
                    if constexpr (MB) {
#pragma unroll
                        for (int i = 0; i < TM; ++i) {
                            csb[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], bw, first ? zero : csb[i][j], 0, 0, 0);
                            csb2[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], bw1, first ? zero : csb2[i][j], 0, 0, 0);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < TM; ++i)
                            csb[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], bw, first ? zero : csb[i][j], 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < TM; ++i) csb[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], bw1, csb[i][j], 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < TM; ++i) csb[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[i], bw, csb[i][j], 0, 0, 0);
#pragma unroll
                        for (int i = 0; i < TM; ++i) csb[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[i], bw1, csb[i][j], 0, 0, 0);
                    }
                } else if constexpr (Q8) {
                    const float dw = reinterpret_cast<const float*>(lds + C::OFF_S)[(P * 2 + s) * BN + wn + 16 * j + li];
                    f32x4_t cv[TM];
#pragma unroll
                    for (int i = 0; i < TM; ++i) cv[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[i], bw, zero, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < TM; ++i) cv[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[i], bw, cv[i], 0, 0, 0);
                    // scale the previous column while this one is in the matrix cores
                    if (s > 0 || j > 0) {
                        const int jp = j > 0 ? j - 1 : TN - 1;
#pragma unroll
                        for (int i = 0; i < TM; ++i)
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[i][jp][r] = __builtin_fmaf(dwp, cvp[i][r], acc[i][jp][r]);
                    }
#pragma unroll
                    for (int i = 0; i < TM; ++i) cvp[i] = cv[i];
                    dwp = dw;
                } else {
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        csb[Q8 ? 0 : i][Q8 ? 0 : j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            ah[i], bw, (CS == 0 && s == 0) ? zero : csb[Q8 ? 0 : i][Q8 ? 0 : j], 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        csb[Q8 ? 0 : i][Q8 ? 0 : j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            al[i], bw, csb[Q8 ? 0 : i][Q8 ? 0 : j], 0, 0, 0);
                }
                if (STORE) {
                    constexpr int R = 2 * TN;
                    const int rg = s * TN + j;
#pragma unroll
                    for (int w = 0; w < NI; ++w)
                        if ((w * R) / NI == rg) item(w, st + 1, IQ{}, IQ{}, ICS1{});
                }
            }
        }
        if (LOAD && ONESET) load(st + 2, IP{}, ICS2{});  // the registers of stage st + 1 are in LDS
        if constexpr (Q8) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][TN - 1][r] = __builtin_fmaf(dwp, cvp[i][r], acc[i][TN - 1][r]);
        } else if constexpr (Q6) {
            if (CS == 3) {  // the super-block's scales: d (and d_x) times its sums
                const int sp = (st >> 2) & 1;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int nl = wn + 16 * j + li;
                    const float d = reinterpret_cast<const float*>(lds + C::OFF_DD)[(sp * BN + nl) * 4];
#pragma unroll
                    for (int i = 0; i < TM; ++i) {
                        if constexpr (MB) {
                            const f32x4_t dxv = *reinterpret_cast<const f32x4_t*>(
                                reinterpret_cast<const float*>(lds + C::OFF_DXB) + sp * BM + wm + 16 * i + 4 * kg);
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc[i][j][r] = __builtin_fmaf(dxv[r] * d, csb[i][j][r] + csb2[i][j][r], acc[i][j][r]);
                            if constexpr (EMIT) {
                                // sumi of the super-block: both parts are exact integers; the
                                // per-16 sums are not formed here (the scales are in the operand)
                                const int n = n0 + nl, spr = (K / 256) * 17;
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int m = m0 + wm + 16 * i + 4 * kg + r;
                                    if (m < M && n < N) {
                                        int32_t* o = a.sums + ((int64_t)m * N + n) * spr + 17 * (st >> 2);
#pragma unroll
                                        for (int q = 0; q < 16; ++q) o[q] = INT32_MIN;
                                        o[16] = (int32_t)csb[i][j][r] + (int32_t)csb2[i][j][r];
                                    }
                                }
                            }
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(d, csb[i][j][r], acc[i][j][r]);
                        }
                    }
                }
            }
        } else if (CS == 3) {
            const int sp = (st >> 2) & 1;
            const half8_t hz = {};
            half8_t ax[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                ax[i] = kg < 2 ? *reinterpret_cast<const half8_t*>(lds + C::OFF_X + (sp * BM + wm + 16 * i + li) * 32 + 16 * kg) : hz;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int nl = wn + 16 * j + li;
                const half8_t bm = kg < 2 ? *reinterpret_cast<const half8_t*>(lds + C::OFF_MJ + (sp * BN + nl) * 16) : hz;
                const float2 dd = *reinterpret_cast<const float2*>(lds + C::OFF_DD + (sp * BN + nl) * 16);
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const f32x4_t cm = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax[i], bm, zero, 0, 0, 0);
                    const f32x4_t& cs = csb[Q8 ? 0 : i][Q8 ? 0 : j];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[i][j][r] = __builtin_fmaf(-dd.y, cm[r], __builtin_fmaf(dd.x, cs[r], acc[i][j][r]));
                }
            }
        }
        __syncthreads();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using T_ = std::true_type;
    using F_ = std::false_type;

    // prologue: stages 0 and 1 in flight, stage 0 staged into buffer 0 (one register
    // set: stage 1 is loaded once stage 0 is staged)
    load(0, I0{}, I0{});
    if (nst > 1 && !ONESET) load(1, I1{}, I1{});
#pragma unroll
    for (int w = 0; w < NI; ++w) item(w, 0, I0{}, I0{}, I0{});
    if (nst > 1 && ONESET) load(1, I1{}, I1{});
    __syncthreads();

    if constexpr (Q8) {
        int st = 0;
        for (; st + 3 < nst; st += 2) {
            iter(st, I0{}, I0{}, T_{}, T_{});
            iter(st + 1, I1{}, I0{}, T_{}, T_{});
        }
        const int rem = nst - st;
        if (rem == 3) {
            iter(st, I0{}, I0{}, T_{}, T_{});
            iter(st + 1, I1{}, I0{}, F_{}, T_{});
            iter(st + 2, I0{}, I0{}, F_{}, F_{});
        } else if (rem == 2) {
            iter(st, I0{}, I0{}, F_{}, T_{});
            iter(st + 1, I1{}, I0{}, F_{}, F_{});
        } else {
            iter(st, I0{}, I0{}, F_{}, F_{});
        }
    } else {
        const int nsb = nst >> 2;
        for (int sb = 0; sb + 1 < nsb; ++sb) {
            const int st = 4 * sb;
            iter(st, I0{}, I0{}, T_{}, T_{});
            iter(st + 1, I1{}, I1{}, T_{}, T_{});
            iter(st + 2, I0{}, I2{}, T_{}, T_{});
            iter(st + 3, I1{}, I3{}, T_{}, T_{});
        }
        const int st = nst - 4;
        iter(st, I0{}, I0{}, T_{}, T_{});
        iter(st + 1, I1{}, I1{}, T_{}, T_{});
        iter(st + 2, I0{}, I2{}, F_{}, T_{});
        iter(st + 3, I1{}, I3{}, F_{}, F_{});
    }

    if constexpr (Q6A) {  // 32 x 32 tiles: lane l holds rows 8 (r / 4) + 4 (l / 32) + r % 4 of column l % 32
#pragma unroll
        for (int i = 0; i < TM2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * hl + (r & 3);
                if (m >= M) continue;
                const float rsv = a.rs[m];
#pragma unroll
                for (int j = 0; j < TN2; ++j) {
                    const int n = n0 + wn + 32 * j + l32;
                    if (n < N) Y[(int64_t)m * N + n] = acc32[i][j][r] * rsv;
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        float rsv[4];
        int mrow[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            mrow[r] = m0 + wm + 16 * i + 4 * kg + r;
            rsv[r] = MB ? 1.0f : mrow[r] < M ? a.rs[mrow[r]] : 0.0f;
        }
        if (EMIT && !Y) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn + 16 * j + li;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (mrow[r] < M) Y[(int64_t)mrow[r] * N + n] = acc[i][j][r] * rsv[r];
        }
    }
}

// ------------------------------------------------------------ launchers ----

typedef void (*GemmKernel)(GemmArgs);

// Raises a kernel's dynamic LDS limit to what it needs, once per device.
static void allow_lds(const void* k, int bytes)
{
    static std::set<std::pair<int, const void*>> done;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::lock_guard<std::mutex> lock(mu);
    if (!done.insert(std::make_pair(dev, k)).second) return;
    (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    (void)hipGetLastError();
}

static int cu_count()
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

struct GemmTile {
    int wm, wn, tm, tn;
};
// Tile shapes, largest first: 128 x 224 fills 256 compute units exactly on
// 512 x 14336; the smaller ones keep short or narrow problems spread out
// (32 x 64 runs the 576-wide projections at M = 307 in 11 us against 18 us
// with 64 x 128).  128 x 256 (waves 2 x 4, 64 x 64 each) serves the Q6_K mode
// (a) path, whose 32 x 32 tiles need even tile counts: one tile per compute
// unit on 512 x 14336 and one weight unit per thread (208 us against 288 us
// with 128 x 128).
static const GemmTile kTiles[] = {{4, 2, 2, 7}, {4, 2, 2, 4}, {2, 4, 4, 4}, {2, 2, 2, 4}, {2, 2, 2, 2}, {2, 2, 1, 2}};

// The tile whose busiest compute unit does the least work: rounds of tiles
// over the compute units times the tile's area, weighted by its operand
// traffic per output (activation pairs over BN, weight bytes over BM).  Q6_K
// leaves out the widest tile (its three accumulators per output would not fit
// the registers).
static GemmTile pick_tile(int64_t M, int64_t N, int fmt, int mode)
{
    const int64_t cus = cu_count();
    GemmTile best = kTiles[fmt == FMT_Q6_K ? 1 : 0];
    double bc = -1.0;
    for (const GemmTile& t : kTiles) {
        if (fmt == FMT_Q6_K && t.tn == 7) continue;
        if (fmt == FMT_Q6_K && mode == MODE_A && t.tm == 1) continue;  // 32 x 32 tiles
        if (t.wn == 4 && !(fmt == FMT_Q6_K && mode == MODE_A)) continue;  // the 32 x 32 path's wide tile
        const int64_t bm = 16 * t.tm * t.wm, bn = 16 * t.tn * t.wn;
        const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        const double cost = (double)((tiles + cus - 1) / cus) * (double)(bm * bn) * (1.0 + 16.0 / bm + 64.0 / bn);
        if (bc < 0 || cost < bc) {
            bc = cost;
            best = t;
        }
    }
    return best;
}

template <int FMT, int MODE, bool EMIT, int WM, int WN, int TM, int TN>
static hipError_t launch_tile(GemmArgs a, hipStream_t s)
{
    using C = GemmCfg<FMT, MODE, WM, WN, TM, TN>;
    static_assert(C::BYTES <= 160 * 1024, "LDS of a compute unit");
    const int nm = (a.M + C::BM - 1) / C::BM;
    a.g.t0[0] = 0;
    for (int p = 0; p < PG_MAX; ++p)
        a.g.t0[p + 1] = a.g.t0[p] + (p < a.g.groups ? (a.g.n[p] + C::BN - 1) / C::BN : 0);
    const int64_t grid = (int64_t)nm * a.g.t0[a.g.groups];
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    a.nm = nm;
    a.remap = grid % 8 == 0 ? 1 : 0;
    GemmKernel k = gemm_kernel<FMT, MODE, WM, WN, TM, TN, EMIT>;
    allow_lds((const void*)k, C::BYTES);
    void* args[] = {&a};
    return hipLaunchKernel((const void*)k, dim3((unsigned)grid), dim3(C::NT), args, C::BYTES, s);
}

template <int FMT, int MODE, bool EMIT>
static hipError_t launch_fmt(const GemmArgs& a, GemmTile t, hipStream_t s)
{
    if constexpr (FMT != FMT_Q6_K)
        if (t.wm == 4 && t.tn == 7) return launch_tile<FMT, MODE, EMIT, 4, 2, 2, 7>(a, s);
    if constexpr (FMT == FMT_Q6_K && MODE == MODE_A)
        if (t.wn == 4) return launch_tile<FMT, MODE, EMIT, 2, 4, 4, 4>(a, s);
    if (t.wm == 4 && t.tn == 4) return launch_tile<FMT, MODE, EMIT, 4, 2, 2, 4>(a, s);
    if (t.tm == 2 && t.tn == 4) return launch_tile<FMT, MODE, EMIT, 2, 2, 2, 4>(a, s);
    if (t.tm == 2) return launch_tile<FMT, MODE, EMIT, 2, 2, 2, 2>(a, s);
    if constexpr (FMT == FMT_Q6_K && MODE == MODE_A) return hipErrorInvalidValue;  // 32 x 32 tiles only
    else return launch_tile<FMT, MODE, EMIT, 2, 2, 1, 2>(a, s);
}

// count problems sharing K, the mode and the prepared activations b (one
// launch; the same per-output arithmetic as separate launches).
hipError_t launch_gemm_group(int fmt, int mode, int count, const void* const* w, const int64_t* Ns, float* const* y,
                             int64_t K, int64_t M, const GemmBufs& b, hipStream_t s, int32_t* sums)
{
    if (count < 1 || count > PG_MAX || (sums && count != 1)) return hipErrorInvalidValue;
    if (mode == MODE_B && fmt != FMT_Q6_K) return launch_gemm_q_group(fmt, count, w, Ns, y, K, M, b, s, sums);
    if (sums && !(fmt == FMT_Q6_K && mode == MODE_B)) return hipErrorInvalidValue;
    GemmArgs a{};
    int64_t ntot = 0;
    for (int p = 0; p < count; ++p) {
        a.g.w[p] = (const uint8_t*)w[p];
        a.g.y[p] = y[p];
        a.g.n[p] = (int)Ns[p];
        ntot += Ns[p];
    }
    a.g.groups = count;
    a.row_bytes = fmt == FMT_Q8_0 ? (K / 32) * 34 : fmt == FMT_Q4_K ? (K / 256) * 144 : (K / 256) * 210;
    a.K = (int)K;
    a.M = (int)M;
    a.hi = b.a0;
    a.lo = b.a1;
    a.rs = b.rs;
    a.xs = b.xs;
    a.dx = b.sd;
    a.sums = sums;
    const GemmTile t = pick_tile(M, ntot, fmt, mode);
    hipError_t e;
    if (fmt == FMT_Q8_0) e = launch_fmt<FMT_Q8_0, MODE_A, false>(a, t, s);
    else if (fmt == FMT_Q4_K) e = launch_fmt<FMT_Q4_K, MODE_A, false>(a, t, s);
    else if (mode == MODE_A) e = launch_fmt<FMT_Q6_K, MODE_A, false>(a, t, s);
    else e = sums ? launch_fmt<FMT_Q6_K, MODE_B, true>(a, t, s) : launch_fmt<FMT_Q6_K, MODE_B, false>(a, t, s);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

int gemm_group_max() { return PG_MAX; }

hipError_t launch_gemm(int fmt, int mode, const void* w, int64_t N, int64_t K, int64_t M, const GemmBufs& b,
                       float* y, hipStream_t s, int32_t* sums)
{
    return launch_gemm_group(fmt, mode, 1, &w, &N, &y, K, M, b, s, sums);
}

}  // namespace qmm
