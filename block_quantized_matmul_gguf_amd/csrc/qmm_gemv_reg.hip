// qmm_gemv_reg.hip -- decode with two to eight activation rows for Q8_0, Q4_K,
// Q4_0, Q5_0 and Q6_K weights (mode (a); mode (b) for Q4_0, Q5_0 and Q6_K),
// the activation operand held in registers.
//
// The pages' decode step streams every weight once per token (page "同一个
// GGUF，CPU 和 Metal 生成的文字不一样", section 修法: the CPU decode is bound by
// the weight bytes), so the weights must keep HBM busy from the start.  The
// tile kernel (qmm_gemv_kernel.h) builds the activation operand of the whole
// K range in LDS (f16 hi and lo of eight rows: 128 KB at K = 4096), which
// leaves room for only two shallow weight stages per wave.  Here K is split
// eight ways instead, one slice per wave of a 512-thread workgroup, and each
// wave keeps its slice's operand in registers (64 VGPRs at K = 4096):
//   * a workgroup owns a run of 16-row tiles; for each tile every wave
//     streams its K slice of the 16 rows through a ring of D stage buffers in
//     LDS filled by 16-byte buffer-to-LDS loads (D stages in flight, the whole
//     LDS but the tile partials available to the ring);
//   * the activation values of the slice are loaded first (lane quads kept
//     inside one row, then moved to the operand lanes), their row maxima
//     taken (the power-of-two scale 2^e of a row is per wave and slice: each
//     wave scales its partial sums back by 2^-e, exactly), then the ring is
//     primed and the values are split into f16 hi and lo while it fills;
//   * v_mfma_f32_16x16x32_f16 with A rows 0..7 = hi and 8..15 = lo of the
//     eight activation rows and the weights as exact f16 integers (Q8_0 q;
//     Q4_K q; Q4_0 q - 8; Q5_0 q - 16; Q6_K sh (q - 32) and sl (q - 32) for
//     its per-16 scale sc = 16 sh + sl), the block scales applied in f32 after
//     each block (Q4_K's mins term from the sub-block sums of x*2^e; Q6_K's d
//     once per super-block);
//   * at the end of a tile the eight slices' partial sums meet in LDS behind
//     one barrier and are added in slice order (deterministic).
// Operand lanes n and n + 8 of a 16-lane row need the same eight x values
// (hi for rows 0..7, lo for rows 8..15): each loads four, splits them, and the
// pair trades the half the other needs with one DPP row rotation.
//
// Mode (b) (page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处: the
// activation rows quantized to Q8_0 for the 32-value formats, to Q8K for Q6_K):
// each wave quantizes the blocks of its slice in registers with the standalone
// quantizer's device functions (a 32-value block sits in eight lanes, whose
// maximum meets in three lane exchanges; a Q8K block in the same eight lanes
// over eight steps, the first element of largest magnitude found with its
// index), A rows 0..7 take the int8 values as exact f16 (rows 8..15 zero), so
// the matrix core's f32 sums are exact integers: S per block, Q6_K's two
// scale-split sums per super-block (sumi = 16 Ch + Cl); acc += S (d_w d_x).
// The traced instances also write the integer parts and the quantized
// activation blocks (Q6_K's per-16 sums from two more matrix-core steps).
#include <mutex>
#include <set>
#include <type_traits>
#include <utility>

#include "qmm_gemv_kernel.h"
#include "qmm_internal.h"

namespace qmm {

struct GemvRegArgs {
    const uint8_t* w;
    int64_t w_bytes;  // N * row_bytes
    int row_bytes;
    int N, K, M;
    int nlu;    // load units per row (block pairs of the 32-value formats, Q4_K super-blocks, Q6_K super-block pairs)
    int tiles;  // 16-row tiles
    int T;      // tiles per workgroup
    const float* x;
    float* y;        // may be null in a traced run
    int32_t* sums;   // traced mode (b): [M][N][K/32] integer block sums
    uint8_t* act;    // traced mode (b): the quantized activations as canonical Q8_0 blocks [M][K/32], or null
};

constexpr int GR_PART_BYTES = 2 * GV_WAVES * 128 * 4;  // tile partials, two slots: [slot][wave][8 rows][16]

// Bytes of a load unit: a block pair of the 32-value formats and a super-block
// pair of Q6_K (pairs keep every unit 4-byte aligned), a Q4_K super-block.
constexpr int gr_lub(int fmt)
{
    return fmt == FMT_Q8_0 ? 68 : fmt == FMT_Q4_0 ? 36 : fmt == FMT_Q5_0 ? 44 : fmt == FMT_Q6_K ? 420 : 144;
}
// Values of a load unit.
constexpr int gr_vpl(int fmt) { return fmt == FMT_Q4_K ? 256 : fmt == FMT_Q6_K ? 512 : 64; }

// U: load units per wave slice (K <= 8 U units), P: units per stage, D: ring depth.
template <int FMT, int MODE, int U, int P, int D>
struct GrCfg {
    static constexpr int LUB = gr_lub(FMT);
    static constexpr int STEPS = gr_vpl(FMT) / 32;           // matrix-core steps (32 values) per unit
    static constexpr int CPR = (LUB * P + 15) / 16;         // 16-byte chunks per row and stage
    static constexpr int SBY = 16 * 16 * CPR;               // one stage buffer (16 rows, unpadded)
    static constexpr int TL = (16 * CPR + 63) / 64;         // load instructions per stage
    static constexpr int SUMS = FMT == FMT_Q4_K ? U * 8 * 8 * 4 : 0;  // per wave: x*2^e sums [U*8 sub-blocks][8 rows]
    // per wave, mode (b): d_x [block][8 rows]; Q8_0 blocks also 1/d [row][block] and the f16 bits of d
    static constexpr int DXB = MODE == MODE_B ? U * STEPS * 8 * (FMT == FMT_Q6_K ? 4 : 10) : 0;
    static constexpr int OFF_PART = GV_WAVES * D * SBY;
    static constexpr int OFF_SUMS = OFF_PART + GR_PART_BYTES;
    static constexpr int OFF_DX = OFF_SUMS + GV_WAVES * SUMS;
    static constexpr int LDS = OFF_DX + GV_WAVES * DXB;
    static_assert(MODE == MODE_A || FMT == FMT_Q8_0 || FMT == FMT_Q4_0 || FMT == FMT_Q5_0 || FMT == FMT_Q6_K,
                  "mode (b) here: the formats with Q8_0 activations, and Q6_K");
    // an odd chunk count puts the 16 rows of a stage in different LDS banks
    static_assert(U % P == 0 && (CPR & 1) == 1 && D >= 2 && (D - 1) * TL <= 63, "ring of LDS-direct stages");
    static_assert(LDS <= GV_LDS_MAX, "LDS of a compute unit");
};

// DPP row_ror:8 -- lane n of a 16-lane row receives lane (n + 8) % 16.
QMM_DEV uint32_t ror8(uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xF, 0xF, false); }
QMM_DEV uint32_t pack_h2(_Float16 a, _Float16 b) { return __builtin_bit_cast(uint32_t, half2_t{a, b}); }

// Eight unsigned codes (bytes of d0, d1, each below 64) -> eight exact f16
// (code - OFF) in order: byte b under 0x64 is the f16 1024 + b, then one packed
// subtraction of 1024 + OFF.
template <int OFF>
QMM_DEV half8_t u8x8_to_f16(uint32_t d0, uint32_t d1)
{
    const half2_t bias = {(_Float16)(-1024.0f - OFF), (_Float16)(-1024.0f - OFF)};
    const half2_t h0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, d0, 0x04010400u)) + bias;
    const half2_t h1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, d0, 0x04030402u)) + bias;
    const half2_t h2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, d1, 0x04010400u)) + bias;
    const half2_t h3 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, d1, 0x04030402u)) + bias;
    half8_t r;
    r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
    r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
    return r;
}

template <int FMT, int MODE, int U, int P, int D, bool EMIT>
__global__ __launch_bounds__(GV_THREADS, 2) void gemv_reg_kernel(GemvRegArgs a)
{
    static_assert(!EMIT || MODE == MODE_B, "integer block sums exist in mode (b) only");
    using C = GrCfg<FMT, MODE, U, P, D>;
    constexpr int LUB = C::LUB, STEPS = C::STEPS, CPR = C::CPR, SBY = C::SBY, TL = C::TL;
    constexpr int S = U / P;  // stages per tile
    static_assert(S == 1 || S == 2, "one or two stages per tile");
    constexpr int VPL = gr_vpl(FMT);
    extern __shared__ __align__(16) uint8_t lds[];

    const int M = a.M, N = a.N, K = a.K;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int r8 = n & 7;         // the activation row of this lane's operand values
    const bool upper = n >= 8;    // operand rows 8..15 (lo); loads values 4..7 of its k-group
    const int t0 = blockIdx.x * a.T;
    const int nt = min(a.T, a.tiles - t0);  // tiles of this workgroup, >= 1
    const int u0 = wave * U;                // first unit of this wave's slice
    const int ureal = max(0, min(U, a.nlu - u0));
    const int sreal = (ureal + P - 1) / P;  // stages of a tile holding real units
    const int Q = nt * S;                   // stages per wave
    uint8_t* ring = lds + wave * (D * SBY);
    float* part = reinterpret_cast<float*>(lds + C::OFF_PART);
    float* sums = reinterpret_cast<float*>(lds + C::OFF_SUMS + wave * C::SUMS);
    float* dxs = reinterpret_cast<float*>(lds + C::OFF_DX + wave * C::DXB);

    // ---- the weight stream: chunk f = 64t + lane of a stage is row f/CPR, chunk f%CPR ----
    uint32_t go[TL];
#pragma unroll
    for (int t = 0; t < TL; ++t) {
        const int f = 64 * t + lane, r = f / CPR, c = f - r * CPR;
        go[t] = f < 16 * CPR ? (uint32_t)(r * a.row_bytes + 16 * c) : 0x80000000u;
    }
    constexpr int TAIL = 16 * CPR - 64 * (TL - 1);  // live lanes of the last load
    int iq = 0;  // next stage to issue
    // stage iq into ring buffer `slot`: the tile's rows as a buffer (rows past N, and
    // stages without real units, read as zero); lanes past the last chunk stay off
    auto issue = [&](int slot) {
        const int tile = t0 + iq / S, s = iq % S;
        const bool real = s < sreal;
        const int64_t tb = (int64_t)tile * 16 * a.row_bytes;
        const int64_t left = a.w_bytes - tb;
        const uint32_t nrec = real && left > 0 ? (uint32_t)min(left, (int64_t)16 * a.row_bytes) : 0u;
        const rsrc_t wr = make_rsrc(a.w + (real ? tb : 0), nrec);
        const uint32_t so = (uint32_t)((u0 + s * P) * LUB);
        uint8_t* buf = ring + slot * SBY;
#pragma unroll
        for (int t = 0; t < TL; ++t)
            if (t < TL - 1 || lane < TAIL) ld128_lds(wr, buf + 1024 * t, go[t] + so);
        ++iq;
    };

    // ---- the activation values of this wave's slice, four per lane and step ----
    // k-group g holds the block's values 8g .. 8g+7 (the even block of a pair, whose
    // weight bytes start two bytes into a dword, is realigned when gathered).
    // Operand lanes n < 8 take the first four, n >= 8 the last four.  They are
    // loaded with each lane quad inside one row (lane l: row l / 8, values
    // 4 (l % 8) .. +3 of the step; quads that span rows took the 128 KB of a
    // workgroup about 2 us longer to arrive) and moved to the operand lanes with
    // one ds_bpermute per dword.  Units past the slice's real ones and rows past
    // M read as zero.  Every wave's activation loads are issued before any
    // weight load of the workgroup, then the first stage follows.
    const rsrc_t xr = make_rsrc(a.x, clamp_u32((int64_t)M * K * 4));
    u32x4_t xt[U * STEPS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool live = u < ureal;
#pragma unroll
        for (int p = 0; p < STEPS; ++p)
            xt[u * STEPS + p] = ld128(xr, live ? (uint32_t)((lane >> 3) * K + (u0 + u) * VPL + 32 * p + 4 * (lane & 7)) * 4
                                               : 0x80000000u);
    }
    __builtin_amdgcn_s_barrier();
    issue(0);  // the first stage flies while the activations arrive
    const int src4 = 4 * (r8 * 8 + 2 * g + (upper ? 1 : 0));  // the load lane holding this lane's four values
    float xv[U * STEPS][4];
#pragma unroll
    for (int i = 0; i < U * STEPS; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) xv[i][e] = __int_as_float(__builtin_amdgcn_ds_bpermute(src4, (int)xt[i][e]));
    // mode (a): the row maximum over the slice; mode (b): each block's maximum |x|
    // (lanes n, n + 8 of every 16-lane row hold row n % 8)
    float mx = 0.0f;
    float bam[MODE == MODE_B ? U * STEPS : 1];
    if constexpr (MODE == MODE_A) {
#pragma unroll
        for (int i = 0; i < U * STEPS; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(xv[i][e]));
        mx = fmaxf(mx, __uint_as_float(ror8(__float_as_uint(mx))));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
    } else if constexpr (FMT != FMT_Q6_K) {
#pragma unroll
        for (int i = 0; i < U * STEPS; ++i) {
            float t = fmaxf(fmaxf(fabsf(xv[i][0]), fabsf(xv[i][1])), fmaxf(fabsf(xv[i][2]), fabsf(xv[i][3])));
            t = fmaxf(t, __uint_as_float(ror8(__float_as_uint(t))));
            t = fmaxf(t, __shfl_xor(t, 16));
            bam[i] = fmaxf(t, __shfl_xor(t, 32));
        }
        // the block scales, two per lane instead of every lane all of its row's: lane l
        // takes row l % 8, blocks l / 8 and l / 8 + 8 (its own maxima, picked by index);
        // 1/d, d and its f16 bits go to LDS for the row's lanes
        float* ids = dxs + U * STEPS * 8;
        uint16_t* dbs = reinterpret_cast<uint16_t*>(ids + U * STEPS * 8);
#pragma unroll
        for (int k = 0; k < (U * STEPS + 7) / 8; ++k) {
            const int bi = (lane >> 3) + 8 * k, row = lane & 7;
            float am = bam[0];
#pragma unroll
            for (int i = 1; i < U * STEPS; ++i) am = bi == i ? bam[i] : am;
            if (bi < U * STEPS) {
                float id, dval;
                uint16_t dbits;
                q8_0_scale(am, id, dbits, dval);
                ids[row * (U * STEPS) + bi] = id;
                dxs[bi * 8 + row] = dval;
                dbs[row * (U * STEPS) + bi] = dbits;
            }
        }
    }
    // mode (b), Q6_K: the Q8K scale of each super-block of x (eight steps): the
    // signed element of largest |x|, the first index on ties; lane (n, g) holds
    // elements 32 p + 8 g + 4 (n >= 8) + e of the block, in index order within the lane
    constexpr int NQK = MODE == MODE_B && FMT == FMT_Q6_K ? U * STEPS / 8 : 1;
    float kis[NQK];
    if constexpr (MODE == MODE_B && FMT == FMT_Q6_K) {
#pragma unroll
        for (int b = 0; b < NQK; ++b) {
            float best = -1.0f, bv = 0.0f;
            int bidx = 0;
#pragma unroll
            for (int p = 0; p < 8; ++p)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = xv[8 * b + p][e];
                    if (fabsf(v) > best) { best = fabsf(v); bv = v; bidx = 32 * p + 8 * g + (upper ? 4 : 0) + e; }
                }
            auto meet = [&](float ob, float obv, int oidx) {
                if (ob > best || (ob == best && oidx < bidx)) { best = ob; bv = obv; bidx = oidx; }
            };
            meet(__uint_as_float(ror8(__float_as_uint(best))), __uint_as_float(ror8(__float_as_uint(bv))), (int)ror8((uint32_t)bidx));
            meet(__shfl_xor(best, 16), __shfl_xor(bv, 16), __shfl_xor(bidx, 16));
            meet(__shfl_xor(best, 32), __shfl_xor(bv, 32), __shfl_xor(bidx, 32));
            float d;
            q8k_scale(bv, best, kis[b], d);
            if (!upper && g == 0) dxs[b * 8 + n] = d;
            if (EMIT && blockIdx.x == 0 && a.act != nullptr && r8 < M && (b >> 1) < ureal && !upper && g == 0)
                *reinterpret_cast<float*>(a.act + ((int64_t)r8 * (K / 256) + 2 * u0 + b) * 292) = d;
        }
    }
    const int ex = MODE == MODE_A ? split_exp(mx) : 0;
    const float sc = ldexpf(1.0f, ex);
    // (every activation load has been waited for above; the ring loads below are
    // not tracked by the compiler and must not be moved ahead of that wait)
    __builtin_amdgcn_sched_barrier(0);

    // the rest of the ring, then the split while it fills
#pragma unroll
    for (int i = 1; i < D; ++i)
        if (iq < Q) issue(i);

    half8_t areg[U][STEPS];
    const bool emit_act = EMIT && blockIdx.x == 0 && a.act != nullptr && r8 < M;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int p = 0; p < STEPS; ++p) {
            const float* v = xv[u * STEPS + p];
            if constexpr (MODE == MODE_B) {
                // the block's Q8_0 scale and values (bytes of the standalone quantizer);
                // lanes n < 8 keep theirs and receive the partner's, lanes n >= 8 are zero rows
                int qv[4];
                if constexpr (FMT == FMT_Q6_K) {
                    const int b = (u * STEPS + p) >> 3, pp = p & 7;
#pragma unroll
                    for (int e = 0; e < 4; ++e) qv[e] = q8k_q(v[e], kis[b]);
                    const uint32_t h0 = pack_h2((_Float16)qv[0], (_Float16)qv[1]), h1 = pack_h2((_Float16)qv[2], (_Float16)qv[3]);
                    const uint32_t s0 = ror8(h0), s1 = ror8(h1);
                    areg[u][p] = __builtin_bit_cast(half8_t, upper ? u32x4_t{0u, 0u, 0u, 0u} : u32x4_t{h0, h1, s0, s1});
                    if (emit_act && u < ureal) {
                        // canonical Q8K block 2 (u0 + u) + (p / 8) of row r8: f32 d, 256 int8,
                        // int16 sums of each 16 values (the pair of k-groups g, g ^ 1)
                        uint8_t* o = a.act + ((int64_t)r8 * (K / 256) + 2 * u0 + b) * 292;
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[4 + 32 * pp + 8 * g + (upper ? 4 : 0) + e] = (uint8_t)qv[e];
                        int s16 = (qv[0] + qv[1]) + (qv[2] + qv[3]);
                        s16 += (int)ror8((uint32_t)s16);
                        s16 += __shfl_xor(s16, 16);
                        if (!upper && (g & 1) == 0) reinterpret_cast<int16_t*>(o + 260)[2 * pp + (g >> 1)] = (int16_t)s16;
                    }
                    continue;
                }
                const float* ids = dxs + U * STEPS * 8;
                const float id = ids[r8 * (U * STEPS) + u * STEPS + p];
#pragma unroll
                for (int e = 0; e < 4; ++e) qv[e] = q8_0_q(v[e], id);
                const uint32_t h0 = pack_h2((_Float16)qv[0], (_Float16)qv[1]), h1 = pack_h2((_Float16)qv[2], (_Float16)qv[3]);
                const uint32_t s0 = ror8(h0), s1 = ror8(h1);
                areg[u][p] = __builtin_bit_cast(half8_t, upper ? u32x4_t{0u, 0u, 0u, 0u} : u32x4_t{h0, h1, s0, s1});
                if (emit_act && u < ureal) {
                    // canonical block 2 (u0 + u) + p of row r8: f16 d, then the 32 int8
                    const uint16_t* dbs = reinterpret_cast<const uint16_t*>(ids + U * STEPS * 8);
                    uint8_t* o = a.act + ((int64_t)r8 * (2 * a.nlu) + 2 * (u0 + u) + p) * 34;
                    if (!upper && g == 0) *reinterpret_cast<uint16_t*>(o) = dbs[r8 * (U * STEPS) + u * STEPS + p];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[2 + 8 * g + (upper ? 4 : 0) + e] = (uint8_t)qv[e];
                }
                continue;
            }
            _Float16 h[4], l[4];
            float xs[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) split_one(v[e], sc, h[e], l[e], xs[e]);
            // operand slots of the four values: in order, but Q4_K slot e holds element
            // nib_perm(e) of the k-group (the order its nibble decoder yields)
            uint32_t h0, h1, l0, l1;
            if constexpr (FMT != FMT_Q4_K) {
                h0 = pack_h2(h[0], h[1]); h1 = pack_h2(h[2], h[3]);
                l0 = pack_h2(l[0], l[1]); l1 = pack_h2(l[2], l[3]);
            } else {
                h0 = pack_h2(h[0], h[2]); h1 = pack_h2(h[1], h[3]);
                l0 = pack_h2(l[0], l[2]); l1 = pack_h2(l[1], l[3]);
            }
            // lanes n < 8 keep hi and receive the partner's hi; lanes n >= 8 keep lo
            const uint32_t s0 = ror8(upper ? h0 : l0), s1 = ror8(upper ? h1 : l1);
            const u32x4_t op = upper ? u32x4_t{s0, s1, l0, l1} : u32x4_t{h0, h1, s0, s1};
            areg[u][p] = __builtin_bit_cast(half8_t, op);
            if constexpr (FMT == FMT_Q4_K) {
                // the sub-block's sum of x*2^e (for the mins term): 32 values over the
                // lanes n, n + 8 of the four k-groups
                float t = ((xs[0] + xs[1]) + xs[2]) + xs[3];
                t += __uint_as_float(ror8(__float_as_uint(t)));
                t += __shfl_xor(t, 16);
                t += __shfl_xor(t, 32);
                if (lane < 8) sums[(u * 8 + p) * 8 + lane] = t;
            }
        }
    }
    // Q4_K: the A operand of the mins term per super-block: rows 0..7 carry the
    // eight sub-block sums of x*2^e of their activation row, divided by 32 (below
    // 2^15: f16-safe) and split into f16 hi (k 0..7) and lo (k 8..15); rows 8..15 zero
    half8_t amin[FMT == FMT_Q4_K ? U : 1];
    if constexpr (FMT == FMT_Q4_K) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            half8_t v;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const float t = (!upper && g < 2) ? sums[(u * 8 + jj) * 8 + r8] * 0.03125f : 0.0f;
                const _Float16 hi = (_Float16)t;
                v[jj] = g == 0 ? hi : (_Float16)(t - (float)hi);
            }
            amin[u] = v;
        }
    }
    // 2^-e of this lane's four output rows 4 (g & 1) + q (row r's exponent sits in lane r)
    float rsc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e0 = __builtin_amdgcn_readlane(ex, q), e1 = __builtin_amdgcn_readlane(ex, 4 + q);
        rsc[q] = MODE == MODE_A ? ldexpf(1.0f, -((g & 1) ? e1 : e0)) : 1.0f;
    }

    // ---- main loop ----
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const f32x4_t zf = {0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t nibm = 0x000f000fu, nibc = 0x64006400u;           // Q4_K nibble decode constants
    asm volatile("" : "+v"(nibm), "+v"(nibc));

    // a block pair's two matrix-core sums (block 2 (u0 + u) and the next) into acc:
    // mode (a) times the weight scales; mode (b) the exact integer sums times d_w d_x
    auto pair_epi = [&](const f32x4_t& Ce, const f32x4_t& Co, float de, float dd, int u, int tile) {
        if constexpr (MODE == MODE_A) {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = fmaf(Co[q], dd, fmaf(Ce[q], de, acc[q]));
        } else {
            const f32x4_t xe = *reinterpret_cast<const f32x4_t*>(dxs + (u * 2) * 8 + 4 * (g & 1));
            const f32x4_t xo = *reinterpret_cast<const f32x4_t*>(dxs + (u * 2 + 1) * 8 + 4 * (g & 1));
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] = fmaf(Co[q], dd * xo[q], fmaf(Ce[q], de * xe[q], acc[q]));
            if constexpr (EMIT) {
                const int ng = tile * 16 + n;
                if (g < 2 && ng < N) {
                    int32_t* o = a.sums + ((int64_t)(4 * g) * N + ng) * (2 * a.nlu) + 2 * (u0 + u);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (4 * g + q < M) {
                            o[(int64_t)q * N * (2 * a.nlu)] = (int32_t)Ce[q];
                            o[(int64_t)q * N * (2 * a.nlu) + 1] = (int32_t)Co[q];
                        }
                    }
                }
            }
        }
    };

    auto compute = [&](const uint8_t* sbuf, auto sc_, int tile) {
        constexpr int s = decltype(sc_)::value;
        const uint8_t* rrow = sbuf + n * (16 * CPR);
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int u = s * P + j;
            if (u >= ureal) break;  // wave-uniform: units past the slice are not the row's
            const uint8_t* rp = rrow + j * LUB;
            if constexpr (FMT == FMT_Q8_0) {
                // even block: values 8g .. 8g+7 are bytes 2+8g .. 9+8g of the pair
                const uint32_t E0 = lds32(rp), E8 = lds32(rp + 32);
                const uint8_t* xe = rp + 8 * g;
                const uint8_t* xo = rp + 36 + 8 * g;
                const uint32_t e0 = lds32(xe), e1 = lds32(xe + 4), e2 = lds32(xe + 8);
                const half8_t Be = i8x8_to_f16(__builtin_amdgcn_alignbyte(e1, e0, 2), __builtin_amdgcn_alignbyte(e2, e1, 2));
                const half8_t Bo = i8x8_to_f16(lds32(xo), lds32(xo + 4));
                const f32x4_t Ce = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[s * P + j][0], Be, zf, 0, 0, 0);
                const f32x4_t Co = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[s * P + j][1], Bo, zf, 0, 0, 0);
                pair_epi(Ce, Co, f16lo(E0), f16hi(E8), s * P + j, tile);
            } else if constexpr (FMT == FMT_Q4_0 || FMT == FMT_Q5_0) {
                // pair of blocks: Q4_0 d | qs[16], Q5_0 d | qh[4] | qs[16], twice.  k-group g
                // takes the low (g < 2) or high nibbles of qs bytes 8 (g & 1) .. +7, Q5_0
                // with bits 8g .. 8g+7 of qh as their fifth bits
                constexpr int QS0 = FMT == FMT_Q4_0 ? 2 : 6, HALF = LUB / 2, QS1 = HALF + QS0;
                constexpr int OFF = FMT == FMT_Q4_0 ? 8 : 16;
                const int sh = 4 * (g >> 1), qo = 8 * (g & 1);
                const uint32_t a0 = lds32(rp + QS0 - 2 + qo), a1 = lds32(rp + QS0 + 2 + qo), a2 = lds32(rp + QS0 + 6 + qo);
                uint32_t ce0 = (__builtin_amdgcn_alignbyte(a1, a0, 2) >> sh) & 0x0f0f0f0fu;
                uint32_t ce1 = (__builtin_amdgcn_alignbyte(a2, a1, 2) >> sh) & 0x0f0f0f0fu;
                uint32_t co0 = (lds32(rp + QS1 + qo) >> sh) & 0x0f0f0f0fu;
                uint32_t co1 = (lds32(rp + QS1 + qo + 4) >> sh) & 0x0f0f0f0fu;
                if constexpr (FMT == FMT_Q5_0) {
                    const uint32_t he = __builtin_amdgcn_alignbyte(lds32(rp + 4), lds32(rp), 2), ho = lds32(rp + HALF + 2);
                    ce0 |= spread4((he >> (8 * g)) & 15u);
                    ce1 |= spread4((he >> (8 * g + 4)) & 15u);
                    co0 |= spread4((ho >> (8 * g)) & 15u);
                    co1 |= spread4((ho >> (8 * g + 4)) & 15u);
                }
                const half8_t Be = u8x8_to_f16<OFF>(ce0, ce1), Bo = u8x8_to_f16<OFF>(co0, co1);
                const f32x4_t Ce = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[s * P + j][0], Be, zf, 0, 0, 0);
                const f32x4_t Co = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[s * P + j][1], Bo, zf, 0, 0, 0);
                pair_epi(Ce, Co, f16lo(lds32(rp)), f16hi(lds32(rp + HALF - 2)), s * P + j, tile);
            } else if constexpr (FMT == FMT_Q6_K) {
                // two super-blocks of ql[128] | qh[64] | sc[16] (int8) | d (f16), the second
                // two bytes into a dword.  Step p (32 values) of one: half h = p / 4, quarter
                // q = p % 4; k-group g takes l = 8g .. 8g+7 of the quarter, low bits in nibble
                // q / 2 of ql[64h + 32 (q & 1) + l], high bits in bit pair q of qh[32h + l],
                // scale sc[2p + g / 2].  The scale enters the weights as 16 sh + sl (sl in
                // 0..15): both products with q - 32 are exact f16 integers, and the two
                // sums of a super-block meet in f32 after its last step.
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const uint8_t* sp = rp + 210 * b;
                    auto ld8 = [&](int off, uint32_t& v0, uint32_t& v1) {
                        if (b == 0) {
                            v0 = lds32(sp + off);
                            v1 = lds32(sp + off + 4);
                        } else {
                            const uint32_t a0 = lds32(sp + off - 2), a1 = lds32(sp + off + 2), a2 = lds32(sp + off + 6);
                            v0 = __builtin_amdgcn_alignbyte(a1, a0, 2);
                            v1 = __builtin_amdgcn_alignbyte(a2, a1, 2);
                        }
                    };
                    f32x4_t Ch = zf, Cl = zf;
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const int h = p >> 2, q = p & 3;
                        uint32_t l0, l1, h0, h1;
                        ld8(64 * h + 32 * (q & 1) + 8 * g, l0, l1);
                        ld8(128 + 32 * h + 8 * g, h0, h1);
                        const int ns = 4 * (q >> 1), hs = 2 * q;
                        const uint32_t c0 = ((l0 >> ns) & 0x0f0f0f0fu) | (((h0 >> hs) & 0x03030303u) << 4);
                        const uint32_t c1 = ((l1 >> ns) & 0x0f0f0f0fu) | (((h1 >> hs) & 0x03030303u) << 4);
                        const half8_t B = u8x8_to_f16<32>(c0, c1);
                        const int sa = 210 * b + 192 + 2 * p + (g >> 1);  // the scale's byte in the unit
                        const int sc = (int)(int8_t)(lds32(rp + (sa & ~3)) >> (8 * (sa & 3)));
                        const _Float16 fh = (_Float16)(sc >> 4), fl = (_Float16)(sc & 15);
                        const half8_t shv = {fh, fh, fh, fh, fh, fh, fh, fh}, slv = {fl, fl, fl, fl, fl, fl, fl, fl};
                        Ch = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[s * P + j][8 * b + p], B * shv, Ch, 0, 0, 0);
                        Cl = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[s * P + j][8 * b + p], B * slv, Cl, 0, 0, 0);
                        if constexpr (EMIT) {
                            // the per-16 sums S_2p, S_2p+1 (weights q - 32): k-groups 0, 1 and 2, 3
                            const half8_t zh = {};
                            const f32x4_t S0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[s * P + j][8 * b + p], g < 2 ? B : zh, zf, 0, 0, 0);
                            const f32x4_t S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[s * P + j][8 * b + p], g < 2 ? zh : B, zf, 0, 0, 0);
                            const int ng = tile * 16 + n, sbk = 2 * (u0 + s * P + j) + b;
                            if (g < 2 && ng < N) {
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    if (4 * g + q < M) {
                                        int32_t* o = a.sums + ((int64_t)(4 * g + q) * N + ng) * (17 * (K / 256)) + 17 * sbk + 2 * p;
                                        o[0] = (int32_t)S0[q];
                                        o[1] = (int32_t)S1[q];
                                    }
                                }
                            }
                        }
                    }
                    const float d = b == 0 ? f16lo(lds32(rp + 208)) : f16hi(lds32(rp + 416));
                    if constexpr (MODE == MODE_A) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[q] = fmaf(fmaf(16.0f, Ch[q], Cl[q]), d, acc[q]);
                    } else {
                        // sumi = 16 Ch + Cl, both exact integers; d_x of the super-block's rows
                        const f32x4_t dx = *reinterpret_cast<const f32x4_t*>(dxs + (2 * (s * P + j) + b) * 8 + 4 * (g & 1));
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[q] = fmaf(fmaf(16.0f, Ch[q], Cl[q]), d * dx[q], acc[q]);
                        if constexpr (EMIT) {
                            const int ng = tile * 16 + n, sbk = 2 * (u0 + s * P + j) + b;
                            if (g < 2 && ng < N) {
#pragma unroll
                                for (int q = 0; q < 4; ++q)
                                    if (4 * g + q < M)
                                        a.sums[((int64_t)(4 * g + q) * N + ng) * (17 * (K / 256)) + 17 * sbk + 16] =
                                            16 * (int32_t)Ch[q] + (int32_t)Cl[q];
                            }
                        }
                    }
                }
            } else {
                const u32x4_t H = lds128(rp);
                const float d = f16lo(H[0]), dmin = f16hi(H[0]);
                const uint32_t s0 = H[1], s1 = H[2], s2 = H[3];
                const uint32_t sc4[2] = {s0 & 0x3f3f3f3fu, (s2 & 0x0f0f0f0fu) | ((s0 >> 2) & 0x30303030u)};
                const uint32_t mn4[2] = {s1 & 0x3f3f3f3fu, ((s2 >> 4) & 0x0f0f0f0fu) | ((s1 >> 2) & 0x30303030u)};
                // the weights enter as exact f16 sc_j q (at most 945: one fused multiply-add
                // on the 1024 + q bit pattern); the super-block's sum stays in the
                // accumulator.  Mins: one more matrix-core step against the sub-block sums
                f32x4_t Cs = zf;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x2_t Qv = lds64(rp + 16 + 32 * c + 8 * g);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int jj = 2 * c + h;
                        const _Float16 sc = (_Float16)(float)((sc4[jj >> 2] >> (8 * (jj & 3))) & 0xffu);
                        const half2_t s2 = {sc, sc}, o2 = {(_Float16)(-1024.0f) * sc, (_Float16)(-1024.0f) * sc};
                        const uint32_t w0 = Qv[0] >> (4 * h), w1 = Qv[1] >> (4 * h);
                        half8_t B;
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const uint32_t src = (t < 2 ? w0 : w1) >> (8 * (t & 1));
                            const half2_t v = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, (src & nibm) | (nibc & ~nibm)), s2, o2);
                            B[2 * t] = v[0];
                            B[2 * t + 1] = v[1];
                        }
                        Cs = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[s * P + j][jj], B, Cs, 0, 0, 0);
                    }
                }
                const half8_t Bm0 = u8x8_to_f16<0>(mn4[0], mn4[1]), zh = {};
                const f32x4_t Cm = __builtin_amdgcn_mfma_f32_16x16x32_f16(amin[s * P + j], g < 2 ? Bm0 : zh, zf, 0, 0, 0);
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[q] = fmaf(d, Cs[q], fmaf(-32.0f * dmin, Cm[q], acc[q]));
            }
        }
    };

    int slot = 0;
    for (int tt = 0; tt < nt; ++tt) {
        auto stage = [&](auto sc_) {
            constexpr int s = decltype(sc_)::value;
            const int q = tt * S + s;
            vm_wait_ahead<TL, D - 1>(min(D - 1, Q - 1 - q));  // stage q has landed
            if (s < sreal) compute(ring + slot * SBY, sc_, t0 + tt);
            if (iq < Q) {
                lgkm_wait0();  // this buffer's reads are done before it is refilled
                issue(slot);
            }
            slot = slot == D - 1 ? 0 : slot + 1;
        };
        stage(std::integral_constant<int, 0>{});
        if constexpr (S > 1) stage(std::integral_constant<int, 1>{});

        // the tile's partial of this slice: hi + lo (lanes g and g + 2), scaled back by
        // 2^-e, parked in LDS; after one barrier the slices are added in order
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += __shfl_xor(acc[q], 32);
        float* ps = part + ((tt & 1) * GV_WAVES + wave) * 128;
        if (lane < 32) {
#pragma unroll
            for (int q = 0; q < 4; ++q) ps[(4 * (g & 1) + q) * 16 + n] = acc[q] * rsc[q];
        }
        acc = zf;
        lgkm_wait0();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (tid < 128) {
            const int m = tid >> 4, ng = (t0 + tt) * 16 + (tid & 15);
            const float* pp = part + (tt & 1) * GV_WAVES * 128 + tid;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < GV_WAVES; ++w) v += pp[w * 128];
            if (m < M && ng < N && a.y) a.y[(int64_t)m * N + ng] = v;
        }
    }
}

typedef void (*GrKernel)(GemvRegArgs);

template <int FMT, int MODE, int U, int P, int D, bool EMIT>
static hipError_t gr_launch(const GemvRegArgs& a, int grid, hipStream_t s)
{
    using C = GrCfg<FMT, MODE, U, P, D>;
    GrKernel k = gemv_reg_kernel<FMT, MODE, U, P, D, EMIT>;
    static std::set<std::pair<int, const void*>> done;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (done.insert(std::make_pair(dev, (const void*)k)).second) {
            (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
            (void)hipGetLastError();
        }
    }
    GemvRegArgs args = a;
    void* argv[] = {&args};
    return hipLaunchKernel((const void*)k, dim3(grid), dim3(GV_THREADS), argv, C::LDS, s);
}

// Units per wave slice for this K, or 0 when the slice's operand would not fit
// the registers (64 VGPRs at most: 8 block pairs, Q4_K 2 super-blocks, so
// K <= 4096).
static int gr_units(int fmt, int64_t K)
{
    const int64_t nlu = K / gr_vpl(fmt);
    const int64_t per = (nlu + GV_WAVES - 1) / GV_WAVES;
    if (fmt == FMT_Q6_K) return per <= 1 ? 1 : 0;
    if (fmt == FMT_Q4_K) return per <= 1 ? 1 : per <= 2 ? 2 : 0;
    return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 0;
}

bool gemv_reg_supported(int fmt, int mode, int M, int64_t N, int64_t K)
{
    if (M < 2 || M > GEMV_MAX_M || N < 1) return false;
    // mode (b): Q4_0, Q5_0, Q6_K (Q8_0 and Q4_K run their integer tile kernel)
    if (mode == MODE_B) { if (fmt != FMT_Q4_0 && fmt != FMT_Q5_0 && fmt != FMT_Q6_K) return false; }
    else if (mode != MODE_A) return false;
    if (fmt == FMT_Q8_0 || fmt == FMT_Q4_0 || fmt == FMT_Q5_0) { if (K % 64 != 0) return false; }
    else if (fmt == FMT_Q4_K) { if (K % 256 != 0) return false; }
    else if (fmt == FMT_Q6_K) { if (K % 512 != 0) return false; }  // super-block pairs: 4-byte-aligned rows
    else return false;
    return gr_units(fmt, K) > 0 && (int64_t)M * K * 4 <= 0xffffffffll;
}

// The instances of the 32-value formats: stages of four block pairs where the
// slice has them (two or one below), and for Q5_0 one pair where two would be an
// even chunk count.
template <int FMT, int MODE, bool EMIT>
static hipError_t gr_launch_pairs(int U, const GemvRegArgs& a, int grid, hipStream_t s)
{
    if (U == 8) return gr_launch<FMT, MODE, 8, 4, 4, EMIT>(a, grid, s);
    if (U == 4) return gr_launch<FMT, MODE, 4, 4, 4, EMIT>(a, grid, s);
    if (U == 2) return gr_launch<FMT, MODE, 2, (FMT == FMT_Q5_0 ? 1 : 2), 4, EMIT>(a, grid, s);
    return gr_launch<FMT, MODE, 1, 1, 4, EMIT>(a, grid, s);
}

template <int FMT>
static hipError_t gr_launch_b(int U, bool emit, const GemvRegArgs& a, int grid, hipStream_t s)
{
    return emit ? gr_launch_pairs<FMT, MODE_B, true>(U, a, grid, s) : gr_launch_pairs<FMT, MODE_B, false>(U, a, grid, s);
}

hipError_t launch_gemv_reg(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, int M, float* y,
                           hipStream_t s, const Trace* tr)
{
    if (!gemv_reg_supported(fmt, mode, M, N, K) || (tr && mode != MODE_B)) return hipErrorInvalidValue;
    GemvRegArgs a{};
    a.w = (const uint8_t*)w;
    a.nlu = (int)(K / gr_vpl(fmt));
    a.row_bytes = a.nlu * gr_lub(fmt);
    a.w_bytes = N * (int64_t)a.row_bytes;
    a.N = (int)N;
    a.K = (int)K;
    a.M = M;
    a.tiles = (int)((N + 15) / 16);
    const int cus = device_cus();
    a.T = (a.tiles + cus - 1) / cus;
    const int grid = (a.tiles + a.T - 1) / a.T;
    a.x = x;
    a.y = y;
    a.sums = tr ? tr->sums : nullptr;
    a.act = tr ? tr->act : nullptr;
    const int U = gr_units(fmt, K);
    if (mode == MODE_B) {
        if (fmt == FMT_Q4_0) return gr_launch_b<FMT_Q4_0>(U, tr != nullptr, a, grid, s);
        if (fmt == FMT_Q5_0) return gr_launch_b<FMT_Q5_0>(U, tr != nullptr, a, grid, s);
        return tr ? gr_launch<FMT_Q6_K, MODE_B, 1, 1, 2, true>(a, grid, s) : gr_launch<FMT_Q6_K, MODE_B, 1, 1, 2, false>(a, grid, s);
    }
    if (fmt == FMT_Q8_0) return gr_launch_pairs<FMT_Q8_0, MODE_A, false>(U, a, grid, s);
    if (fmt == FMT_Q4_0) return gr_launch_pairs<FMT_Q4_0, MODE_A, false>(U, a, grid, s);
    if (fmt == FMT_Q5_0) return gr_launch_pairs<FMT_Q5_0, MODE_A, false>(U, a, grid, s);
    if (fmt == FMT_Q6_K) return gr_launch<FMT_Q6_K, MODE_A, 1, 1, 2, false>(a, grid, s);  // 432-byte stage rows: two fit
    if (U == 2) return gr_launch<FMT_Q4_K, MODE_A, 2, 1, 4, false>(a, grid, s);
    return gr_launch<FMT_Q4_K, MODE_A, 1, 1, 4, false>(a, grid, s);
}

}  // namespace qmm
