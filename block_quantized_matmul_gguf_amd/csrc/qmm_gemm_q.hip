// qmm_gemm_q.hip -- prefill kernel (M > 8) for mode (b) on the int8 matrix cores.
//
// Mode (b) quantizes every activation row first (Q8_0 blocks of 32 values for
// Q8_0 weights, Q8K blocks of 256 for Q4_K) and sums integer products block by
// block, each integer block sum scaled by the weight and activation block
// scales (page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处).
// Here every 32-value block is one v_mfma_i32_32x32x32_i8: int8 activations
// against int8 weights (Q8_0: q; Q4_K: the 4-bit values 0..15) give the exact
// int32 block sums S of a 32 x 32 output tile, which are scaled in f32:
//   Q8_0: acc += (d_x * d_w) * S                  for every block;
//   Q4_K: acc += (d_x * d * sc_j) * S_j           for every sub-block j,
//         acc -= (d_x * dmin) * sum_j m_j * bsum_j once per super-block.
// The mins term is one v_mfma_f32_32x32x16_f16 on exact f16 operands: m_j
// against the activation's 32-value sums bsum_j, each split into a multiple
// of 64 and a remainder in [0, 63] (exact f16 integers), so the f32 result is
// the exact integer sum.
//
// A workgroup of 128*MW threads owns a (32*MW) x (32*TN) output tile: MW
// slices of 32 rows times two K groups (the launched 128 x 224 tile: 512
// threads, one workgroup per compute unit on 512 x 14336).  K advances 64
// values (two blocks) per stage, group g takes block g of every stage over
// all 32*TN columns, and the two groups' partial sums are added through LDS at
// the end.  Registers hold the stage after the one in LDS: they are written
// to the idle LDS buffer one item per MFMA of the current stage, then the
// following stage is loaded; one barrier per stage.  Consecutive lanes load
// consecutive 16-byte pieces of one weight row, so that a load instruction
// touches few rows; the Q8_0 blocks (two bytes of scale before their values)
// are realigned in registers with one lane exchange and a byte permute per
// dword.
#include <map>
#include <mutex>
#include <set>
#include <type_traits>
#include <utility>

#include "qmm_device.h"

namespace qmm {

struct QGemmArgs {
    PrefillGroup g;       // the problems: weights, outputs (EMIT instances: may be null), rows
    int64_t row_bytes;
    int K, M;
    int nm;               // row tiles of the output
    int remap;            // 1: give each XCD a contiguous run of tiles
    const int8_t* q;      // quantized activations [M][K]
    const float* dx;      // activation block scales, block-major: Q8_0 [K/32][M], Q8K [K/256][M]
    const _Float16* bsx;  // Q8K: [K/256][M][16] sub-block sums, multiples of 64 then remainders
    int32_t* sums;        // EMIT: Q8_0 S per block; Q4_K S_0..S_7 and summins per super-block (slot 8 left)
};


// An LDS row of one block: 32 int8 as two 16-byte halves; half h of row r
// sits in slot h ^ ((r >> 3) & 1), so the 16 rows an MFMA operand read
// touches at once cover all banks.
QMM_DEV uint32_t qswz(int row, int h) { return (uint32_t)(row * 32 + ((h ^ ((row >> 3) & 1)) << 4)); }

// MW waves of 32 rows per K group: BM = 32*MW rows, 128*MW threads.  A
// stage is KB block pairs, 64*KB values: group g takes blocks g, g+2, ...
template <int FMT, int MW, int TN, int KB>
struct QCfg {
    static constexpr bool Q8 = FMT == FMT_Q8_0;
    static constexpr int Q_BM = 32 * MW, Q_NT = 128 * MW;
    static constexpr int BN = 32 * TN;
    static constexpr int SB = 2 * KB;        // blocks per stage
    static constexpr int SV = 32 * SB;       // values per stage
    static constexpr int A_BLK = Q_BM * 32;  // one block of the activation tile, bytes
    static constexpr int B_BLK = BN * 32;
    // [buffer][block] images of the activation and weight tiles and d_x
    // [buffer][block][BM] f32.  Column scales: Q8_0 d_w [buffer][block][BN]
    // f32; Q4_K, by super-block parity, d * sc_j [2][8][BN] f32, dmin [2][BN]
    // f32, m_j [2][BN][8] f16 and the activation sub-block sums [2][BM][16] f16.
    static constexpr int OFF_A = 0;
    static constexpr int OFF_B = OFF_A + 2 * SB * A_BLK;
    static constexpr int OFF_DX = OFF_B + 2 * SB * B_BLK;
    static constexpr int OFF_DW = OFF_DX + 2 * SB * Q_BM * 4;
    static constexpr int OFF_DMIN = OFF_DW + (Q8 ? 2 * SB : 16) * BN * 4;
    static constexpr int OFF_MJ = OFF_DMIN + 2 * BN * 4;
    static constexpr int OFF_BSX = OFF_MJ + 2 * BN * 16;
    static constexpr int STAGE_BYTES = Q8 ? OFF_DMIN : OFF_BSX + 2 * Q_BM * 32;
    static constexpr int RED_BYTES = Q_BM * BN * 4;  // the K groups' sum
    static constexpr int BYTES = STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES;
    static constexpr int AU = Q_BM * 2 * SB / Q_NT;  // 16-byte activation pieces per thread
    // weight load units: Q8_0 (row, block pair, 16-byte quarter of its 64
    // bytes); Q4_K (row, 32-byte chunk, 16-byte half)
    static constexpr int UPR = Q8 ? 4 * KB : 2 * KB;  // units per row
    static constexpr int UNITS = UPR * BN;
    static constexpr int BU = (UNITS + Q_NT - 1) / Q_NT;
    static_assert(AU * Q_NT == Q_BM * 2 * SB, "activation pieces must split evenly");
    static_assert(Q8 || 256 % SV == 0, "a Q4_K stage must not cross a super-block");
};

// EMIT: the same kernel, which also writes the exact int32 block sums its
// matrix-core steps produce (Q8_0: S per 32-value block; Q4_K: S_j per
// sub-block and the super-block's mins sum).
template <int FMT, int MW, int TN, int KB, bool EMIT>
__global__ __launch_bounds__(128 * MW, 2) void gemm_q_kernel(QGemmArgs a)
{
    using C = QCfg<FMT, MW, TN, KB>;
    constexpr int BN = C::BN, BU = C::BU, AU = C::AU, Q_BM = C::Q_BM, Q_NT = C::Q_NT, SB = C::SB, SV = C::SV;
    constexpr bool Q8 = C::Q8;
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
    const int m0 = (t % a.nm) * Q_BM, n0 = (t / a.nm - tile0) * BN;
    const int wm = (wave % MW) * 32, g = wave / MW;
    const int l32 = lane & 31, hl = lane >> 5;
    const int nst = (K + SV - 1) / SV;
    const int kb_last = ((K - (nst - 1) * SV) / 32) >> 1;  // block pairs in the last stage
    const int64_t rb = a.row_bytes;

    // Loads past the end of a resource return zeros: rows past M or N read
    // zeros.  The block-major scale arrays get a resource per block row,
    // starting at this tile's first row, so their offsets stay small at any
    // M and K.  Past the end of a ragged last stage, the staging reads the
    // next row's bytes into blocks that are never multiplied.
    const rsrc_t rq = make_rsrc(a.q + (int64_t)m0 * K, clamp_u32((int64_t)(M - m0) * K));
    const rsrc_t rw = make_rsrc(W + (int64_t)n0 * rb, clamp_u32((int64_t)(N - n0) * rb));
    const uint32_t dx_bytes = clamp_u32((int64_t)(M - m0) * 4), bsx_bytes = clamp_u32((int64_t)(M - m0) * 32);
    auto rdx_of = [&](int blk) { return make_rsrc(a.dx + (int64_t)blk * M + m0, dx_bytes); };

    // ---- staging roles, fixed for the whole K loop ----
    // activations: (row, 16-byte piece of the stage's SV bytes)
    uint32_t ag[AU], as_[AU];
#pragma unroll
    for (int i = 0; i < AU; ++i) {
        const int idx = tid + Q_NT * i, row = idx / (2 * SB), part = idx % (2 * SB);
        ag[i] = (uint32_t)(row * K + 16 * part);
        as_[i] = (uint32_t)((part >> 1) * C::A_BLK + qswz(row, part & 1));
    }
    // activation scales (waves 0..DW-1): one row per lane
    constexpr int DW = MW / 2 > 0 ? MW / 2 : 1;
    const int drow = tid & (Q_BM - 1);
    const uint32_t dg = (uint32_t)(drow * 4);
    // weight units, consecutive lanes along a row so that a load instruction
    // touches few rows; threads past the last unit repeat earlier ones (same
    // values to the same places)
    constexpr int UPR = C::UPR;
    uint32_t bg[BU];
    int brow[BU];
    const int bp = Q8 ? (tid & 3) : (tid & 1);                 // quarter (Q8_0) or half (Q4_K)
    const int bpair = Q8 ? (tid >> 2) % KB : (tid >> 1) % KB;  // block pair (Q8_0) or chunk (Q4_K) in the stage
#pragma unroll
    for (int i = 0; i < BU; ++i) {
        const int u = (tid + Q_NT * i) % C::UNITS;
        brow[i] = u / UPR;
        bg[i] = (uint32_t)(brow[i] * rb + (Q8 ? 68 * bpair + 16 * bp : 32 * bpair + 16 * bp));
    }
    // Q8_0 realignment: a block pair's 68 bytes are d0 q0..q31 d1 q0..q31;
    // quarter p holds bytes 16p..16p+15 and needs the next dword (the next
    // quarter's first; bytes 64..67 for the last): quarters 0, 1 shift by 2
    // bytes (the pair's first block, halves 0 and 1), 2, 3 by 4 (its second).
    const uint32_t psel = bp < 2 ? 0x05040302u : 0x07060504u;
    // Q4_K activation sub-block sums (waves 0..MW-1): (row, half)
    const int xrow = (tid >> 1) & (Q_BM - 1), xpart = tid & 1;
    const uint32_t xg = (uint32_t)((xrow * 16 + 8 * xpart) * 2);

    // ---- staging registers ----
    uint4 ra[AU];
    float rdx[Q8 ? SB : 1];
    uint4 rw4[BU];
    uint32_t rtail[Q8 ? BU : 1];
    uint4 rhd[Q8 ? 1 : BU];
    uint4 rbx;

    auto load = [&](int st) {
#pragma unroll
        for (int i = 0; i < AU; ++i)
            ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, ag[i], SV * st, 0));
        if (wave < DW) {
            if constexpr (Q8) {
#pragma unroll
                for (int b = 0; b < SB; ++b)
                    rdx[b] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdx_of(SB * st + b), dg, 0, 0));
            } else {
                rdx[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdx_of(SV * st / 256), dg, 0, 0));
            }
        }
        if constexpr (Q8) {
#pragma unroll
            for (int i = 0; i < BU; ++i) {
                rw4[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, bg[i], 68 * KB * st, 0));
                if (bp == 3) rtail[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, bg[i] + 16, 68 * KB * st, 0);
            }
        } else {
            const int sb = SV * st / 256, c0 = (SV * st % 256) / 64;
#pragma unroll
            for (int i = 0; i < BU; ++i) {
                rw4[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, bg[i] + 16 + 32 * c0, 144 * sb, 0));
                if (c0 == 0)
                    rhd[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, brow[i] * (uint32_t)rb, 144 * sb, 0));
            }
            if (c0 == 0 && wave < MW)
                rbx = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    make_rsrc(a.bsx + ((int64_t)sb * M + m0) * 16, bsx_bytes), xg, 0, 0));
        }
    };

    // registers of stage st -> LDS buffer P, as NI items that the compute
    // loop spreads over its MFMAs: item 0 the activation pieces and scales,
    // item 1 + i weight unit i
    constexpr int NI = 1 + BU;
    auto store_item = [&](int w, int st, auto pc) {
        constexpr int P = decltype(pc)::value;
        uint8_t* sb_ = lds + C::OFF_B + P * SB * C::B_BLK;
        const int sb = SV * st / 256, c0 = (SV * st % 256) / 64, par = sb & 1;  // Q4_K position
        if (w == 0) {
#pragma unroll
            for (int i = 0; i < AU; ++i) *reinterpret_cast<uint4*>(lds + C::OFF_A + P * SB * C::A_BLK + as_[i]) = ra[i];
            if (wave < DW) {
                float* sdx = reinterpret_cast<float*>(lds + C::OFF_DX) + P * SB * Q_BM + drow;
#pragma unroll
                for (int b = 0; b < SB; ++b) sdx[b * Q_BM] = Q8 ? rdx[Q8 ? b : 0] : rdx[0];
            }
            if constexpr (!Q8) {
                if (c0 == 0 && wave < MW)
                    *reinterpret_cast<uint4*>(lds + C::OFF_BSX + par * Q_BM * 32 + qswz(xrow, xpart)) = rbx;
            }
            return;
        }
        const int i = w - 1;
        if constexpr (Q8) {
            float* sdw = reinterpret_cast<float*>(lds + C::OFF_DW) + P * SB * BN;
            const uint4 v = rw4[i];
            const uint32_t nx = (uint32_t)__builtin_amdgcn_update_dpp((int)v.x, (int)v.x, 0xF9, 0xF, 0xF, false);
            const uint32_t e = bp == 3 ? rtail[i] : nx;
            const uint4 o = make_uint4(__builtin_amdgcn_perm(v.y, v.x, psel), __builtin_amdgcn_perm(v.z, v.y, psel),
                                       __builtin_amdgcn_perm(v.w, v.z, psel), __builtin_amdgcn_perm(e, v.w, psel));
            const int blk = 2 * bpair + (bp >> 1);
            *reinterpret_cast<uint4*>(sb_ + blk * C::B_BLK + qswz(brow[i], bp & 1)) = o;
            if (bp == 0) sdw[blk * BN + brow[i]] = f16lo(v.x);
            if (bp == 2) sdw[blk * BN + brow[i]] = f16hi(v.x);
        } else {
            const uint4 nb = rw4[i];
            const uint32_t mk = 0x0f0f0f0fu;
            // low nibbles of chunk c: sub-block 2c (stage block 2*bpair); high: 2c+1
            *reinterpret_cast<uint4*>(sb_ + 2 * bpair * C::B_BLK + qswz(brow[i], bp)) =
                make_uint4(nb.x & mk, nb.y & mk, nb.z & mk, nb.w & mk);
            *reinterpret_cast<uint4*>(sb_ + (2 * bpair + 1) * C::B_BLK + qswz(brow[i], bp)) =
                make_uint4((nb.x >> 4) & mk, (nb.y >> 4) & mk, (nb.z >> 4) & mk, (nb.w >> 4) & mk);
            if (c0 == 0 && bpair == 0) {
                const uint4 hd = rhd[i];
                if (bp == 0) {  // d * sc_j for the eight sub-blocks
                    const float d = f16lo(hd.x);
                    float* sds = reinterpret_cast<float*>(lds + C::OFF_DW) + par * 8 * BN + brow[i];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        int sc, mn;
                        q4k_scale_min(hd.y, hd.z, hd.w, j, sc, mn);
                        sds[j * BN] = d * (float)sc;
                    }
                } else {  // dmin and the mins m_j
                    reinterpret_cast<float*>(lds + C::OFF_DMIN)[par * BN + brow[i]] = f16hi(hd.x);
                    half8_t mj;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        int sc, mn;
                        q4k_scale_min(hd.y, hd.z, hd.w, j, sc, mn);
                        mj[j] = (_Float16)(float)mn;
                    }
                    *reinterpret_cast<half8_t*>(lds + C::OFF_MJ + (par * BN + brow[i]) * 16) = mj;
                }
            }
        }
    };
    auto store = [&](int st, auto pc) {
#pragma unroll
        for (int w = 0; w < NI; ++w) store_item(w, st, pc);
    };

    f32x16_t acc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    const i32x16_t izero = {};
    const f32x16_t fzero = {};
    const f32x32_t fzero32 = {};

    // block blk of stage st out of buffer P
    auto block = [&](int st, int blk, auto pc, auto hook) {
        constexpr int P = decltype(pc)::value;
        constexpr int NPAIR = (TN + 1) / 2;
        const uint8_t* sa = lds + C::OFF_A + (P * SB + blk) * C::A_BLK;
        const uint8_t* sbb = lds + C::OFF_B + (P * SB + blk) * C::B_BLK;
        const i32x4_t af = *reinterpret_cast<const i32x4_t*>(sa + qswz(wm + l32, hl));
        const int sub = 2 * ((SV * st % 256) / 64) + blk;  // Q4_K sub-block
        const float* sdw = reinterpret_cast<const float*>(lds + C::OFF_DW) + l32 +
                           (Q8 ? (P * SB + blk) * BN : (((SV * st / 256) & 1) * 8 + sub) * BN);
        i32x4_t bn = *reinterpret_cast<const i32x4_t*>(sbb + qswz(l32, hl));
        // outer-product operands: d_x of row wm + l32 in both halves, the
        // column scale of tile 2p + hl (the last tile repeated for odd TN)
        const float dxa = reinterpret_cast<const float*>(lds + C::OFF_DX)[(P * SB + blk) * Q_BM + wm + l32];
        float dwb[NPAIR];
#pragma unroll
        for (int q = 0; q < NPAIR; ++q) dwb[q] = sdw[32 * (2 * q + 1 < TN ? 2 * q + hl : 2 * q)];
        f32x32_t s2;
        i32x16_t cp;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const i32x4_t bf = bn;
            const i32x16_t cv = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf, izero, 0, 0, 0);
            if constexpr (EMIT) {
                // block blk of stage st: Q8_0 block SB*st + blk; Q4_K sub-block `sub` of super-block SV*st/256
                const int n = n0 + 32 * j + l32;
                const int spr = Q8 ? K / 32 : (K / 256) * 10;
                const int idx = Q8 ? SB * st + blk : (SV * st / 256) * 10 + sub;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm + 8 * (r >> 2) + 4 * hl + (r & 3);
                    if (m < M && n < N) a.sums[((int64_t)m * N + n) * spr + idx] = cv[r];
                }
            }
            // issue the MFMA before the previous tile's scaling, which then
            // runs while the matrix cores work (never waits on this result)
            __builtin_amdgcn_sched_barrier(0);
            hook(j);
            // next tile's operand while this one is in the matrix cores
            if (j + 1 < TN) bn = *reinterpret_cast<const i32x4_t*>(sbb + qswz(32 * (j + 1) + l32, hl));
            // scale the previous tile's sums: acc += (d_x d_w) * S
            if (j > 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[j - 1][r] = __builtin_fmaf(s2[16 * ((j - 1) & 1) + r], (float)cp[r], acc[j - 1][r]);
                asm volatile("" : "+v"(acc[j - 1]));  // done here, not sunk past the staging
            }
            // the d_x d_w tiles of tiles j, j+1 (32x32 outer products, two per MFMA)
            if ((j & 1) == 0) s2 = __builtin_amdgcn_mfma_f32_32x32x1f32(dxa, dwb[j / 2], fzero32, 0, 0, 0);
            cp = cv;
            // keep one tile's sums in flight: hoisting the MFMAs ahead would
            // hold all TN results at once
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[TN - 1][r] = __builtin_fmaf(s2[16 * ((TN - 1) & 1) + r], (float)cp[r], acc[TN - 1][r]);
        asm volatile("" : "+v"(acc[TN - 1]));
    };

    // the group's blocks of stage st, then (Q4_K) the mins term at the end of
    // a super-block, over the tiles of this group's parity
    auto compute = [&](int st, auto pc, int kb, auto hook) {
        constexpr int P_LAST = decltype(pc)::value;
        block(st, g, pc, hook);  // every stage has at least one block pair
#pragma unroll
        for (int k = 1; k < KB; ++k)
            if (k < kb) block(st, 2 * k + g, pc, [](int) {});
        if constexpr (!Q8) {
            if ((SV * (st + 1)) % 256 == 0) {
                const int par = (SV * st / 256) & 1;
                // d_x of this lane's 16 output rows wm + 8q + 4hl + (0..3)
                float dxv[16];
                const float* sdx = reinterpret_cast<const float*>(lds + C::OFF_DX) + P_LAST * SB * Q_BM + wm + 4 * hl;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(sdx + 8 * q);
                    dxv[4 * q] = v.x; dxv[4 * q + 1] = v.y; dxv[4 * q + 2] = v.z; dxv[4 * q + 3] = v.w;
                }
                const half8_t ax = *reinterpret_cast<const half8_t*>(lds + C::OFF_BSX + par * Q_BM * 32 + qswz(wm + l32, hl));
                const float* sdm = reinterpret_cast<const float*>(lds + C::OFF_DMIN) + par * BN + l32;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if ((j & 1) != g) continue;
                    const half8_t bm = *reinterpret_cast<const half8_t*>(lds + C::OFF_MJ + (par * BN + 32 * j + l32) * 16);
                    const float dm = sdm[32 * j];
                    const f32x16_t cm = __builtin_amdgcn_mfma_f32_32x32x16_f16(ax, bm, fzero, 0, 0, 0);
                    if constexpr (EMIT) {  // summins: an exact integer in f32
                        const int n = n0 + 32 * j + l32;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int m = m0 + wm + 8 * (r >> 2) + 4 * hl + (r & 3);
                            if (m < M && n < N) a.sums[((int64_t)m * N + n) * (K / 256) * 10 + (SV * st / 256) * 10 + 9] = (int32_t)cm[r];
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[j][r] = __builtin_fmaf(-dxv[r] * dm, cm[r], acc[j][r]);
                }
            }
        }
    };

    // The registers hold the stage after the one in LDS: while a stage's first
    // MFMAs run they are written to the idle buffer, one item per MFMA, then
    // the stage after that is loaded, so a load has about a stage of MFMAs to
    // arrive.  Past the end the last stage is restaged into the idle buffer
    // rather than branch.
    const int last = nst - 1;
    load(0);
    store(0, std::integral_constant<int, 0>{});
    load(nst > 1 ? 1 : 0);
    __syncthreads();
    auto iter = [&](int st, auto pc) {
        constexpr int P = decltype(pc)::value;
        const int nx = st + 1 < nst ? st + 1 : last, nx2 = st + 2 < nst ? st + 2 : last;
        compute(st, pc, st == last ? kb_last : KB, [&](int j) {
            // item j after MFMA j; a narrow tile runs the rest after its last MFMA
#pragma unroll
            for (int w = 0; w < NI; ++w)
                if (w == j || (j == TN - 1 && w > j)) store_item(w, nx, std::integral_constant<int, P ^ 1>{});
            if (j == (NI < TN ? NI : TN - 1)) load(nx2);
        });
        __syncthreads();
    };
    int st = 0;
    for (; st + 1 < nst; st += 2) {
        iter(st, std::integral_constant<int, 0>{});
        iter(st + 1, std::integral_constant<int, 1>{});
    }
    if (st < nst) iter(st, std::integral_constant<int, 0>{});

    // group 1 hands its sums to group 0 through LDS, which writes the tile
    float* red = reinterpret_cast<float*>(lds);
    auto crow = [&](int r) { return wm + 8 * (r >> 2) + 4 * hl + (r & 3); };
    if (g == 1) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[crow(r) * BN + 32 * j + l32] = acc[j][r];
    }
    __syncthreads();
    if (g == 0) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + 32 * j + l32;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + crow(r);
                if (m < M && (!EMIT || Y)) Y[(int64_t)m * N + n] = acc[j][r] + red[crow(r) * BN + 32 * j + l32];
            }
        }
    }
}

// ------------------------------------------------------------ launchers ----

// Raises a kernel's dynamic LDS limit to what it needs, once per device.
static void allow_lds_q(const void* k, int bytes)
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

static int cu_count_q()
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

constexpr int Q_KB = 1;  // block pairs per stage: 64 values

struct QTile {
    int mw, tn;
};
// Tiles, (32*MW) x (32*TN): 128 x 224 puts one tile on each of 256 compute
// units on 512 x 14336; 64 x 128 and 64 x 64 (two or more workgroups per
// compute unit) keep narrow or short problems spread out.  (A 32 x 64 tile
// measured slower than 64 x 64 on every shape tried.)
static const QTile kQTiles[] = {{4, 7}, {2, 4}, {2, 2}};

// The tile whose busiest compute unit finishes first: its tiles times a
// tile's area, over the SIMDs its waves keep busy (a tile has 2*MW waves, a
// compute unit 4 SIMDs), weighted by the operand reads per output.
static QTile pick_qtile(int64_t M, int64_t N)
{
    const int64_t cus = cu_count_q();
    QTile best = kQTiles[0];
    double bc = -1.0;
    for (const QTile& t : kQTiles) {
        const int64_t bm = 32 * t.mw, bn = 32 * t.tn;
        const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        const int64_t per_cu = (tiles + cus - 1) / cus;
        const int64_t simds = 2 * t.mw * per_cu < 4 ? 2 * t.mw * per_cu : 4;
        const double cost = (double)per_cu * (double)(bm * bn) / (double)simds * (1.0 + 8.0 / bn + 16.0 / bm);
        if (bc < 0 || cost < bc) {
            bc = cost;
            best = t;
        }
    }
    return best;
}

template <int FMT, int MW, int TN, bool EMIT>
static hipError_t launch_q(QGemmArgs a, hipStream_t s)
{
    using C = QCfg<FMT, MW, TN, Q_KB>;
    const int nm = (a.M + C::Q_BM - 1) / C::Q_BM;
    a.g.t0[0] = 0;
    for (int p = 0; p < PG_MAX; ++p)
        a.g.t0[p + 1] = a.g.t0[p] + (p < a.g.groups ? (a.g.n[p] + C::BN - 1) / C::BN : 0);
    const int64_t grid = (int64_t)nm * a.g.t0[a.g.groups];
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    a.nm = nm;
    a.remap = grid % 8 == 0 ? 1 : 0;
    const void* k = (const void*)gemm_q_kernel<FMT, MW, TN, Q_KB, EMIT>;
    allow_lds_q(k, C::BYTES);
    void* args[] = {&a};
    return hipLaunchKernel(k, dim3((unsigned)grid), dim3(C::Q_NT), args, C::BYTES, s);
}

template <int FMT, bool EMIT>
static hipError_t launch_q_fmt(const QGemmArgs& a, QTile t, hipStream_t s)
{
    if (t.mw == 4) return launch_q<FMT, 4, 7, EMIT>(a, s);
    if (t.tn == 4) return launch_q<FMT, 2, 4, EMIT>(a, s);
    return launch_q<FMT, 2, 2, EMIT>(a, s);
}

// Q4_K traced runs: sumi = sum_j sc_j S_j of every super-block, from the S_j
// the prefill kernel wrote and the weights' 6-bit scales (the kernel itself
// scales each S_j in f32 and never forms sumi).
__global__ __launch_bounds__(256) void q4k_sumi_kernel(const uint8_t* __restrict__ w, int64_t N, int K, int M,
                                                       int32_t* __restrict__ sums)
{
    const int nsb = K / 256;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (m, n, super-block)
    if (i >= (int64_t)M * N * nsb) return;
    const int64_t mn = i / nsb;
    const int sb = (int)(i - mn * nsb);
    const int64_t n = mn % N;
    const uint32_t* h = reinterpret_cast<const uint32_t*>(w + (n * nsb + sb) * 144);
    int32_t* o = sums + i * 10;
    int si = 0;
    for (int j = 0; j < 8; ++j) {
        int sc, mn_;
        q4k_scale_min(h[1], h[2], h[3], j, sc, mn_);
        si += sc * o[j];
    }
    o[8] = si;
}

hipError_t launch_gemm_q_group(int fmt, int count, const void* const* w, const int64_t* Ns, float* const* y,
                               int64_t K, int64_t M, const GemmBufs& b, hipStream_t s, int32_t* sums)
{
    if (count < 1 || count > PG_MAX || (sums && count != 1)) return hipErrorInvalidValue;
    QGemmArgs a{};
    int64_t ntot = 0;
    for (int p = 0; p < count; ++p) {
        a.g.w[p] = (const uint8_t*)w[p];
        a.g.y[p] = y[p];
        a.g.n[p] = (int)Ns[p];
        ntot += Ns[p];
    }
    a.g.groups = count;
    a.row_bytes = fmt == FMT_Q8_0 ? (K / 32) * 34 : (K / 256) * 144;
    a.K = (int)K;
    a.M = (int)M;
    a.q = (const int8_t*)b.a0;
    a.dx = b.sd;
    a.bsx = b.xs;
    a.sums = sums;
    const QTile t = pick_qtile(M, ntot);
    const bool emit = sums != nullptr;
    hipError_t e;
    if (fmt == FMT_Q8_0) e = emit ? launch_q_fmt<FMT_Q8_0, true>(a, t, s) : launch_q_fmt<FMT_Q8_0, false>(a, t, s);
    else e = emit ? launch_q_fmt<FMT_Q4_K, true>(a, t, s) : launch_q_fmt<FMT_Q4_K, false>(a, t, s);
    if (e != hipSuccess) return e;
    if (emit && fmt == FMT_Q4_K) {
        const int64_t items = M * Ns[0] * (K / 256);
        hipLaunchKernelGGL(q4k_sumi_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, (const uint8_t*)w[0],
                           Ns[0], (int)K, (int)M, sums);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_q(int fmt, const void* w, int64_t N, int64_t K, int64_t M, const GemmBufs& b, float* y,
                         hipStream_t s, int32_t* sums)
{
    return launch_gemm_q_group(fmt, 1, &w, &N, &y, K, M, b, s, sums);
}

}  // namespace qmm
