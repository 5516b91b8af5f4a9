// qmm_gemv_kernel.h -- the decode kernel (M <= 8) for y = x . W^T on GGUF blocks,
// included by the sources that instantiate it (qmm_gemv.hip: mode (a) and the
// launchers; qmm_gemv_b.hip: mode (b); qmm_gemv_emit.hip: mode (b) with its
// integer sums written out).
//
// The weight stream is the cost (the pages' CPU decode step is dominated by
// it: page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 修法, 7 ms
// Q8_0 vs 15 ms dequantized f32).  Layout of the work:
//   * a wave owns 16 weight rows (one matrix-core tile) and one slice of K,
//     streamed in stages of P load units (Q8_0 block pairs or Q4_K
//     super-blocks).  A stage is read row by row in 16-byte chunks, so four
//     consecutive lanes always read 64 consecutive bytes of one row (loads
//     whose lane quads span several rows run at half the rate), two stages in
//     flight;
//   * each stage lands in a small per-wave LDS buffer, from which every lane
//     gathers its matrix-core operand (lane l: row l%16, k-group l/16);
//   * the activation operand is built once per workgroup, in LDS, in operand
//     order; lanes whose operand rows are structurally zero (the two-block
//     trick below, or activation rows >= M) mask their 16 bytes to zero;
//   * the eight waves of a workgroup split each tile's K range among
//     themselves (kw waves per tile) and sum their partials through LDS once at
//     the end, so no second kernel is needed unless the activation operand
//     exceeds LDS (then K is also split across workgroups and a small kernel
//     adds the partials in a fixed order);
//   * mode (a): v_mfma_f32_16x16x32_f16 with the weights as exact f16 integers
//     (q for Q8_0, the 4-bit q for Q4_K) against activation rows 0..7 = f16 hi
//     part and rows 8..15 = f16 lo part of x*2^e;
//   * mode (b): v_mfma_i32_16x16x64_i8 over two 32-value (sub-)blocks at once
//     (A rows 0..7 carry the first, 8..15 the second, zeros elsewhere), giving
//     the int32 block sums; scaled in f32 (Q8_0: dw*dx*S; Q4_K: sub-block
//     scales in int32, then dx*(d*sumi - dmin*summins)).
#pragma once
#include <algorithm>

#include "qmm_act.h"

namespace qmm {

constexpr int GV_WAVES = 8;
constexpr int GV_THREADS = 64 * GV_WAVES;
constexpr int GV_XMAX = 64 * GV_THREADS;  // activation values one workgroup prepares (64 per thread)
constexpr int GV_GPW_MAX = 16;            // tile groups per workgroup
constexpr int GV_RED = 128;               // floats per (tile, slice) partial: 8 rows x 16 columns
constexpr int GV_RED_BYTES = GV_WAVES * GV_RED * 4;  // partials of one tile group
constexpr int GV_MISC_BYTES = 128;
constexpr int GV_LDS_MAX = 160 * 1024;

// Per format and mode: bytes per load unit and row (a Q8_0 block pair or a
// Q4_K super-block), matrix-core steps per load unit, activation values per
// unit; per activation-row slot count MS (1 when M == 1, else 8): image
// bytes per matrix-core step and scale bytes per load unit.
template <int FMT, int MODE, int MS>
struct GvFmt {
    static constexpr int LUB = FMT == FMT_Q8_0 ? 68 : 144;
    static constexpr int OPS = FMT == FMT_Q8_0 ? (MODE == MODE_A ? 2 : 1) : (MODE == MODE_A ? 8 : 4);
    static constexpr int VPL = FMT == FMT_Q8_0 ? 64 : 256;
    // one zero slot closes each matrix-core step when some lanes' operand rows are
    // structurally zero (mode b's two-block trick, and M == 1): those lanes read it
    static constexpr int ZS = MODE == MODE_B || MS == 1 ? 16 : 0;
    static constexpr int OPB = (MODE == MODE_A ? 128 : 64) * MS + ZS;
    static constexpr int SCB = FMT == FMT_Q8_0 ? (MODE == MODE_A ? 0 : 8 * MS) : (MODE == MODE_A ? 64 * MS : 36 * MS);
};

static inline void gv_fmt(int fmt, int mode, int ms, int& lub, int& ops, int& vpl, int& opb, int& scb)
{
    lub = fmt == FMT_Q8_0 ? 68 : 144;
    ops = fmt == FMT_Q8_0 ? (mode == MODE_A ? 2 : 1) : (mode == MODE_A ? 8 : 4);
    vpl = fmt == FMT_Q8_0 ? 64 : 256;
    opb = (mode == MODE_A ? 128 : 64) * ms + (mode == MODE_B || ms == 1 ? 16 : 0);
    scb = fmt == FMT_Q8_0 ? (mode == MODE_A ? 0 : 8 * ms) : (mode == MODE_A ? 64 * ms : 36 * ms);
}

// 16-byte chunks per row in a stage of P load units (the last may run past
// the stage: those bytes are read but not used).
constexpr int gv_cpr(int fmt, int P) { return fmt == FMT_Q8_0 ? (68 * P + 15) / 16 : 9 * P; }
constexpr bool gv_ring_ok(int fmt, int P) { return (gv_cpr(fmt, P) & 1) == 1; }
constexpr int kRingMax = 3;  // LDS-direct stage buffers per wave at most (4 measured slower)
constexpr int kRingMin = 2;  // fewer than this fit: register staging
// LDS row stride of the stage buffer: an odd number of 16-byte units, so the
// 16 rows a wave gathers from start in different banks.
constexpr int gv_rs(int fmt, int P) { return 16 * (gv_cpr(fmt, P) | 1); }

struct GemvArgs {
    const uint8_t* w;
    int64_t w_bytes;  // N * row_bytes
    int row_bytes;
    int N, K, M;
    int nlu;          // load units per row
    int lus_split;    // load units per K split
    int ks;           // K splits (across workgroups)
    int kw;           // waves per tile (K slices inside the workgroup)
    int slice;        // load units per wave slice (a multiple of the stage size)
    int G;            // tiles per workgroup step (GV_WAVES / kw)
    int groups;       // tile groups per split
    int gpw;          // tile groups per workgroup
    int sc_off, red_off, misc_off, stg_off;  // LDS byte offsets
    const float* x;
    float* part;
    float* y;          // EMIT instances: may be null (only the integer parts are wanted)
    int32_t* sums;     // EMIT: integer block sums [M][N][per row]
    uint8_t* act;      // EMIT: canonical quantized activation blocks [M][row bytes], or null
};

QMM_DEV u32x4_t ld128(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
QMM_DEV float4 ldx16(rsrc_t r, uint32_t off)
{
    const f32x4_t v = __builtin_bit_cast(f32x4_t, ld128(r, off));
    return make_float4(v[0], v[1], v[2], v[3]);
}

// Eight int8 (two dwords) -> eight exact f16 in order.
QMM_DEV half8_t i8x8_to_f16(uint32_t d0, uint32_t d1)
{
    uint32_t a0, a1, b0, b1;
    i8x4_to_f16(d0, a0, a1);
    i8x4_to_f16(d1, b0, b1);
    return __builtin_bit_cast(half8_t, u32x4_t{a0, a1, b0, b1});
}

QMM_DEV void st16(uint8_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    *reinterpret_cast<u32x4_t*>(p) = u32x4_t{a, b, c, d};
}
QMM_DEV uint32_t lds32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
QMM_DEV u32x2_t lds64(const uint8_t* p) { return *reinterpret_cast<const u32x2_t*>(p); }
QMM_DEV u32x4_t lds128(const uint8_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Workgroup counters in LDS that let some waves wait for others without a
// full barrier (waves still queueing weight loads do not hold the rest up).
// The wait is bounded, so a wave can never spin forever.
QMM_DEV void wg_signal(int* c, bool release)
{
    if (release) __hip_atomic_fetch_add(c, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    else __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// The counters and the data they guard are in LDS, whose reads a wave performs
// in order, and the signalling wave's LDS writes are complete before its
// release add: a relaxed read plus a compiler barrier orders the reads after
// the wait.  (An acquire read would also wait for every outstanding global
// load, the weight stream's prefetch included.)
QMM_DEV void wg_wait(int* c, int target)
{
    for (int spin = 0; spin < (1 << 22); ++spin) {
        if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// 16 bytes per lane from the buffer at voff into LDS at dst + 16 * lane (dst wave-uniform)
QMM_DEV void ld128_lds(rsrc_t r, uint8_t* dst, uint32_t voff)
{
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, voff, 0, 0, 0);
}

// R: activation rows per lane the arithmetic covers (1 when M == 1, else 4:
// lane l holds output rows 4*(l/16 % 2) + r of its tile column l%16).
// D: 0 = each stage is loaded into registers (two stages in flight) and
// written to one LDS buffer per wave; D >= 2 = a ring of D stage buffers per
// wave filled by 16-byte loads that write LDS directly (lane i of a load lands
// at its base + 16 i, so the stage keeps the row-major chunk layout), D
// stages in flight and no registers or LDS writes spent on the stream.
template <int FMT, int MODE, int P, int R, bool EMIT, int D>
__global__ __launch_bounds__(GV_THREADS, 4) void gemv_kernel(GemvArgs a)
{
    constexpr int MS = R == 1 ? 1 : 8;
    using F = GvFmt<FMT, MODE, MS>;
    constexpr int LUB = F::LUB, OPS = F::OPS, VPL = F::VPL, OPB = F::OPB, SCB = F::SCB;
    constexpr int CPR = gv_cpr(FMT, P), RS = gv_rs(FMT, P);
    constexpr int T = (16 * CPR + 63) / 64;  // load instructions per stage
    static_assert(D == 0 || (D >= 2 && (D - 1) * T <= 63), "ring of LDS-direct stages");
    constexpr int RSW = D > 0 ? 16 * CPR : RS;  // stage row stride in LDS (direct loads: unpadded)
    constexpr int SBY = 16 * RSW;               // bytes of one stage buffer
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t* s_img = lds;
    float* s_scf = reinterpret_cast<float*>(lds + a.sc_off);
    int32_t* s_sci = reinterpret_cast<int32_t*>(lds + a.sc_off);
    float* s_red = reinterpret_cast<float*>(lds + a.red_off);
    float* s_misc = reinterpret_cast<float*>(lds + a.misc_off);  // mode a: [0,8) 2^e, [8,16) 2^-e, [16,24) amax

    const int M = a.M, N = a.N, K = a.K;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int split = blockIdx.x % a.ks, wgi = blockIdx.x / a.ks;
    const int lu_beg = split * a.lus_split;
    const int lu_cnt = min(a.lus_split, a.nlu - lu_beg);  // real load units of this split
    const int tg = wave / a.kw, sl = wave - tg * a.kw;
    const int grp0 = wgi * a.gpw;
    const int ngrp = min(a.gpw, a.groups - grp0);
    const int sl_lu0 = sl * a.slice;                          // first unit of this wave's slice
    const int sl_real = max(0, min(a.slice, lu_cnt - sl_lu0));
    // every wave runs S stages per tile, so the waves reach each tile's end together;
    // the stages of a short last slice past its real units load nothing
    const int S = a.slice / P;
    const int S_real = (sl_real + P - 1) / P;
    const int Q = ngrp * S;                                   // stages per wave
    uint8_t* stg = lds + a.stg_off + wave * ((D > 0 ? D : 1) * SBY);

    // ---- the weight stream: chunk f = 64t + lane of a stage is row f/CPR, chunk f%CPR ----
    uint32_t go[T], lw[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int f = 64 * t + lane, r = f / CPR, c = f - r * CPR;
        go[t] = f < 16 * CPR ? (uint32_t)(r * a.row_bytes + 16 * c) : 0x80000000u;
        lw[t] = (uint32_t)(r * RS + 16 * c);
    }
    constexpr int TAIL = 16 * CPR - 64 * (T - 1);  // live lanes of the last load

    int iq = 0, iu = 0, is = 0;  // next stage to queue: index, tile, stage within the tile
    // the next stage's source: the tile's rows as a buffer (rows past N, and stages
    // past the wave's real units, read as zero) and the stage's byte offset in a row
    auto next_src = [&](rsrc_t& wr, uint32_t& so) {
        const bool real = iq < Q && is < S_real;
        const int tile = (grp0 + iu) * a.G + tg;
        const int64_t t0 = (int64_t)tile * 16 * a.row_bytes;
        const int64_t left = a.w_bytes - t0;
        const uint32_t nrec = real && left > 0 ? (uint32_t)min(left, (int64_t)16 * a.row_bytes) : 0u;
        wr = make_rsrc(a.w + (real ? t0 : 0), nrec);
        so = (uint32_t)((lu_beg + sl_lu0 + is * P) * LUB);
        ++iq;
        if (++is == S) { is = 0; ++iu; }
    };
    auto issue = [&](u32x4_t (&r)[T]) {
        rsrc_t wr;
        uint32_t so;
        next_src(wr, so);
#pragma unroll
        for (int t = 0; t < T; ++t) r[t] = ld128(wr, go[t] + so);
    };
    // LDS-direct form: the next stage into ring buffer `slot` (lanes past the
    // stage's last chunk stay off, so nothing lands beyond the buffer)
    auto issue_lds = [&](int slot) {
        rsrc_t wr;
        uint32_t so;
        next_src(wr, so);
        uint8_t* buf = stg + slot * SBY;
#pragma unroll
        for (int t = 0; t < T; ++t)
            if (t < T - 1 || lane < TAIL)
                ld128_lds(wr, buf + 1024 * t, go[t] + so);
    };
    u32x4_t rA[D > 0 ? 1 : T], rB[D > 0 ? 1 : T];
    // the first stages of the stream: two into registers, or the whole ring
    auto prime = [&]() {
        if constexpr (D > 0) {
#pragma unroll
            for (int i = 0; i < D; ++i)
                if (iq < Q) issue_lds(i);
        } else {
            issue(rA);
            issue(rB);
        }
    };

    // ---- the activation operand of this K split, once per workgroup ----
    // Each task fills one 16-byte operand slot (mode b: 16 int8 of one half of a
    // (sub-)block; mode a: 8 values of one k-group as f16 hi and lo) from exactly
    // the x values that slot holds, in slot order; the lanes of one block meet
    // through shuffles for its scale.  Waves with no task queue their weight
    // stages at once; the others after their slots are written.
    constexpr int VT = MODE == MODE_A ? 8 : 16;   // x values per task
    constexpr int NTPT = MODE == MODE_A ? 8 : 4;  // tasks per thread at most (64 values)
    const int nb32 = lu_cnt * (VPL / 32);         // 32-value blocks in this split
    const int ntasks = MODE == MODE_A ? M * nb32 * 4 : (FMT == FMT_Q8_0 ? M * nb32 * 2 : M * lu_cnt * 16);
    // mode (a) with eight rows: wave w takes row w whole (tasks lane, lane + 64, ...),
    // so each row's maximum is a reduction inside one wave; otherwise task t =
    // tid + 512 c, the waves sharing rows and the maxima meeting in LDS
    const int per_row = ntasks / M;
    const bool wrow = MODE == MODE_A && M == GV_WAVES && per_row <= 64 * NTPT;
    const int npw = wrow ? GV_WAVES : min(GV_WAVES, (ntasks + 63) / 64);  // waves with tasks (the first npw)
    const bool xw = wave < npw;
    // task c of this thread: its row m, its index r in the row, and whether it exists
    auto task = [&](int c, int& m, int& r, bool& live) {
        if (wrow) {
            m = wave;
            r = lane + 64 * c;
            live = r < per_row;
        } else {
            const int t = tid + GV_THREADS * c;
            live = t < ntasks;
            m = t / per_row;
            r = t - m * per_row;
        }
    };
    // whether this wave has a task c at all (uniform per wave)
    auto has_task = [&](int c) { return wrow ? 64 * c < per_row : 64 * wave + GV_THREADS * c < ntasks; };
    int* s_sync = reinterpret_cast<int*>(s_misc) + 24;  // row maxima in, operand ready
    const rsrc_t xr = make_rsrc(a.x, (uint32_t)(M * K * 4));
    const int k0 = lu_beg * VPL;
    float xv[NTPT][VT];
    if (xw) {
#pragma unroll
        for (int c = 0; c < NTPT; ++c) {
            if (!has_task(c)) break;
            int m, r;
            bool live;
            task(c, m, r, live);
            uint32_t o[4];  // float offsets of the slot's values: 4 + 4 + 4 + 4, or 4 + 2 + 2 (mode a)
            if constexpr (MODE == MODE_A) {
                const int b = r >> 2, kg = r & 3;
                const int base = m * K + k0 + 32 * b;
                int o0 = 8 * kg, o2 = 8 * kg + 6;
                if (FMT == FMT_Q8_0 && !(b & 1)) {  // even block: q[2+8kg ..]; group 3: q26..q31, q0, q1
                    o0 = kg < 3 ? 2 + 8 * kg : 26;
                    o2 = kg < 3 ? o0 + 6 : 0;
                }
                o[0] = base + o0; o[1] = base + o0 + 4; o[2] = base + o2; o[3] = 0;
            } else if constexpr (FMT == FMT_Q8_0) {
                const int b = r >> 1, h = r & 1;
                const int base = m * K + k0 + 32 * b;
                // even block: half 0 = q2..q17, half 1 = q18..q31, q0, q1; odd block: natural
                const int s0 = (b & 1) ? 16 * h : 2 + 16 * h;
                o[0] = base + s0; o[1] = base + s0 + 4; o[2] = base + s0 + 8;
                o[3] = base + ((b & 1) || !h ? s0 + 12 : 28);  // 4 values; the last 2 of half 1 (even) wrap
            } else {
                const int sb = r >> 4, sl16 = r & 15;
                const int base = m * K + k0 + 256 * sb + 16 * sl16;
                o[0] = base; o[1] = base + 4; o[2] = base + 8; o[3] = base + 12;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = live ? o[i] * 4 : 0x80000000u;
            if constexpr (MODE == MODE_A) {
                const float4 v0 = ldx16(xr, o[0]);
                const u32x2_t v1 = __builtin_amdgcn_raw_buffer_load_b64(xr, o[1], 0, 0);
                const u32x2_t v2 = __builtin_amdgcn_raw_buffer_load_b64(xr, o[2], 0, 0);
                xv[c][0] = v0.x; xv[c][1] = v0.y; xv[c][2] = v0.z; xv[c][3] = v0.w;
                xv[c][4] = __uint_as_float(v1[0]); xv[c][5] = __uint_as_float(v1[1]);
                xv[c][6] = __uint_as_float(v2[0]); xv[c][7] = __uint_as_float(v2[1]);
            } else {
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const float4 v = ldx16(xr, o[i]);
                    xv[c][4 * i] = v.x; xv[c][4 * i + 1] = v.y; xv[c][4 * i + 2] = v.z; xv[c][4 * i + 3] = v.w;
                }
                if constexpr (FMT == FMT_Q8_0) {
                    // last 4 values: the slot's q12..q15 (halves of odd blocks, half 0 of even
                    // blocks) or q30, q31, q0, q1 (half 1 of an even block)
                    const int r2 = r & 3;  // (b & 1) << 1 | h
                    const bool wrap = r2 == 1;
                    const u32x2_t lo = __builtin_amdgcn_raw_buffer_load_b64(xr, wrap ? o[3] + 8 : o[3], 0, 0);
                    const u32x2_t hi2 = __builtin_amdgcn_raw_buffer_load_b64(
                        xr, wrap ? (live ? (uint32_t)(m * K + k0 + 32 * (r >> 1)) * 4 : 0x80000000u)
                                 : o[3] + 8, 0, 0);
                    xv[c][12] = __uint_as_float(lo[0]); xv[c][13] = __uint_as_float(lo[1]);
                    xv[c][14] = __uint_as_float(hi2[0]); xv[c][15] = __uint_as_float(hi2[1]);
                } else {
                    const float4 v = ldx16(xr, o[3]);
                    xv[c][12] = v.x; xv[c][13] = v.y; xv[c][14] = v.z; xv[c][15] = v.w;
                }
            }
        }
    }
    // the barrier orders every x load before any weight load, so x is not stuck behind the stream
    if (tid < GV_MISC_BYTES / 4) s_misc[tid] = 0.0f;
    __syncthreads();
    if (xw) {
        // zero what the slices may read past the split's last unit, and the partials
        const u32x4_t z = {0u, 0u, 0u, 0u};
        const int lu_img = a.kw * a.slice, pthreads = 64 * npw;
        for (int i = lu_cnt * OPS * OPB / 16 + tid; i < lu_img * OPS * OPB / 16; i += pthreads)
            reinterpret_cast<u32x4_t*>(s_img)[i] = z;
        if constexpr (SCB > 0)
            for (int i = lu_cnt * SCB / 4 + tid; i < lu_img * SCB / 4; i += pthreads) s_sci[i] = 0;
        for (int i = tid; i < GV_RED_BYTES / 16; i += pthreads) reinterpret_cast<u32x4_t*>(s_red)[i] = z;
        if constexpr (F::ZS > 0) {
            for (int i = tid; i < lu_cnt * OPS; i += pthreads) *reinterpret_cast<u32x4_t*>(s_img + i * OPB + OPB - 16) = z;
        } else if (M < MS) {  // mode (a), 2 <= M < 8: the slots of rows M..7 read as zero
            const int dead = MS - M;
            for (int i = tid; i < lu_cnt * OPS * 8 * dead; i += pthreads) {
                const int st = i / (8 * dead), rem = i - st * 8 * dead, sl = rem / dead, m = M + (rem - sl * dead);
                *reinterpret_cast<u32x4_t*>(s_img + st * OPB + (sl * MS + m) * 16) = z;
            }
        }
    } else {
        prime();
    }
    float wmax = 0.0f;  // wave-per-row form: this wave's row maximum
    if constexpr (MODE == MODE_A) {
        // power-of-two scale per row over this split, then the hi/lo f16 split; a wave
        // whose tasks share a row reduces its maximum first (one LDS atomic per wave)
        if (xw && wrow) {
            // (tasks past the row are zeros: they leave the maximum unchanged)
#pragma unroll
            for (int c = 0; c < NTPT; ++c) {
                if (!has_task(c)) break;
#pragma unroll
                for (int i = 0; i < 8; ++i) wmax = fmaxf(wmax, fabsf(xv[c][i]));
            }
            wmax = wave_max(wmax);
            if (lane == 0) s_misc[16 + wave] = wmax;  // for the outputs' 2^-e
        } else if (xw) {
#pragma unroll
            for (int c = 0; c < NTPT; ++c) {
                if (64 * wave + GV_THREADS * c >= ntasks) break;
                const int t = tid + GV_THREADS * c, t0 = 64 * wave + GV_THREADS * c;
                float am = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(xv[c][i]));
                const int m0 = t0 / per_row;
                if (min(t0 + 63, ntasks - 1) / per_row == m0) {
                    am = wave_max(am);
                    if (lane == 0) atomicMax(reinterpret_cast<unsigned*>(&s_misc[16 + m0]), __float_as_uint(am));
                } else if (t < ntasks) {
                    atomicMax(reinterpret_cast<unsigned*>(&s_misc[16 + t / per_row]), __float_as_uint(am));
                }
            }
            if (lane == 0) wg_signal(&s_sync[1], true);
            wg_wait(&s_sync[1], npw);
        }
    }
    if (xw) {
#pragma unroll
        for (int c = 0; c < NTPT; ++c) {
            if (!has_task(c)) break;
            int m, r;
            bool live;
            task(c, m, r, live);
            if constexpr (MODE == MODE_A) {
                const int b = r >> 2, kg = r & 3;
                const float rmax = wrow ? wmax : __uint_as_float(reinterpret_cast<const unsigned*>(s_misc)[16 + (live ? m : 0)]);
                const float sc = ldexpf(1.0f, split_exp(rmax));
                half8_t vh, vl;
                float sum = 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    // Q4_K: the nibble decoder yields k-group elements in order {0,2,1,3,4,6,5,7}
                    const int k = FMT == FMT_Q4_K ? nib_perm(u) : u;
                    _Float16 h, l;
                    float xs;
                    split_one(xv[c][k], sc, h, l, xs);
                    vh[u] = h;
                    vl[u] = l;
                    sum += xs;
                }
                if (live) {
                    uint8_t* op = s_img + b * OPB;
                    *reinterpret_cast<half8_t*>(op + ((kg * 2) * MS + m) * 16) = vh;
                    *reinterpret_cast<half8_t*>(op + ((kg * 2 + 1) * MS + m) * 16) = vl;
                }
                if constexpr (FMT == FMT_Q4_K) {  // mins term: sum of x*2^e over the 32 values (hi rows)
                    sum += dpp_f<DPP_X1>(sum);
                    sum += dpp_f<DPP_X2>(sum);
                    if (live && kg == 0) {
                        s_scf[b * 2 * MS + m] = sum;
                        s_scf[b * 2 * MS + MS + m] = 0.0f;
                    }
                }
            } else if constexpr (FMT == FMT_Q8_0) {
                const int b = r >> 1, h = r & 1;
                float am = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(xv[c][i]));
                am = fmaxf(am, dpp_f<DPP_X1>(am));  // the block's other half
                float id, dval;
                uint16_t dbits;
                q8_0_scale(am, id, dbits, dval);
                int q[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) q[i] = q8_0_q(xv[c][i], id);
                if (live) {
                    const int par = b & 1;
                    *reinterpret_cast<u32x4_t*>(s_img + (b >> 1) * OPB + ((par * 2 + h) * MS + m) * 16) =
                        u32x4_t{pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]),
                                pack4(q[8], q[9], q[10], q[11]), pack4(q[12], q[13], q[14], q[15])};
                    if (h == 0) s_scf[(b >> 1) * 2 * MS + par * MS + m] = dval;
                    if (EMIT && a.act && wgi == 0) {
                        // canonical block: the slot's values are elements s0.. of the block, or
                        // for half 1 of an even block 18..31 then 0, 1
                        uint8_t* o = a.act + ((int64_t)m * (K / 32) + 2 * lu_beg + b) * 34;
                        if (h == 0) *reinterpret_cast<uint16_t*>(o) = dbits;
                        const int s0 = (b & 1) ? 16 * h : 2 + 16 * h;
#pragma unroll
                        for (int i = 0; i < 16; ++i) o[2 + (s0 + i) % 32] = (uint8_t)q[i];
                    }
                }
            } else {
                const int sb = r >> 4, sl16 = r & 15;
                // the super-block's signed element of largest |x|, first index on ties:
                // this lane's first element of largest |x|, then over the 16 lanes
                float best = -1.0f, bv = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float av = fabsf(xv[c][i]);
                    if (av > best) { best = av; bv = xv[c][i]; }
                }
                bv = q8k_row16_max(best, bv, best);
                float iscale, d;
                q8k_scale(bv, best, iscale, d);
                int q[16], s16 = 0;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    q[i] = q8k_q(xv[c][i], iscale);
                    s16 += q[i];
                }
                const int pr = s16 + dpp_i<DPP_X1>(s16);  // the sub-block's two halves
                if (EMIT && a.act && wgi == 0 && live) {  // canonical Q8K block: f32 d, 256 int8, int16 bsums
                    uint8_t* o = a.act + ((int64_t)m * (K / 256) + lu_beg + sb) * 292;
                    if (sl16 == 0) *reinterpret_cast<float*>(o) = d;
                    uint32_t* oq = reinterpret_cast<uint32_t*>(o + 4 + 16 * sl16);
#pragma unroll
                    for (int i = 0; i < 4; ++i) oq[i] = pack4(q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]);
                    reinterpret_cast<int16_t*>(o + 260)[sl16] = (int16_t)s16;
                }
                if (live) {
                    // slot sl16 = sub-block j (two halves); step 2*(j/4) + j%2 holds sub-blocks
                    // (4cc+h) in rows 0..7 and (4cc+2+h) in rows 8..15
                    const int j = sl16 >> 1, half = sl16 & 1;
                    const int isb = (j >> 1) & 1, op = 2 * (j >> 2) + (j & 1);
                    *reinterpret_cast<u32x4_t*>(s_img + (sb * 4 + op) * OPB + ((isb * 2 + half) * MS + m) * 16) =
                        u32x4_t{pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]),
                                pack4(q[8], q[9], q[10], q[11]), pack4(q[12], q[13], q[14], q[15])};
                    if (sl16 == 0) s_scf[sb * 9 * MS + m] = d;
                    if (half == 0) s_sci[sb * 9 * MS + MS + j * MS + m] = pr;
                }
            }
        }
        if (lane == 0) wg_signal(&s_sync[2], true);  // this wave's slots are written
        prime();
    }
    wg_wait(&s_sync[2], npw);  // the whole operand is in place

    // ---- main loop ----
    // activation operand of this lane: its slot, or the step's zero slot for rows that
    // are structurally zero (mode a with M >= 2 zeroes rows M..7 in place instead)
    int aslot;
    {
        const int mrow = n & 7;
        bool alive;
        if constexpr (MODE == MODE_A) {
            aslot = (g * 2 + (n >> 3)) * MS + mrow;
            alive = mrow < M;
        } else {
            aslot = ((g >> 1) * 2 + (g & 1)) * MS + mrow;
            alive = ((n >> 3) == (g >> 1)) && mrow < M;
        }
        if (!alive && F::ZS > 0) aslot = (OPB - 16) / 16;
    }
    const uint8_t* aimg = s_img + aslot * 16;
    const int moff = MS == 8 ? 4 * (g & 1) : 0;  // this lane's first output row within the slots

    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const i32x4_t zi = {0, 0, 0, 0};
    const f32x4_t zf = {0.0f, 0.0f, 0.0f, 0.0f};
    // Q8_0 mode b: k-group 1 completes its 16 bytes with q0, q1 from the pair's first dword
    const uint32_t selp = g == 1 ? 0x07060100u : 0x03020100u;
    // Q8_0 mode a: k-group 3 of the even block takes q30, q31, q0, q1
    const uint32_t sel3 = g == 3 ? 0x07060100u : 0x03020100u;
    const int dsh = g < 2 ? 0 : 16;
    // Q4_K mode a: nibble decode constants, held in registers (opaque to constant folding)
    uint32_t nibm = 0x000f000fu, nibc = 0x64006400u;
    asm volatile("" : "+v"(nibm), "+v"(nibc));


    auto compute = [&](const uint8_t* sbuf, int lu0, int tile) {
        const uint8_t* rrow = sbuf + n * RSW;  // this lane's weight row in the stage buffer
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int lu = lu0 + j;  // load unit within the split
            const uint8_t* rp = rrow + j * LUB;
            if constexpr (FMT == FMT_Q8_0 && MODE == MODE_B) {
                const uint8_t* xp = rp + 4 + 16 * g;
                const uint32_t x0 = lds32(xp), x1 = lds32(xp + 4), x2 = lds32(xp + 8), x3 = lds32(xp + 12);
                const uint32_t E = lds32(rp + (g < 2 ? 0 : 32));
                const uint32_t b3 = __builtin_amdgcn_perm(E, x3, selp);
                const i32x4_t B = {(int)x0, (int)x1, (int)x2, (int)b3};
                const i32x4_t A = __builtin_bit_cast(i32x4_t, lds128(aimg + lu * OPB));
                const i32x4_t C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, zi, 0, 0, 0);
                const float dw = (float)__builtin_bit_cast(_Float16, (uint16_t)(E >> dsh));
                const float* dxp = s_scf + lu * 2 * MS + (g >> 1) * MS + moff;
                if constexpr (R == 1) {
                    acc[0] = fmaf((float)C[0], dw * dxp[0], acc[0]);
                } else {
                    const f32x4_t dx = *reinterpret_cast<const f32x4_t*>(dxp);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[q] = fmaf((float)C[q], dw * dx[q], acc[q]);
                }
                if constexpr (EMIT) {
                    const int ng = tile * 16 + n, blk = 2 * (lu_beg + lu) + (g >> 1);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int m = 4 * (g & 1) + q;
                        // (a stage may run past the split's last unit: those units are not the row's)
                        if (m < M && ng < N && lu < lu_cnt) a.sums[((int64_t)m * N + ng) * (2 * a.nlu) + blk] = C[q];
                    }
                }
            } else if constexpr (FMT == FMT_Q8_0) {
                const uint32_t E0 = lds32(rp), E8 = lds32(rp + 32);
                const uint8_t* xe = rp + 4 + 8 * g;
                const uint8_t* xo = rp + 36 + 8 * g;
                const half8_t Be = i8x8_to_f16(lds32(xe), __builtin_amdgcn_perm(E0, lds32(xe + 4), sel3));
                const half8_t Bo = i8x8_to_f16(lds32(xo), lds32(xo + 4));
                const half8_t Ae = __builtin_bit_cast(half8_t, lds128(aimg + (2 * lu) * OPB));
                const half8_t Ao = __builtin_bit_cast(half8_t, lds128(aimg + (2 * lu + 1) * OPB));
                const f32x4_t Ce = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, Be, zf, 0, 0, 0);
                const f32x4_t Co = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, Bo, zf, 0, 0, 0);
                const float de = f16lo(E0), dd = f16hi(E8);
#pragma unroll
                for (int q = 0; q < R; ++q) acc[q] = fmaf(Co[q], dd, fmaf(Ce[q], de, acc[q]));
            } else if constexpr (MODE == MODE_B) {
                const u32x4_t H = lds128(rp);
                const int ssh = 16 * (g >> 1);  // this lane's sub-blocks: j0 + {0, 1, 4, 5}, j0 = 2*(g>>1)
                const uint32_t sa = H[1] >> ssh, sb_ = H[2] >> ssh, sc_ = H[3] >> ssh;
                const uint32_t sc_lo = sa & 0x3f3fu, mn_lo = sb_ & 0x3f3fu;
                const uint32_t sc_hi = (sc_ & 0x0f0fu) | ((sa >> 2) & 0x3030u);
                const uint32_t mn_hi = ((sc_ >> 4) & 0x0f0fu) | ((sb_ >> 2) & 0x3030u);
                i32x4_t sumi = zi;
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const u32x4_t Qv = lds128(rp + 16 * (1 + 4 * cc + g));
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const i32x4_t B = {(int)((Qv[0] >> (4 * h)) & 0x0f0f0f0fu), (int)((Qv[1] >> (4 * h)) & 0x0f0f0f0fu),
                                           (int)((Qv[2] >> (4 * h)) & 0x0f0f0f0fu), (int)((Qv[3] >> (4 * h)) & 0x0f0f0f0fu)};
                        const i32x4_t A = __builtin_bit_cast(i32x4_t, lds128(aimg + (lu * 4 + 2 * cc + h) * OPB));
                        const i32x4_t C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, zi, 0, 0, 0);
                        const int scj = (int)(((cc ? sc_hi : sc_lo) >> (8 * h)) & 0xffu);
#pragma unroll
                        for (int q = 0; q < R; ++q) sumi[q] += scj * C[q];
                        if constexpr (EMIT) {
                            const int ng = tile * 16 + n, jj = 2 * (g >> 1) + 4 * cc + h;
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int m = 4 * (g & 1) + q;
                                if (m < M && ng < N && lu < lu_cnt)
                                    a.sums[(((int64_t)m * N + ng) * a.nlu + lu_beg + lu) * 10 + jj] = C[q];
                            }
                        }
                    }
                }
                const int mn0 = mn_lo & 0xff, mn1 = (mn_lo >> 8) & 0xff, mn4 = mn_hi & 0xff, mn5 = (mn_hi >> 8) & 0xff;
                const int32_t* bsp = s_sci + lu * 9 * MS + MS + 2 * (g >> 1) * MS + moff;
                const float* dqp = s_scf + lu * 9 * MS + moff;
                const float d = f16lo(H[0]), dmin = f16hi(H[0]);
                i32x4_t summ = zi;
                if constexpr (R == 1) {
                    summ[0] = mn0 * bsp[0] + mn1 * bsp[MS] + mn4 * bsp[4 * MS] + mn5 * bsp[5 * MS];
                    acc[0] = fmaf(dqp[0], d * (float)sumi[0] - dmin * (float)summ[0], acc[0]);
                } else {
                    const i32x4_t b0 = *reinterpret_cast<const i32x4_t*>(bsp);
                    const i32x4_t b1 = *reinterpret_cast<const i32x4_t*>(bsp + MS);
                    const i32x4_t b4 = *reinterpret_cast<const i32x4_t*>(bsp + 4 * MS);
                    const i32x4_t b5 = *reinterpret_cast<const i32x4_t*>(bsp + 5 * MS);
                    const f32x4_t dq = *reinterpret_cast<const f32x4_t*>(dqp);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        summ[q] = mn0 * b0[q] + mn1 * b1[q] + mn4 * b4[q] + mn5 * b5[q];
                        acc[q] = fmaf(dq[q], d * (float)sumi[q] - dmin * (float)summ[q], acc[q]);
                    }
                }
                if constexpr (EMIT) {
                    const int ng = tile * 16 + n;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int ti = sumi[q] + __shfl_xor(sumi[q], 32);
                        const int tm = summ[q] + __shfl_xor(summ[q], 32);
                        const int m = 4 * (g & 1) + q;
                        if (g < 2 && m < M && ng < N && lu < lu_cnt) {
                            int32_t* o = a.sums + (((int64_t)m * N + ng) * a.nlu + lu_beg + lu) * 10;
                            o[8] = ti;
                            o[9] = tm;
                        }
                    }
                }
            } else {
                const u32x4_t H = lds128(rp);
                const float d = f16lo(H[0]), dmin = f16hi(H[0]);
                const uint32_t s0 = H[1], s1 = H[2], s2 = H[3];
                const uint32_t sc4[2] = {s0 & 0x3f3f3f3fu, (s2 & 0x0f0f0f0fu) | ((s0 >> 2) & 0x30303030u)};
                const uint32_t mn4[2] = {s1 & 0x3f3f3f3fu, ((s2 >> 4) & 0x0f0f0f0fu) | ((s1 >> 2) & 0x30303030u)};
                const float* xsp = s_scf + (lu * 8) * 2 * MS + (g >> 1) * MS + moff;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x2_t Qv = lds64(rp + 16 + 32 * c + 8 * g);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int jj = 2 * c + h;
                        const half8_t B = nib8_to_f16(Qv[0], Qv[1], 4 * h, nibm, nibc);
                        const half8_t A = __builtin_bit_cast(half8_t, lds128(aimg + (lu * 8 + jj) * OPB));
                        const f32x4_t C = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, zf, 0, 0, 0);
                        const float dsc = d * (float)((sc4[jj >> 2] >> (8 * (jj & 3))) & 0xffu);
                        const float dmm = dmin * (float)((mn4[jj >> 2] >> (8 * (jj & 3))) & 0xffu);
                        if constexpr (R == 1) {
                            acc[0] = fmaf(-dmm, xsp[jj * 2 * MS], fmaf(C[0], dsc, acc[0]));
                        } else {
                            const f32x4_t xs = *reinterpret_cast<const f32x4_t*>(xsp + jj * 2 * MS);
#pragma unroll
                            for (int q = 0; q < 4; ++q) acc[q] = fmaf(-dmm, xs[q], fmaf(C[q], dsc, acc[q]));
                        }
                    }
                }
            }
        }
    };

    int cq = 0, cu = 0, cs = 0;  // next stage to compute: index, tile group, stage within the tile
    // computes stage cq from sbuf (r: its registers, to land first) and closes its tile group
    auto consume = [&](const uint8_t* sbuf, const u32x4_t* r) {
        {
            if (cs < S_real) {
                if constexpr (D == 0) {
                    // land the stage in this wave's LDS buffer (the gather below reads other lanes' chunks)
#pragma unroll
                    for (int t = 0; t < T; ++t)
                        if (t < T - 1 || lane < TAIL) *reinterpret_cast<u32x4_t*>(stg + lw[t]) = r[t];
                }
                compute(sbuf, sl_lu0 + cs * P, (grp0 + cu) * a.G + tg);
            }
            if (cs == S - 1) {
                // the tile group is done in every wave: fold the two lane halves, park the
                // partials in LDS, sum the slices, and free the buffer for the next group
                float* red = s_red;
#pragma unroll
                for (int q = 0; q < R; ++q) acc[q] += __shfl_xor(acc[q], 32);
                if (lane < 32) {
                    float* o = red + (tg * a.kw + sl) * GV_RED + 4 * (lane >> 4) * 16 + n;
#pragma unroll
                    for (int q = 0; q < R; ++q) o[16 * q] = acc[q];
                }
                acc = zf;
                __syncthreads();
                if (!EMIT || a.y != nullptr) {
                    const int per = 16 * M;
                    for (int i = tid; i < a.G * per; i += GV_THREADS) {
                        const int t = i / per, rem = i - t * per, m = rem >> 4, nn = rem & 15;
                        const int ng = ((grp0 + cu) * a.G + t) * 16 + nn;
                        if (ng < N) {
                            const float* p = red + t * a.kw * GV_RED + m * 16 + nn;
                            float v = 0.0f;
                            for (int sl2 = 0; sl2 < a.kw; ++sl2) v += p[sl2 * GV_RED];
                            if constexpr (MODE == MODE_A)
                                v *= ldexpf(1.0f, -split_exp(__uint_as_float(reinterpret_cast<const unsigned*>(s_misc)[16 + m])));
                            if (a.ks == 1) a.y[(int64_t)m * N + ng] = v;
                            else a.part[((int64_t)split * GEMV_MAX_M + m) * N + ng] = v;
                        }
                    }
                }
                __syncthreads();
            }
        }
        ++cq;
        if (++cs == S) { cs = 0; ++cu; }
    };
    if constexpr (D == 0) {
        auto step = [&](u32x4_t (&r)[T]) {
            if (cq < Q) {
                consume(stg, r);
            } else {
                ++cq;
                if (++cs == S) { cs = 0; ++cu; }
            }
            issue(r);
        };
        for (int q = 0; q < Q; q += 2) {
            step(rA);
            step(rB);
        }
    } else {
        // stage q sits in ring buffer q % D; once it is consumed, stage q + D takes its place
        int slot = 0;
        for (int q = 0; q < Q; ++q) {
            vm_wait_ahead<T, D - 1>(min(D - 1, Q - 1 - q));  // stage q has landed
            consume(stg + slot * SBY, nullptr);
            if (iq < Q) {
                lgkm_wait0();  // this buffer's reads are done before it is refilled
                issue_lds(slot);
            }
            slot = slot == D - 1 ? 0 : slot + 1;
        }
    }
}

typedef void (*GvKernel)(GemvArgs);

// The instance for a stage size P, rows per lane R and ring depth D (stage
// sizes without the ring map every depth to register staging).
template <int FMT, int MODE, int P, int R, bool EMIT>
GvKernel gv_pick_d(int D)
{
    constexpr bool ok = gv_ring_ok(FMT, P);
    if (D == 3) return gemv_kernel<FMT, MODE, P, R, EMIT, ok ? 3 : 0>;
    if (D == 2) return gemv_kernel<FMT, MODE, P, R, EMIT, ok ? 2 : 0>;
    return gemv_kernel<FMT, MODE, P, R, EMIT, 0>;
}
template <int FMT, int MODE, bool EMIT>
GvKernel gv_pick(int P, int R, int D)
{
    if constexpr (FMT == FMT_Q8_0) {
        if (P == 4) return R == 1 ? gv_pick_d<FMT, MODE, 4, 1, EMIT>(D) : gv_pick_d<FMT, MODE, 4, 4, EMIT>(D);
        if (P == 3) return R == 1 ? gv_pick_d<FMT, MODE, 3, 1, EMIT>(D) : gv_pick_d<FMT, MODE, 3, 4, EMIT>(D);
        if (P == 2) return R == 1 ? gv_pick_d<FMT, MODE, 2, 1, EMIT>(D) : gv_pick_d<FMT, MODE, 2, 4, EMIT>(D);
        return R == 1 ? gv_pick_d<FMT, MODE, 1, 1, EMIT>(D) : gv_pick_d<FMT, MODE, 1, 4, EMIT>(D);
    } else {
        if (P == 2) return R == 1 ? gv_pick_d<FMT, MODE, 2, 1, EMIT>(D) : gv_pick_d<FMT, MODE, 2, 4, EMIT>(D);
        if (P == 3) return R == 1 ? gv_pick_d<FMT, MODE, 3, 1, EMIT>(D) : gv_pick_d<FMT, MODE, 3, 4, EMIT>(D);
        return R == 1 ? gv_pick_d<FMT, MODE, 1, 1, EMIT>(D) : gv_pick_d<FMT, MODE, 1, 4, EMIT>(D);
    }
}

// Mode (b) kernel instances, compiled in their own sources.
GvKernel gv_kernel_b(int fmt, int P, int R, int D);
GvKernel gv_kernel_emit(int fmt, int P, int R, int D);

}  // namespace qmm
