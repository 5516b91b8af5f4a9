// qmm_gemv_row.hip -- decode kernel for one activation row (M == 1), Q8_0,
// Q4_K, Q4_0, Q5_0 and Q6_K weights, modes (a) and (b).
//
// Mode (a) is the Metal form of the same page and section: f32 activations
// against the dequantized weights, y[n] = sum_k w[n][k] x[k], w = d q (Q8_0)
// or d sc_j q - dmin m_j (Q4_K, sub-block j).
// Mode (b) is the CPU form of page "同一个 GGUF，CPU 和 Metal 生成的文字不一样"
// (section 出处): the activation row is quantized on its own, per 32 values to
// Q8_0 for Q8_0 weights (page "自己量化", section 和下载的 Q8_0 逐字节比) and per
// 256 values to Q8K for Q4_K weights, and the products are integer block dot
// products scaled by the block scales:
//     Q8_0: y[n] = sum over blocks b of d_w d_x S_b, S_b the int8 dot product
//           of the 32 weight and activation values;
//     Q4_K: y[n] = sum over super-blocks of d_x (d sum_j sc_j S_j
//           - dmin sum_j m_j B_j), S_j the dot product of sub-block j's 4-bit
//           values with the activation values, B_j the sum of those values.
//
// With a single activation row no weight byte is used twice: the kernel is a
// weight stream, laid out for what this chip's memory system rewards.
//   * Every weight row is read as one contiguous run: 16-byte non-temporal
//     loads, 1 KB per instruction, landing directly in LDS (lane i of a load
//     writes its base + 16 i).  Wave g of W takes rows g, g + W, g + 2W, ...,
//     so at any moment the whole chip reads one contiguous window of the
//     matrix.  A plain read of the 14336 x 4096 Q8_0 matrix (eight copies
//     rotated) in this order runs at about 6.2 TB/s, against about 5.3 TB/s
//     for 16-row tiles read 272 bytes of each row at a time.
//   * A row is cut into segments of 64 lane tasks: Q8_0, 64 block pairs
//     (4352 bytes), lane l taking pair l (it aligns the even block's values,
//     which start two bytes into a dword); Q4_K, 16 super-blocks (2304
//     bytes), lane l taking quarter l % 4 of super-block l / 4 (32 bytes of
//     4-bit values: sub-blocks 2c and 2c + 1 in the low and high nibbles).  The
//     dot products are v_dot4 against activation values the lane holds in
//     registers; a Q4_K super-block's four lanes add their scaled integer
//     sums exactly before the f32 step.
//   * Each wave keeps two segments in flight (deeper measured slower, for
//     either format, also when only the prologue runs deeper).  With three
//     segment buffers (where LDS allows) segment u + 2 is issued before
//     segment u is summed, so the stream never waits on the arithmetic; with
//     two it is issued after.  Every segment issues the same number of load
//     instructions with every lane on (lanes past the segment re-read its
//     first bytes into the buffer's tail), which keeps the explicit waits
//     exact and the issue free of branches.
//   * The activation row is brought into LDS ahead of the stream.  Mode (b)
//     quantizes it once per workgroup with the device functions every other
//     activation quantizer uses, so its blocks are the same bytes; mode (a)
//     keeps it f32.  Each lane then holds its activation values in registers
//     for all of its rows (mode (a): 64 f32, so rows of one segment only).
//   * Mode (a) decodes the lane's weights to exact f32 integers (signed bytes,
//     nibbles) and forms per-block sums of q x with fused multiply-adds; the
//     block then scales them: Q8_0 d S, Q4_K (d sc_j) S_j - (dmin m_j) sum x
//     over the sub-block (the decomposition the tile kernel uses too).
//   * A row's per-lane f32 sums are added across the wave in a fixed order:
//     a run is deterministic.
#include <algorithm>
#include <mutex>
#include <set>
#include <utility>

#include "qmm_act.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int GR_WAVES = 8;
constexpr int GR_THREADS = 64 * GR_WAVES;
constexpr int GR_NSEG_MAX = 4;          // segments per row (K <= 16384)
constexpr int GR_LDS_MAX = 160 * 1024;

// Per format: bytes and activation values of one lane task, tasks per unit of
// the weight format (pair or super-block quarter), bytes of a full segment
// (64 tasks) and of its buffer (the segment's load instructions x 1 KB).
// Q4_0 and Q5_0 weights (mode (b)) take the Q8_0 path with their own block
// pairs (36 and 44 bytes, 4-byte aligned since K % 64 == 0) and Q8_0
// activations; S = sum q x - offset * sum x per block, exact in int32.
constexpr int gr_unit_bytes(int fmt)
{
    return fmt == FMT_Q8_0 ? 68 : fmt == FMT_Q4_0 ? 36 : fmt == FMT_Q5_0 ? 44 : fmt == FMT_Q6_K ? 210 : 144;
}
constexpr bool gr_kq(int fmt) { return fmt == FMT_Q4_K || fmt == FMT_Q6_K; }  // super-blocks, Q8K activations
constexpr int gr_unit_values(int fmt) { return gr_kq(fmt) ? 256 : 64; }
constexpr int gr_seg_units(int fmt) { return gr_kq(fmt) ? 16 : 64; }
constexpr int gr_seg_bytes(int fmt) { return gr_seg_units(fmt) * gr_unit_bytes(fmt); }
constexpr bool gr_pairs(int fmt) { return fmt == FMT_Q4_0 || fmt == FMT_Q5_0; }  // 4-bit pairs with an offset

template <int FMT>
struct GrFmt {
    static constexpr int UNIT_BYTES = gr_unit_bytes(FMT);  // a block pair / a super-block
    static constexpr int UNIT_VALUES = gr_unit_values(FMT);
    static constexpr int LANES_PER_UNIT = gr_kq(FMT) ? 4 : 1;
    static constexpr int SEG_UNITS = 64 / LANES_PER_UNIT;
    static constexpr int SEG_BYTES = SEG_UNITS * UNIT_BYTES;  // 4352 / 2304 / 2304 / 2816
    static constexpr int LPU_MAX = (SEG_BYTES + 1023) / 1024;  // 5 / 3 / 3 / 3
    static constexpr int OFF = FMT == FMT_Q4_0 ? 8 : 16;      // Q4_0 / Q5_0 code offset
};

constexpr int GR_GROUP_MAX = 4;  // problems sharing x in one launch

// Problems p = 0..groups-1 share x and K; their rows are numbered end to end:
// global row r belongs to the last p with row0[p] <= r, local row r - row0[p].
struct GemvRowArgs {
    const uint8_t* w[GR_GROUP_MAX];
    float* y[GR_GROUP_MAX];
    int row0[GR_GROUP_MAX + 1];
    int groups;
    const float* x;
    int N, K;  // N: rows of all problems
    int row_bytes;  // units x unit bytes
    int nunit;      // units per row (Q8_0 block pairs, Q4_K super-blocks)
    int nxi;        // 1 KB load instructions that bring x into LDS
    int xq_off, xd_off, xb_off, ring_off;  // LDS byte offsets (f32 x staged at 0)
    // EMIT instances (mode (b), one problem): the integer parts of the run
    int32_t* sums;  // per row: Q8_0/Q4_0/Q5_0 S per block; Q4_K per super-block S_0..S_7, sumi, summins
    uint8_t* act;   // the quantized activation row as canonical Q8_0 / Q8K blocks (workgroup 0 writes it)
};

QMM_DEV uint32_t gr_lds32(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

typedef __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// 16 bytes per lane from src (per lane) to LDS at dst + 16 * lane (dst the same
// in every lane).  AUX 2: non-temporal (the weight stream is read once).
template <int AUX>
QMM_DEV void ldg16_lds(const uint8_t* src, uint8_t* dst)
{
    __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)dst, 16, 0, AUX);
}

// 16 bytes per lane from a buffer resource at byte offset voff to LDS at
// dst + 16 * lane: offsets past the resource's bytes read no memory (the
// weight rows need not be a multiple of 16 bytes long).  AUX 2: non-temporal.
template <int AUX>
QMM_DEV void buf16_lds(rsrc_t r, uint8_t* dst, uint32_t voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)dst, 16, voff, 0, 0, AUX);
}

// Sum over the wave in a fixed order, the same value in every lane: within each
// 16-lane row by lane exchanges, then the four rows.
QMM_DEV float wave_sum(float v)
{
    v += dpp_f<DPP_X1>(v);
    v += dpp_f<DPP_X2>(v);
    v += dpp_f<DPP_HMIRROR>(v);
    v += dpp_f<DPP_MIRROR>(v);
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// LPU: load instructions per segment, ceil(min(row bytes, segment bytes) / 1024);
// a segment buffer holds LPU KB.  NSEG: segments per row.  RING: segment
// buffers per wave (2 or 3); two segments are in flight either way.  Every
// global load of the kernel writes LDS directly, so all waits on them are the
// explicit ones.  EMIT (mode (b), one problem): the same run, which also
// writes the integer block sums it forms and its quantized activations.
template <int FMT, int MODE, int LPU, int NSEG, int RING, bool EMIT>
__global__ __launch_bounds__(GR_THREADS) void gemv_row_kernel(GemvRowArgs a)
{
    static_assert(MODE == MODE_B || NSEG == 1, "mode (a) holds one segment's activations");
    static_assert(MODE == MODE_B || !EMIT, "integer sums exist in mode (b) only");
    const bool emit_act = EMIT && blockIdx.x == 0 && a.act != nullptr;
    using F = GrFmt<FMT>;
    constexpr int SLOT = 1024 * LPU;
    extern __shared__ __align__(16) uint8_t lds[];
    const float* s_xf = reinterpret_cast<const float*>(lds);
    int8_t* s_xq = reinterpret_cast<int8_t*>(lds + a.xq_off);
    float* s_xd = reinterpret_cast<float*>(lds + a.xd_off);    // Q8_0: per block; Q8K: per super-block
    int32_t* s_xb = reinterpret_cast<int32_t*>(lds + a.xb_off);  // Q8K: sum of each 32 values
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nw = (int)gridDim.x * GR_WAVES, gw = (int)blockIdx.x * GR_WAVES + wave;
    const int N = a.N, K = a.K;
    const int nrows = gw < N ? (N - 1 - gw) / nw + 1 : 0;  // rows gw, gw + nw, ...
    const int U = nrows * NSEG;                             // segments this wave streams
    static_assert(RING == 2 || RING == 3, "ring of 2 or 3 segment buffers");
    constexpr int AHEAD = 2;  // segments in flight
    uint8_t* ring = lds + a.ring_off + wave * (RING * SLOT);
    // problem of global row r (wave-uniform r) and its local row
    auto locate = [&](int r, int& p) {
        p = 0;
#pragma unroll
        for (int q = 1; q < GR_GROUP_MAX; ++q)
            if (q < a.groups && r >= a.row0[q]) p = q;
        return r - a.row0[p];
    };

    // ---- x (f32) into LDS first, so it is not queued behind the stream ----
    {
        const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x);
        const int xbytes = 4 * K;
        for (int i = wave; i < a.nxi; i += GR_WAVES) {
            const int off = 1024 * i + 16 * lane;  // past the end: x's first bytes again, into the pad
            ldg16_lds<0>(xb + (off < xbytes ? off : 0), lds + 1024 * i);
        }
    }

    // ---- the first segments of the stream (they need no activations) ----
    // segment u of this wave into ring buffer `slot`; a wave with fewer than two
    // segments loads its last row (or the matrix's) again for the missing ones.
    // Every lane loads (lanes past the segment read no memory and write zeros
    // into the buffer's tail), so each segment is exactly LPU instructions.
    auto issue = [&](int u, int slot) {
        const int j = u / NSEG, sg = u - j * NSEG;
        int p;
        const int row = locate(min(gw + nw * j, N - 1), p);
        const uint8_t* src = a.w[p] + (int64_t)row * a.row_bytes + sg * F::SEG_BYTES;
        const int bytes = min(F::SEG_BYTES, a.row_bytes - sg * F::SEG_BYTES);
        uint8_t* dst = ring + slot * SLOT;
        // a resource over the segment's bytes: the load that straddles the end of a
        // row (a length not a multiple of 16) reads nothing past it
        const rsrc_t r = make_rsrc(src, (uint32_t)bytes);
#pragma unroll
        for (int t = 0; t < LPU; ++t) buf16_lds<2>(r, dst + 1024 * t, (uint32_t)(1024 * t + 16 * lane));
    };
#pragma unroll
    for (int u = 0; u < AHEAD; ++u) issue(u < U ? u : max(U - 1, 0), u);

    vm_wait<AHEAD * LPU>();  // this wave's share of x has landed (loads retire in order)
    asm volatile("s_barrier" ::: "memory");  // ... and every other wave's

    // ---- quantize x into LDS (mode b) ----
    if constexpr (MODE == MODE_A) {
    } else if constexpr (!gr_kq(FMT)) {
        // 8 values per task, the four tasks of a 32-value block a lane quad
        for (int t = tid; t < K / 8; t += GR_THREADS) {
            const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(s_xf + 8 * t);
            const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(s_xf + 8 * t + 4);
            const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
            am = fmaxf(am, dpp_f<DPP_X1>(am));
            am = fmaxf(am, dpp_f<DPP_X2>(am));
            float id, dval;
            uint16_t dbits;
            q8_0_scale(am, id, dbits, dval);
            int q[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = q8_0_q(v[i], id);
            *reinterpret_cast<u32x2_t*>(s_xq + 8 * t) = u32x2_t{pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7])};
            if ((t & 3) == 0) s_xd[t >> 2] = dval;
            if (emit_act) {  // canonical block t/4: f16 d, then 32 int8 (2-byte aligned)
                uint16_t* o = reinterpret_cast<uint16_t*>(a.act + 34 * (t >> 2));
                if ((t & 3) == 0) o[0] = dbits;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[1 + 4 * (t & 3) + i] = (uint16_t)((uint8_t)q[2 * i] | ((uint8_t)q[2 * i + 1] << 8));
            }
        }
    } else {
        // Q8K, a 16-lane row per 256 values (16 per lane): the signed value of
        // largest |x|, first index on ties, found with lane exchanges in the row
        for (int t = tid; t < K / 16; t += GR_THREADS) {
            const int sb = t >> 4, part = t & 15;
            float v[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const f32x4_t q4 = *reinterpret_cast<const f32x4_t*>(s_xf + 16 * t + 4 * c);
                v[4 * c] = q4[0]; v[4 * c + 1] = q4[1]; v[4 * c + 2] = q4[2]; v[4 * c + 3] = q4[3];
            }
            float best = -1.0f, bv = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float av = fabsf(v[i]);
                if (av > best) { best = av; bv = v[i]; }
            }
            bv = q8k_row16_max(best, bv, best);
            float iscale, d;
            q8k_scale(bv, best, iscale, d);
            int q[16], s16 = 0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                q[i] = q8k_q(v[i], iscale);
                s16 += q[i];
            }
            *reinterpret_cast<u32x4_t*>(s_xq + 16 * t) = u32x4_t{pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]),
                                                              pack4(q[8], q[9], q[10], q[11]), pack4(q[12], q[13], q[14], q[15])};
            const int pair = s16 + dpp_i<DPP_X1>(s16);  // the 32 values of sub-block part / 2
            if ((part & 1) == 0) s_xb[8 * sb + (part >> 1)] = pair;
            if (part == 0) s_xd[sb] = d;
            if (emit_act) {  // canonical Q8K block sb: f32 d, 256 int8, int16 bsums[16]
                uint8_t* o = a.act + 292 * sb;
                if (part == 0) *reinterpret_cast<float*>(o) = d;
                uint32_t* oq = reinterpret_cast<uint32_t*>(o + 4 + 16 * part);
#pragma unroll
                for (int i = 0; i < 4; ++i) oq[i] = pack4(q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]);
                reinterpret_cast<int16_t*>(o + 260)[part] = (int16_t)s16;
            }
        }
    }
    if constexpr (MODE == MODE_B) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- mode (a): this lane's 64 f32 activation values (and Q4_K's sub-block sums) ----
    // Q6_K: lane quarter c of a super-block takes values 128 h + l + 32 k, h = c / 2,
    // l in 16 (c % 2) .. +15, k = 0..3 (the values whose low and high bits share its
    // bytes), as four runs of 16; XS their sums
    float XF[MODE == MODE_A ? 64 : 1];
    float XS[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (MODE == MODE_A && FMT == FMT_Q6_K) {
        const int unit = min(lane / 4, a.nunit - 1), c = lane & 3;
        const float* base = s_xf + 256 * unit + 128 * (c >> 1) + 16 * (c & 1);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const f32x4_t v = *reinterpret_cast<const f32x4_t*>(base + 32 * k + 4 * cc);
#pragma unroll
                for (int e = 0; e < 4; ++e) XF[16 * k + 4 * cc + e] = v[e];
            }
            float t = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) t += XF[16 * k + i];
            XS[k] = t;
        }
    } else if constexpr (MODE == MODE_A) {
        const int unit = min(lane / F::LANES_PER_UNIT, a.nunit - 1);
        const f32x4_t* q = reinterpret_cast<const f32x4_t*>(s_xf + F::UNIT_VALUES * unit + 64 * (lane % F::LANES_PER_UNIT));
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
            const f32x4_t v = q[cc];
#pragma unroll
            for (int e = 0; e < 4; ++e) XF[4 * cc + e] = v[e];
        }
        if constexpr (FMT == FMT_Q4_K) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float t = 0.0f;
#pragma unroll
                for (int i = 0; i < 32; ++i) t += XF[32 * h + i];
                XS[h] = t;
            }
        }
    }

    // ---- mode (b): this lane's activation values for each segment, held for every row ----
    // Q8_0: pair p = 64 sg + lane (two blocks, their scales).  Q4_K: values
    // 64c..64c+63 of super-block sb = 16 sg + lane/4, c = lane % 4, the sums of
    // its two sub-blocks and the super-block's scale.
    constexpr int NB = MODE == MODE_B ? NSEG : 1;
    int X[NB][16];
    float DX[NB][2];
    int XB[NB][4];
#pragma unroll
    for (int sg = 0; sg < NB && MODE == MODE_B; ++sg) {
        const int unit = min(sg * F::SEG_UNITS + lane / F::LANES_PER_UNIT, a.nunit - 1);
        const int c = lane % F::LANES_PER_UNIT;
        if constexpr (FMT == FMT_Q6_K) {
            // the four runs of 16 (see mode (a)) and the sum of each
            const int8_t* base = s_xq + 256 * unit + 128 * (c >> 1) + 16 * (c & 1);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(base + 32 * k);
                int t = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    X[sg][4 * k + e] = (int)v[e];
                    t = __builtin_amdgcn_sdot4((int)v[e], 0x01010101, t, false);
                }
                XB[sg][k] = t;
            }
            DX[sg][0] = DX[sg][1] = s_xd[unit];
            continue;
        }
        const u32x4_t* q = reinterpret_cast<const u32x4_t*>(s_xq + F::UNIT_VALUES * unit + 64 * c);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const u32x4_t v = q[cc];
#pragma unroll
            for (int e = 0; e < 4; ++e) X[sg][4 * cc + e] = (int)v[e];
        }
        if constexpr (FMT != FMT_Q4_K) {
            DX[sg][0] = s_xd[2 * unit];
            DX[sg][1] = s_xd[2 * unit + 1];
            XB[sg][0] = XB[sg][1] = 0;
            if constexpr (gr_pairs(FMT)) {
                // the sum of each block's activation values, for the weights' offset
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int k = 0; k < 8; ++k) XB[sg][h] = __builtin_amdgcn_sdot4(X[sg][8 * h + k], 0x01010101, XB[sg][h], false);
            }
        } else {
            DX[sg][0] = DX[sg][1] = s_xd[unit];
            XB[sg][0] = s_xb[8 * unit + 2 * c];
            XB[sg][1] = s_xb[8 * unit + 2 * c + 1];
        }
    }

    // ---- the stream ----
    float yv = 0.0f;
    int u = 0, slot = 0;
    for (int j = 0; j < nrows; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int sg = 0; sg < NSEG; ++sg, ++u) {
            vm_wait_ahead<LPU, AHEAD - 1>(min(AHEAD - 1, U - 1 - u));  // segment u has landed
            const int nslot = slot + AHEAD >= RING ? slot + AHEAD - RING : slot + AHEAD;  // segment u + 2's buffer
            const bool refill = u + AHEAD < U;
            if (RING > AHEAD && refill) {
                lgkm_wait0();  // segment u - 1's reads of that buffer are done
                issue(u + AHEAD, nslot);
            }
            const int units = min(F::SEG_UNITS, a.nunit - sg * F::SEG_UNITS);
            const uint8_t* sbuf = ring + slot * SLOT;
            if constexpr (gr_pairs(FMT)) {
                if (lane < units) {
                    const uint32_t* wp = reinterpret_cast<const uint32_t*>(sbuf + F::UNIT_BYTES * lane);
                    uint32_t W[F::UNIT_BYTES / 4];
#pragma unroll
                    for (int k = 0; k < F::UNIT_BYTES / 4; ++k) W[k] = wp[k];
                    uint32_t v[2][8];
                    float d[2];
                    pair_codes<FMT>(W, v, d);
                    static_assert(MODE == MODE_B, "Q4_0 / Q5_0 take this kernel in mode (b) only");
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        int sq = 0;
#pragma unroll
                        for (int k = 0; k < 8; ++k) sq = __builtin_amdgcn_sdot4((int)v[h][k], X[sg][8 * h + k], sq, false);
                        acc = fmaf((float)(sq - F::OFF * XB[sg][h]), d[h] * DX[sg][h], acc);
                        if constexpr (EMIT)
                            a.sums[(int64_t)(gw + nw * j) * (2 * a.nunit) + 2 * (sg * F::SEG_UNITS + lane) + h] = sq - F::OFF * XB[sg][h];
                    }
                }
            } else if constexpr (MODE == MODE_A && FMT == FMT_Q8_0) {
                if (lane < units) {
                    const uint32_t* wp = reinterpret_cast<const uint32_t*>(sbuf + 68 * lane);
                    uint32_t W[17];
#pragma unroll
                    for (int k = 0; k < 17; ++k) W[k] = wp[k];
                    // even block: values in bytes 2-33; odd block: values in bytes 36-67
                    float s0a = 0.0f, s0b = 0.0f, s1a = 0.0f, s1b = 0.0f;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const uint32_t e = __builtin_amdgcn_alignbyte(W[k + 1], W[k], 2), o = W[9 + k];
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const float qe = (float)(int8_t)(e >> (8 * b)), qo = (float)(int8_t)(o >> (8 * b));
                            if (b < 2) {
                                s0a = fmaf(qe, XF[4 * k + b], s0a);
                                s1a = fmaf(qo, XF[32 + 4 * k + b], s1a);
                            } else {
                                s0b = fmaf(qe, XF[4 * k + b], s0b);
                                s1b = fmaf(qo, XF[32 + 4 * k + b], s1b);
                            }
                        }
                    }
                    acc = fmaf(s0a + s0b, f16lo(W[0]), acc);
                    acc = fmaf(s1a + s1b, f16hi(W[8]), acc);
                }
            } else if constexpr (FMT == FMT_Q6_K) {
                // super-block ui (210 bytes: ql[128] | qh[64] | sc[16] int8 | d f16; the odd
                // ones start two bytes into a dword), lane quarter c: values 128 hh + 32 k +
                // l, l in l0 .. l0+15: low bits in nibble k / 2 of ql[64 hh + 32 (k & 1) + l],
                // high bits in bit pair k of qh[32 hh + l], scale sc[8 hh + 2 k + c % 2].
                // Lanes past the segment read its last super-block and add nothing.
                const bool live = lane < 4 * units;
                const int c = lane & 3, hh = c >> 1, l0 = 16 * (c & 1);
                const int ui = min(lane >> 2, units - 1);
                const uint8_t* sp = sbuf + 210 * ui;
                const uint32_t sh = (uint32_t)(ui & 1) * 2u;  // byte shift of this super-block
                auto ld = [&](int off, uint32_t* r, int nd) {  // nd dwords from sp + off
                    const uint8_t* pa = sp + off - sh;
                    uint32_t w[5];
#pragma unroll
                    for (int i = 0; i < 5; ++i) w[i] = i <= nd ? gr_lds32(pa + 4 * i) : 0u;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (i < nd) r[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], sh);
                };
                uint32_t qa[4], qb[4], qh[4], scw[2];
                ld(64 * hh + l0, qa, 4);
                ld(64 * hh + 32 + l0, qb, 4);
                ld(128 + 32 * hh + l0, qh, 4);
                ld(192 + 8 * hh, scw, 2);
                const uint32_t dw = gr_lds32(sp + 208 - sh);
                const float d = sh ? f16hi(dw) : f16lo(dw);
                uint32_t code[4][4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    code[0][t] = (qa[t] & 0x0f0f0f0fu) | ((qh[t] & 0x03030303u) << 4);
                    code[1][t] = (qb[t] & 0x0f0f0f0fu) | (((qh[t] >> 2) & 0x03030303u) << 4);
                    code[2][t] = ((qa[t] >> 4) & 0x0f0f0f0fu) | (((qh[t] >> 4) & 0x03030303u) << 4);
                    code[3][t] = ((qb[t] >> 4) & 0x0f0f0f0fu) | (((qh[t] >> 6) & 0x03030303u) << 4);
                }
                int sc[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int bi = 2 * k + (c & 1);
                    sc[k] = (int)(int8_t)(scw[bi >> 2] >> (8 * (bi & 3)));
                }
                if constexpr (MODE == MODE_A) {
                    // exact f32 codes against the f32 values; q - 32 through the run sums
                    float t = 0.0f;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        float sa = 0.0f, sb = 0.0f;
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) {
                            uint32_t cw = code[k][tt];
                            asm volatile("" : "+v"(cw));  // one v_cvt_f32_ubyteN per value
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                const float qf = (float)((cw >> (8 * b)) & 0xffu);
                                if (b < 2) sa = fmaf(qf, XF[16 * k + 4 * tt + b], sa);
                                else sb = fmaf(qf, XF[16 * k + 4 * tt + b], sb);
                            }
                        }
                        t = fmaf((float)sc[k], (sa + sb) - 32.0f * XS[k], t);
                    }
                    if (live) acc = fmaf(d, t, acc);
                } else {
                    int si = 0, S[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        int sk = 0;
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) sk = __builtin_amdgcn_sdot4((int)code[k][tt], X[sg][4 * k + tt], sk, false);
                        S[k] = sk - 32 * XB[sg][k];
                        si += sc[k] * S[k];
                    }
                    si += dpp_i<DPP_X1>(si);  // the super-block's four lanes (exact)
                    si += dpp_i<DPP_X2>(si);
                    if (live && c == 0) acc = fmaf(DX[sg][0], d * (float)si, acc);
                    if constexpr (EMIT) {
                        if (live) {  // per super-block: S_0..S_15, sumi
                            int32_t* o = a.sums + ((int64_t)(gw + nw * j) * a.nunit + sg * F::SEG_UNITS + (lane >> 2)) * 17;
#pragma unroll
                            for (int k = 0; k < 4; ++k) o[8 * hh + 2 * k + (c & 1)] = S[k];
                            if (c == 0) o[16] = si;
                        }
                    }
                }
            } else if constexpr (MODE == MODE_A) {
                if (lane < 4 * units) {
                    const int c = lane & 3;
                    const uint8_t* sp = sbuf + 144 * (lane >> 2);
                    const u32x4_t H = *reinterpret_cast<const u32x4_t*>(sp);  // d | dmin, 12 scale bytes
                    const u32x4_t Qa = *reinterpret_cast<const u32x4_t*>(sp + 16 + 32 * c);
                    const u32x4_t Qb = *reinterpret_cast<const u32x4_t*>(sp + 32 + 32 * c);
                    const uint32_t Q[8] = {Qa[0], Qa[1], Qa[2], Qa[3], Qb[0], Qb[1], Qb[2], Qb[3]};
                    // sub-block 2c: low nibbles against values 0-31; 2c + 1: high nibbles against 32-63
                    float s0a = 0.0f, s0b = 0.0f, s1a = 0.0f, s1b = 0.0f;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        uint32_t lo = Q[k] & 0x0f0f0f0fu, hi = (Q[k] >> 4) & 0x0f0f0f0fu;
                        // opaque to the combiner, so each byte converts with one v_cvt_f32_ubyteN
                        // instead of a bit-field extract and a convert
                        asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const float ql = (float)((lo >> (8 * b)) & 0xffu), qh = (float)((hi >> (8 * b)) & 0xffu);
                            if (b < 2) {
                                s0a = fmaf(ql, XF[4 * k + b], s0a);
                                s1a = fmaf(qh, XF[32 + 4 * k + b], s1a);
                            } else {
                                s0b = fmaf(ql, XF[4 * k + b], s0b);
                                s1b = fmaf(qh, XF[32 + 4 * k + b], s1b);
                            }
                        }
                    }
                    int sc0, m0, sc1, m1;
                    q4k_scale_min(H[1], H[2], H[3], 2 * c, sc0, m0);
                    q4k_scale_min(H[1], H[2], H[3], 2 * c + 1, sc1, m1);
                    const float d = f16lo(H[0]), dmin = f16hi(H[0]);
                    acc = fmaf(-(dmin * (float)m0), XS[0], fmaf(s0a + s0b, d * (float)sc0, acc));
                    acc = fmaf(-(dmin * (float)m1), XS[1], fmaf(s1a + s1b, d * (float)sc1, acc));
                }
            } else if constexpr (FMT == FMT_Q8_0) {
                if (lane < units) {
                    const uint32_t* wp = reinterpret_cast<const uint32_t*>(sbuf + 68 * lane);
                    uint32_t W[17];
#pragma unroll
                    for (int k = 0; k < 17; ++k) W[k] = wp[k];
                    // even block: d in bytes 0-1, values in 2-33; odd block: d in 34-35, values in 36-67
                    int s0 = 0, s1 = 0;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        s0 = __builtin_amdgcn_sdot4((int)__builtin_amdgcn_alignbyte(W[k + 1], W[k], 2), X[sg][k], s0, false);
                        s1 = __builtin_amdgcn_sdot4((int)W[9 + k], X[sg][8 + k], s1, false);
                    }
                    acc = fmaf((float)s0, f16lo(W[0]) * DX[sg][0], acc);
                    acc = fmaf((float)s1, f16hi(W[8]) * DX[sg][1], acc);
                    if constexpr (EMIT) {
                        int32_t* o = a.sums + (int64_t)(gw + nw * j) * (2 * a.nunit) + 2 * (sg * F::SEG_UNITS + lane);
                        o[0] = s0;
                        o[1] = s1;
                    }
                }
            } else {
                // a super-block's four lanes are all live or all not; lanes past the
                // segment read its last super-block and add nothing
                const bool live = lane < 4 * units;
                const int c = lane & 3;
                const uint8_t* sp = sbuf + 144 * min(lane >> 2, units - 1);
                const u32x4_t H = *reinterpret_cast<const u32x4_t*>(sp);  // d | dmin, 12 scale bytes
                const u32x4_t Qa = *reinterpret_cast<const u32x4_t*>(sp + 16 + 32 * c);
                const u32x4_t Qb = *reinterpret_cast<const u32x4_t*>(sp + 32 + 32 * c);
                int s0 = 0, s1 = 0;  // sub-blocks 2c (low nibbles) and 2c + 1 (high nibbles)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    s0 = __builtin_amdgcn_sdot4((int)(Qa[k] & 0x0f0f0f0fu), X[sg][k], s0, false);
                    s1 = __builtin_amdgcn_sdot4((int)((Qa[k] >> 4) & 0x0f0f0f0fu), X[sg][8 + k], s1, false);
                    s0 = __builtin_amdgcn_sdot4((int)(Qb[k] & 0x0f0f0f0fu), X[sg][4 + k], s0, false);
                    s1 = __builtin_amdgcn_sdot4((int)((Qb[k] >> 4) & 0x0f0f0f0fu), X[sg][12 + k], s1, false);
                }
                int sc0, m0, sc1, m1;
                q4k_scale_min(H[1], H[2], H[3], 2 * c, sc0, m0);
                q4k_scale_min(H[1], H[2], H[3], 2 * c + 1, sc1, m1);
                int si = sc0 * s0 + sc1 * s1, sm = m0 * XB[sg][0] + m1 * XB[sg][1];
                si += dpp_i<DPP_X1>(si);  // the super-block's four lanes (exact)
                si += dpp_i<DPP_X2>(si);
                sm += dpp_i<DPP_X1>(sm);
                sm += dpp_i<DPP_X2>(sm);
                if (live && c == 0) acc = fmaf(DX[sg][0], f16lo(H[0]) * (float)si - f16hi(H[0]) * (float)sm, acc);
                if constexpr (EMIT) {
                    if (live) {  // per super-block: S_0..S_7, sumi, summins
                        int32_t* o = a.sums + ((int64_t)(gw + nw * j) * a.nunit + sg * F::SEG_UNITS + (lane >> 2)) * 10;
                        o[2 * c] = s0;
                        o[2 * c + 1] = s1;
                        if (c == 0) {
                            o[8] = si;
                            o[9] = sm;
                        }
                    }
                }
            }
            if (RING == AHEAD && refill) {
                lgkm_wait0();  // this buffer's reads are done before it is refilled
                issue(u + AHEAD, nslot);
            }
            slot = slot + 1 == RING ? 0 : slot + 1;
        }
        // the row is complete: add the lanes' sums (fixed order), park it in lane j % 64;
        // outputs leave 64 rows at a time, or after the last row
        const float t = wave_sum(acc);
        if (lane == (j & 63)) yv = t;
        if ((j & 63) == 63 || j == nrows - 1) {
            const int j0 = j & ~63;
            if (lane <= (j & 63) && (!EMIT || a.y[0])) {
                const int r = gw + nw * (j0 + lane);  // this lane's row (differs per lane)
                float* yp = a.y[0];
                int r0 = 0;
#pragma unroll
                for (int q = 1; q < GR_GROUP_MAX; ++q)
                    if (q < a.groups && r >= a.row0[q]) { yp = a.y[q]; r0 = a.row0[q]; }
                yp[r - r0] = yv;
            }
        }
    }
}

typedef void (*GrKernel)(GemvRowArgs);

template <int FMT, int MODE, int RING, bool EMIT>
static GrKernel gr_kernel_ring(int lpu, int nseg)
{
    constexpr int L = GrFmt<FMT>::LPU_MAX;
    if constexpr (MODE == MODE_B) {
        if (nseg == 4) return gemv_row_kernel<FMT, MODE, L, 4, RING, EMIT>;
        if (nseg == 3) return gemv_row_kernel<FMT, MODE, L, 3, RING, EMIT>;
        if (nseg == 2) return gemv_row_kernel<FMT, MODE, L, 2, RING, EMIT>;
    }
    switch (lpu) {
    case 1: return gemv_row_kernel<FMT, MODE, 1, 1, RING, EMIT>;
    case 2: return gemv_row_kernel<FMT, MODE, (2 < L ? 2 : L), 1, RING, EMIT>;
    case 3: return gemv_row_kernel<FMT, MODE, (3 < L ? 3 : L), 1, RING, EMIT>;
    case 4: return gemv_row_kernel<FMT, MODE, (4 < L ? 4 : L), 1, RING, EMIT>;
    default: return gemv_row_kernel<FMT, MODE, L, 1, RING, EMIT>;
    }
}

template <int FMT, int MODE, bool EMIT>
static GrKernel gr_kernel_mode(int lpu, int nseg, int ring)
{
    return ring == 3 ? gr_kernel_ring<FMT, MODE, 3, EMIT>(lpu, nseg) : gr_kernel_ring<FMT, MODE, 2, EMIT>(lpu, nseg);
}

template <int FMT>
static GrKernel gr_kernel_b(int lpu, int nseg, int ring, bool emit)
{
    return emit ? gr_kernel_mode<FMT, MODE_B, true>(lpu, nseg, ring) : gr_kernel_mode<FMT, MODE_B, false>(lpu, nseg, ring);
}

static GrKernel gr_kernel(int fmt, int mode, int lpu, int nseg, int ring, bool emit)
{
    if (fmt == FMT_Q8_0)
        return mode == MODE_A ? gr_kernel_mode<FMT_Q8_0, MODE_A, false>(lpu, nseg, ring) : gr_kernel_b<FMT_Q8_0>(lpu, nseg, ring, emit);
    if (fmt == FMT_Q4_0) return gr_kernel_b<FMT_Q4_0>(lpu, nseg, ring, emit);  // mode (b) only
    if (fmt == FMT_Q5_0) return gr_kernel_b<FMT_Q5_0>(lpu, nseg, ring, emit);
    if (fmt == FMT_Q6_K)
        return mode == MODE_A ? gr_kernel_mode<FMT_Q6_K, MODE_A, false>(lpu, nseg, ring) : gr_kernel_b<FMT_Q6_K>(lpu, nseg, ring, emit);
    return mode == MODE_A ? gr_kernel_mode<FMT_Q4_K, MODE_A, false>(lpu, nseg, ring) : gr_kernel_b<FMT_Q4_K>(lpu, nseg, ring, emit);
}

// LDS layout: x as f32 (padded to whole 1 KB loads), x quantized (int8), its
// scales, its 32-value sums (Q8K), then the eight waves' segment rings.
struct GrLayout {
    int nxi, xq_off, xd_off, xb_off, ring_off, bytes;
};
static GrLayout gr_layout(int fmt, int64_t K, int ring)
{
    GrLayout l{};
    l.nxi = (int)((4 * K + 1023) / 1024);
    l.xq_off = 1024 * l.nxi;
    l.xd_off = l.xq_off + (int)K;
    l.xb_off = l.xd_off + (int)(!gr_kq(fmt) ? K / 8 : K / 64);
    l.ring_off = (l.xb_off + (int)(!gr_kq(fmt) ? 0 : K / 8) + 15) / 16 * 16;
    const int slot_max = 1024 * ((gr_seg_bytes(fmt) + 1023) / 1024);
    l.bytes = l.ring_off + GR_WAVES * ring * slot_max;
    return l;
}

// Three segment buffers per wave where they fit, else two.
static int gr_ring(int fmt, int64_t K)
{
    return gr_layout(fmt, K, 3).bytes <= GR_LDS_MAX ? 3 : 2;
}

// Rows shorter than a segment leave lanes idle while the per-row arithmetic
// still costs the whole wave: with fewer than half the lanes busy and more
// than four rows per wave, both modes stay on the tile kernel (the 49152 x 576
// lm_head with its blocks in the caches: mode (a) 21.6 us here against 8.5 us
// there, mode (b) 13.0 against 7.8 us; 576-row shapes run faster here).
bool gemv_row_supported(int fmt, int mode, int M, int64_t N, int64_t K, bool emit)
{
    if ((mode != MODE_A && mode != MODE_B) || M != 1 || (emit && mode != MODE_B)) return false;
    if (fmt != FMT_Q8_0 && fmt != FMT_Q4_K && fmt != FMT_Q4_0 && fmt != FMT_Q5_0 && fmt != FMT_Q6_K) return false;
    if (fmt == FMT_Q6_K && K % 512 != 0) return false;  // an even super-block count: 4-byte-aligned rows
    // Q4_0 / Q5_0 mode (a): the staged-activation kernel is faster (on the 8-layer
    // 14336 x 4096 stack 10.3 against 14.0 us for Q4_0), so only mode (b) comes here
    if (gr_pairs(fmt) && mode == MODE_A) return false;
    const int vpu = gr_unit_values(fmt);
    const int nseg_max = mode == MODE_A ? 1 : GR_NSEG_MAX;  // mode (a) holds one segment's f32 activations
    if (K % vpu != 0 || K / vpu > (int64_t)nseg_max * gr_seg_units(fmt)) return false;
    {
        const int64_t lanes = (K / vpu) * (gr_kq(fmt) ? 4 : 1);
        const int64_t rows_per_wave = (N + GR_WAVES * (int64_t)device_cus() - 1) / (GR_WAVES * (int64_t)device_cus());
        if (lanes < 32 && rows_per_wave > 4) return false;
    }
    return gr_layout(fmt, K, gr_ring(fmt, K)).bytes <= GR_LDS_MAX;
}

int gemv_row_group_max() { return GR_GROUP_MAX; }

hipError_t launch_gemv_row_group(int fmt, int mode, int count, const void* const* w, const int64_t* Ns, float* const* y,
                                 const float* x, int64_t K, hipStream_t s, const Trace* tr)
{
    const bool emit = tr != nullptr;
    if (emit && (count != 1 || mode != MODE_B)) return hipErrorInvalidValue;
    if (count < 1 || count > GR_GROUP_MAX) return hipErrorInvalidValue;
    int64_t N = 0;
    for (int i = 0; i < count; ++i) {
        if (Ns[i] <= 0) return hipErrorInvalidValue;
        N += Ns[i];
    }
    if (!gemv_row_supported(fmt, mode, 1, N, K, false) || N > 0x7fffffff) return hipErrorInvalidValue;
    const int ring = gr_ring(fmt, K);
    const GrLayout l = gr_layout(fmt, K, ring);
    GemvRowArgs a{};
    a.groups = count;
    for (int i = 0; i < count; ++i) {
        a.w[i] = (const uint8_t*)w[i];
        a.y[i] = y[i];
        a.row0[i + 1] = a.row0[i] + (int)Ns[i];
    }
    a.x = x;
    a.N = (int)N;
    a.K = (int)K;
    a.nunit = (int)(K / gr_unit_values(fmt));
    a.row_bytes = a.nunit * gr_unit_bytes(fmt);
    a.nxi = l.nxi;
    a.xq_off = l.xq_off;
    a.xd_off = l.xd_off;
    a.xb_off = l.xb_off;
    a.ring_off = l.ring_off;
    const int nseg = (a.nunit + gr_seg_units(fmt) - 1) / gr_seg_units(fmt);
    const int lpu = (std::min(a.row_bytes, gr_seg_bytes(fmt)) + 1023) / 1024;
    // the fewest rows per wave that spread N over every compute unit, then the
    // workgroups that this takes
    const int64_t cus = device_cus();
    const int64_t rpw = (N + GR_WAVES * cus - 1) / (GR_WAVES * cus);
    const int64_t grid = (N + GR_WAVES * rpw - 1) / (GR_WAVES * rpw);
    const GrKernel k = gr_kernel(fmt, mode, lpu, nseg, ring, emit);
    if (emit) {
        a.sums = tr->sums;
        a.act = tr->act;
    }
    static std::set<std::pair<int, const void*>> done;  // dynamic LDS above 64 KB, once per device
    static std::mutex mu;
    {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        std::lock_guard<std::mutex> lock(mu);
        if (done.insert(std::make_pair(dev, (const void*)k)).second) {
            (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, GR_LDS_MAX);
            (void)hipGetLastError();
        }
    }
    void* args[] = {&a};
    const hipError_t e = hipLaunchKernel((const void*)k, dim3((unsigned)grid), dim3(GR_THREADS), args, l.bytes, s);
    return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_gemv_row(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, float* y, hipStream_t s,
                           const Trace* tr)
{
    return launch_gemv_row_group(fmt, mode, 1, &w, &N, &y, x, K, s, tr);
}

}  // namespace qmm
