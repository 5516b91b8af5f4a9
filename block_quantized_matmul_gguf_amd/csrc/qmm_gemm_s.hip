// qmm_gemm_s.hip -- prefill (M > 8) of Q8_0, Q4_0, Q5_0 and Q4_K weights with
// short rows (K <= 1536), the activation preparation done inside the launch.
//
// The pages' SmolLM2-135M prefill (page "GGUF", section 在 candle 里跑一个 GGUF:
// a 37-token prompt, then 270 teacher-forced tokens) is 211 products with K =
// 576 or 1536 at M = 307.  There the K-staged tile kernels (qmm_gemm.hip,
// qmm_gemm_q.hip) wait on one global round trip per 64-value stage, after a
// separate launch that prepares the activations.  Here a 512-thread workgroup
// owns 16 activation rows x 64 weight rows and takes its K range in one go:
//   * each pair of waves copies its column block's 16 weight rows (raw blocks,
//     whole rows, or pieces of at most 576 values where LDS is short) into an
//     LDS buffer with 16-byte buffer-to-LDS loads; rows past N read as zero;
//   * the workgroup loads its 16 activation rows (f32) into registers, a row
//     per 16 lanes, and prepares them itself: mode (a) the row's power-of-two
//     scale and the f16 hi/lo split, mode (b) the Q8_0 (Q8K for Q4_K) blocks
//     through the standalone quantizer's device functions (the same bytes),
//     written to LDS in matrix-core operand order;
//   * v_mfma_f32_16x16x32_f16 per 32-value block: A = the 16 rows' hi and
//     then lo parts (mode (a)) or their int8 values as exact f16 (mode (b):
//     the f32 sum is the exact integer block sum), B = the block's weights as
//     exact f16 (Q8_0 q, Q4_0 q - 8, Q5_0 q - 16, decoded from block pairs,
//     the 4-byte-aligned load units); acc += d_w C (mode (a)), (d_w d_x) C (b).
//     Q4_K: the nibbles q per 32-value sub-block, with the scales, mins and
//     (mode (b)) the integer sumi and summins applied per super-block.
// Grouped launches number the problems' column tiles end to end; traced runs
// (mode (b)) write the block sums and the quantized activation blocks.
#include <algorithm>
#include <mutex>
#include <set>
#include <utility>

#include "qmm_act.h"
#include "qmm_gemv_kernel.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int GS_NT = 512;                 // threads: eight waves
constexpr int GS_BM = 16;                  // activation rows per tile
constexpr int GS_BN = 64;                  // weight rows per tile, 16 per wave
constexpr int GS_KMAX = 1536;              // longest row
constexpr int GS_JMAX = GS_KMAX / 64;      // 16-byte activation loads per thread
constexpr int GS_PIECE = 576;              // most values of a row staged at once
constexpr int64_t GS_NMAX = 8192;          // widest launch (all problems' rows)
constexpr int GS_TLP = 12;                 // most loads of one wave's piece (pieces of at most 576 values)

struct GemmSArgs {
    PrefillGroup g;
    const float* x;
    int32_t* sums;  // traced runs: [M][N][K/32]
    uint8_t* act;   // traced runs: canonical Q8_0 blocks [M][K/32], or null
    int K, M, nm, remap;
    int row_bytes;  // K / 64 block pairs of gs_lub(fmt) bytes
    int kp;         // values per staged piece of a row (divides K, a multiple of 64)
    int cpr;        // pieces: 16-byte chunks per LDS weight row (odd: the 16 rows in different banks)
    int nbuf;       // weight buffers per wave (2: piece p + 1 lands while p is summed)
    int bsz;        // bytes of one weight buffer
    int off_dx;     // mode (a): row exponents [16]; mode (b): d_x [K/32][16]
    int off_b;      // the weight buffers, [wave][nbuf]
};

// Bytes of a block pair (64 values): Q8_0 d | 32 int8, Q4_0 d | qs[16],
// Q5_0 d | qh[4] | qs[16], twice.
constexpr int gs_lub(int fmt) { return fmt == FMT_Q8_0 ? 68 : fmt == FMT_Q4_0 ? 36 : 44; }
// Bytes of a row: block pairs, or Q4_K super-blocks (144 B per 256 values).
constexpr int64_t gs_row_bytes(int fmt, int64_t K) { return fmt == FMT_Q4_K ? K / 256 * 144 : K / 64 * gs_lub(fmt); }

// Eight 5-bit codes (bytes of c0, c1) -> eight exact f16 (code - OFF) in order:
// byte b under 0x64 is the f16 1024 + b, then one packed subtraction.
template <int OFF>
QMM_DEV half8_t gs_codes_f16(uint32_t c0, uint32_t c1)
{
    const half2_t bias = {(_Float16)(-1024.0f - OFF), (_Float16)(-1024.0f - OFF)};
    u32x4_t r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c0, 0x04010400u)) + bias);
    r[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c0, 0x04030402u)) + bias);
    r[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c1, 0x04010400u)) + bias);
    r[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, c1, 0x04030402u)) + bias);
    return __builtin_bit_cast(half8_t, r);
}

// One block pair's operands: w = the weight dwords (the even block's three,
// the odd block's two, the two holding d0 and d1, Q5_0's two of fifth bits);
// a = the activation operand chunks
// (mode (a): even hi, even lo, odd hi, odd lo; mode (b): even, odd, then d_x of
// the lane's four rows for each block).
struct GsPair {
    uint32_t w[9];
    u32x4_t a[4];
};

QMM_DEV uint32_t gs_h2(_Float16 a, _Float16 b) { return __builtin_bit_cast(uint32_t, half2_t{a, b}); }

// Eight waves: waves w and w + 4 share column block w (its 16 weight rows), each
// issuing half of the block's loads and of the activation loads and taking half
// of the block pairs; their partial sums are added at the end, lower half first.
// The loads leave eight waves per workgroup faster than four (four waves, one
// per column block: a 576 x 576 product at M = 307 took 7.6 against 7.1 us,
// 576 x 1536 in mode (b) 14.8 against 12.1 us, in mode (a) 16.1 against 13.6).
template <int FMT, int MODE, bool EMIT>
__global__ __launch_bounds__(GS_NT, 2) void gemm_s_kernel(GemmSArgs a)
{
    constexpr int S = 2;  // halves of the workgroup
    constexpr int LUB = gs_lub(FMT), HALF = LUB / 2;
    constexpr bool QK = FMT == FMT_Q4_K;  // Q4_K (whole rows): super-blocks, not block pairs
    static_assert(!EMIT || MODE == MODE_B, "integer block sums exist in mode (b) only");
    extern __shared__ __align__(16) uint8_t lds[];
    const int K = a.K, M = a.M, nb = K / 32;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = wave & 3, hf = wave >> 2;  // column block, half
    // the tile: row tiles of one column tile are consecutive, and with the
    // remap each XCD (workgroups id % 8) takes a contiguous run of them
    const int G = (int)gridDim.x, id = (int)blockIdx.x;
    const int L = a.remap ? (id & 7) * (G >> 3) + (id >> 3) : id;
    const int mt = L % a.nm, nt = L / a.nm;
    const uint8_t* W;
    float* Y;
    int N, tile0;
    pg_locate(a.g, nt, W, Y, N, tile0);
    const int m0 = mt * GS_BM;
    const int n0 = (nt - tile0) * GS_BN + 16 * blk;  // the first weight row of the wave's column block

    // ---- activations: row rho of the tile in lanes 16 rho .. +15 (one DPP row),
    // lane c16 holding values 64 j + 4 c16 .. +3; rows past M read as zero ----
    // (half hf takes the chunks j = 2 i + hf; for Q4_K whole super-blocks, the
    // chunks of super-blocks hf, hf + 2, ..., so a Q8K block stays in one half)
    auto jof = [&](int i) { return QK ? 4 * (2 * (i >> 2) + hf) + (i & 3) : S * i + hf; };
    const int rho = (tid & 255) >> 4, c16 = tid & 15, nj = K / 64;
    const rsrc_t xr = make_rsrc(a.x + (int64_t)m0 * K, clamp_u32((int64_t)(M - m0) * K * 4));
    constexpr int JI = GS_JMAX / S;
    f32x4_t xv[JI];
#pragma unroll
    for (int i = 0; i < JI; ++i) {
        const int j = jof(i);
        xv[i] = j < nj ? __builtin_bit_cast(f32x4_t, ld128(xr, (uint32_t)(rho * K + 64 * j + 4 * c16) * 4u))
                       : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // ---- weights: piece p (values p*kp .. +kp of each row) of column block blk's 16
    // rows, half of the loads from each of the block's two waves.
    // Whole rows (kp == K): the 16 rows are one contiguous, 16-byte aligned run of
    // bytes, copied as is (LDS row stride = row_bytes).  Pieces: row r's chunk c
    // (16 bytes from the piece's start) lands at row r * 16 cpr; a row's last chunk
    // may run past its piece (into bytes never read back). ----
    const bool whole = a.kp == K;
    const int rs = whole ? a.row_bytes : 16 * a.cpr, pb = QK ? 0 : a.kp / 64 * LUB;
    const int64_t wb = (int64_t)n0 * a.row_bytes, wleft = (int64_t)N * a.row_bytes - wb;
    const rsrc_t wr = make_rsrc(W + (wleft > 0 ? wb : 0), wleft > 0 ? (uint32_t)min(wleft, (int64_t)16 * a.row_bytes) : 0u);
    const int nchunk = whole ? a.row_bytes : 16 * a.cpr, tl = (nchunk + 63) / 64;
    const int th = (tl + S - 1) / S, t0 = hf * th, t1 = min(tl, t0 + th);  // this wave's loads of a piece
    auto issue = [&](int p) {
        uint8_t* buf = lds + a.off_b + (blk * a.nbuf + p % a.nbuf) * a.bsz;
        for (int t = t0; t < t1; ++t) {
            const int f = 64 * t + lane;
            if (f < nchunk) {
                uint32_t off = 16u * (uint32_t)f;
                if (!whole) {
                    const int r = f / a.cpr;
                    off = (uint32_t)(r * a.row_bytes + p * pb + 16 * (f - r * a.cpr));
                }
                ld128_lds(wr, buf + 1024 * t, off);
            }
        }
    };
    const int np = K / a.kp;
    issue(0);
    if (a.nbuf > 1 && np > 1) issue(1);

    // operand chunks: mode (a) [block][hi, lo][64 lanes][16 B], mode (b) [block][64 lanes][16 B];
    // lane r + 16 g of a chunk holds row r's values 8 g .. 8 g + 7 of the block
    uint8_t* A = lds;
    const int blk_hi = c16 >> 3, kg = (c16 & 7) >> 1, half_off = 8 * (c16 & 1);
    if constexpr (MODE == MODE_A) {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < JI; ++i)
            if (jof(i) < nj)
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(xv[i][e]));
        mx = fmaxf(mx, dpp_f<DPP_X1>(mx));
        mx = fmaxf(mx, dpp_f<DPP_X2>(mx));
        mx = fmaxf(mx, dpp_f<DPP_HMIRROR>(mx));
        mx = fmaxf(mx, dpp_f<DPP_MIRROR>(mx));
        {  // the two halves' maxima of the row meet in LDS
            float* hm = reinterpret_cast<float*>(lds + a.off_dx + 64);
            if (c16 == 0) hm[16 * hf + rho] = mx;
            __syncthreads();
            mx = fmaxf(hm[rho], hm[16 + rho]);
        }
        const int ex = split_exp(mx);
        const float sc = ldexpf(1.0f, ex);
        if (c16 == 0 && hf == 0) reinterpret_cast<int*>(lds + a.off_dx)[rho] = ex;
#pragma unroll
        for (int i = 0; i < JI; ++i) {
            const int j = jof(i);
            if (j < nj) {
                _Float16 h[4], l[4];
                float xs[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) split_one(xv[i][e], sc, h[e], l[e], xs[e]);
                const int s = 2 * j + blk_hi;
                if constexpr (QK) {
                    // the 32-value sub-block's sum of x*2^e (the mins term), over its eight lanes
                    float t = (xs[0] + xs[1]) + (xs[2] + xs[3]);
                    t += dpp_f<DPP_X1>(t);
                    t += dpp_f<DPP_X2>(t);
                    t += dpp_f<DPP_HMIRROR>(t);
                    if ((c16 & 7) == 0) reinterpret_cast<float*>(lds + a.off_dx + 256)[s * 16 + rho] = t;
                }
                uint8_t* dst = A + ((2 * s) * 64 + rho + 16 * kg) * 16 + half_off;
                *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{gs_h2(h[0], h[1]), gs_h2(h[2], h[3])};
                *reinterpret_cast<u32x2_t*>(dst + 1024) = u32x2_t{gs_h2(l[0], l[1]), gs_h2(l[2], l[3])};
            }
        }
    } else if constexpr (QK) {
        // Q8K per 256 values (super-block u: chunks 4u .. 4u+3, all in half u % 2):
        // the signed element of largest |x|, the first index on ties, met over the
        // row's 16 lanes (DPP); the values, the sums of each 16 and of each 32 (the
        // mins term) in LDS
        const int nsb = K / 256;
        float* dxk = reinterpret_cast<float*>(lds + a.off_dx);                  // [u][16] d_x
        int* bsub = reinterpret_cast<int*>(lds + a.off_dx + nsb * 64);          // [K/32][16] sums of 32
        float kis[GS_JMAX / 4];
#pragma unroll
        for (int u = 0; u < GS_JMAX / 4; ++u) {
            float best = -1.0f, bv = 0.0f;
            int bidx = 0;
#pragma unroll
            for (int i = 0; i < JI; ++i) {
                const int j = jof(i);
                if (j < nj && (j >> 2) == u) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float v = xv[i][e];
                        if (fabsf(v) > best) { best = fabsf(v); bv = v; bidx = 64 * (j & 3) + 4 * c16 + e; }
                    }
                }
            }
            auto meet1 = [&](float ob, float obv, int oidx) {
                if (ob > best || (ob == best && oidx < bidx)) { best = ob; bv = obv; bidx = oidx; }
            };
            meet1(dpp_f<DPP_X1>(best), dpp_f<DPP_X1>(bv), dpp_i<DPP_X1>(bidx));
            meet1(dpp_f<DPP_X2>(best), dpp_f<DPP_X2>(bv), dpp_i<DPP_X2>(bidx));
            meet1(dpp_f<DPP_HMIRROR>(best), dpp_f<DPP_HMIRROR>(bv), dpp_i<DPP_HMIRROR>(bidx));
            meet1(dpp_f<DPP_MIRROR>(best), dpp_f<DPP_MIRROR>(bv), dpp_i<DPP_MIRROR>(bidx));
            float dk;
            q8k_scale(bv, best, kis[u], dk);
            if (u < nsb && c16 == 0 && (u & 1) == hf) dxk[u * 16 + rho] = dk;
            if constexpr (EMIT)
                if (u < nsb && c16 == 0 && (u & 1) == hf && nt == 0 && a.act != nullptr && m0 + rho < M)
                    *reinterpret_cast<float*>(a.act + ((int64_t)(m0 + rho) * nsb + u) * 292) = dk;
        }
#pragma unroll
        for (int i = 0; i < JI; ++i) {
            const int j = jof(i);
            if (j < nj) {
                float isc = kis[0];
#pragma unroll
                for (int u = 1; u < GS_JMAX / 4; ++u) isc = (j >> 2) == u ? kis[u] : isc;
                int q[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e] = q8k_q(xv[i][e], isc);
                const int s = 2 * j + blk_hi;
                uint8_t* dst = A + (s * 64 + rho + 16 * kg) * 16 + half_off;
                *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{gs_h2((_Float16)q[0], (_Float16)q[1]), gs_h2((_Float16)q[2], (_Float16)q[3])};
                // sums of 16 (a lane quad) and of 32 (eight lanes)
                int s16 = (q[0] + q[1]) + (q[2] + q[3]);
                s16 += dpp_i<DPP_X1>(s16);
                s16 += dpp_i<DPP_X2>(s16);
                const int s32 = s16 + dpp_i<DPP_HMIRROR>(s16);
                if ((c16 & 7) == 0) bsub[s * 16 + rho] = s32;
                if constexpr (EMIT) {
                    if (nt == 0 && a.act != nullptr && m0 + rho < M) {
                        // canonical Q8K block j / 4 of row m0 + rho: f32 d, 256 int8, int16 sums of 16
                        uint8_t* o = a.act + ((int64_t)(m0 + rho) * nsb + (j >> 2)) * 292;
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[4 + 64 * (j & 3) + 4 * c16 + e] = (uint8_t)q[e];
                        if ((c16 & 3) == 0) reinterpret_cast<int16_t*>(o + 260)[4 * (j & 3) + (c16 >> 2)] = (int16_t)s16;
                    }
                }
            }
        }
    } else {
        float* dxs = reinterpret_cast<float*>(lds + a.off_dx);
#pragma unroll
        for (int i = 0; i < JI; ++i) {
            const int j = jof(i);
            if (j < nj) {
                // the block's max |x| over its eight lanes
                float am = fmaxf(fmaxf(fabsf(xv[i][0]), fabsf(xv[i][1])), fmaxf(fabsf(xv[i][2]), fabsf(xv[i][3])));
                am = fmaxf(am, dpp_f<DPP_X1>(am));
                am = fmaxf(am, dpp_f<DPP_X2>(am));
                am = fmaxf(am, dpp_f<DPP_HMIRROR>(am));
                float qid, dval;
                uint16_t dbits;
                q8_0_scale(am, qid, dbits, dval);
                int q[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e] = q8_0_q(xv[i][e], qid);
                const int s = 2 * j + blk_hi;
                uint8_t* dst = A + (s * 64 + rho + 16 * kg) * 16 + half_off;
                *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{gs_h2((_Float16)q[0], (_Float16)q[1]), gs_h2((_Float16)q[2], (_Float16)q[3])};
                if ((c16 & 7) == 0) dxs[s * 16 + rho] = dval;
                if constexpr (EMIT) {
                    // canonical block s of row m0 + rho: f16 d, then the 32 int8 (column tile 0 writes them)
                    if (nt == 0 && a.act != nullptr && m0 + rho < M) {
                        uint8_t* o = a.act + ((int64_t)(m0 + rho) * nb + s) * 34;
                        if ((c16 & 7) == 0) {
                            o[0] = (uint8_t)(dbits & 0xffu);
                            o[1] = (uint8_t)(dbits >> 8);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[2 + 4 * (c16 & 7) + e] = (uint8_t)q[e];
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- blocks: lane (n, g) holds outputs rows 4 g + i, column n0 + n ----
    const int n = lane & 15, g = lane >> 4, col = n0 + n;
    const float* dxs = reinterpret_cast<const float*>(lds + a.off_dx);
    const f32x4_t zf = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4_t acc = zf;
    const int ppp = a.kp / 64;  // block pairs per piece
    for (int p = 0; p < np; ++p) {
        // both halves read the block's rows: each waits for its loads of piece p (traced
        // runs' stores count too, so they wait for everything), then a barrier; piece
        // p + 1 then goes into the buffer of piece p - 1, which every wave is done with
        // (pieces 0 and 1 were issued at the start)
        if (EMIT || a.nbuf == 1 || p + 1 >= np || p > 0) vm_wait<0>();
        else vm_wait_ahead<1, GS_TLP>(t1 - t0);
        __syncthreads();
        if (a.nbuf > 1 && p >= 1 && p + 1 < np) issue(p + 1);
        const uint8_t* rrow = lds + a.off_b + (blk * a.nbuf + p % a.nbuf) * a.bsz + n * rs;
        if constexpr (QK) {
            // super-blocks u of this wave's half: f16 d, dmin | 12 bytes of 6-bit scales
            // and mins | 128 bytes of nibbles (sub-block 2c: low nibbles of bytes 32c ..
            // 32c+31, 2c+1: high nibbles); the weights enter as exact f16 q (0 .. 15),
            // acc += (d sc_j) C_j - (dmin m_j) X_j with X_j the sub-block's sum of x*2^e
            // mode (b): S_j exact (q up to 15 against int8 values: below 2^24), sumi and
            // summins in int32, acc += d_x (d sumi - dmin summins)
            const int nsb = K / 256, hq = (nsb + 1) / 2, ua = hf * hq, ub = min(nsb, ua + hq);
            const float* xsum = reinterpret_cast<const float*>(lds + a.off_dx + 256);
            const float* dxk = reinterpret_cast<const float*>(lds + a.off_dx);
            const int* bsub = reinterpret_cast<const int*>(lds + a.off_dx + nsb * 64);
            for (int u = ua; u < ub; ++u) {
                const uint8_t* rp = rrow + 144 * u;
                const u32x4_t H = lds128(rp);
                const float d = f16lo(H[0]), dmin = f16hi(H[0]);
                int sumi[4] = {0, 0, 0, 0}, summ[4] = {0, 0, 0, 0};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x2_t Qv = lds64(rp + 16 + 32 * c + 8 * g);
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int jj = 2 * c + hh, s = 8 * u + jj;
                        int scj, mnj;
                        q4k_scale_min(H[1], H[2], H[3], jj, scj, mnj);
                        const half8_t B = gs_codes_f16<0>((Qv[0] >> (4 * hh)) & 0x0f0f0f0fu, (Qv[1] >> (4 * hh)) & 0x0f0f0f0fu);
                        if constexpr (MODE == MODE_A) {
                            f32x4_t C = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, lds128(A + ((2 * s) * 64 + lane) * 16)), B, zf, 0, 0, 0);
                            C = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, lds128(A + ((2 * s + 1) * 64 + lane) * 16)), B, C, 0, 0, 0);
                            const f32x4_t X = *reinterpret_cast<const f32x4_t*>(xsum + s * 16 + 4 * g);
                            const float ds = d * (float)scj, dm = dmin * (float)mnj;
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[i] = fmaf(-dm, X[i], fmaf(ds, C[i], acc[i]));
                        } else {
                            const f32x4_t C = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, lds128(A + (s * 64 + lane) * 16)), B, zf, 0, 0, 0);
                            const i32x4_t Bs = *reinterpret_cast<const i32x4_t*>(bsub + s * 16 + 4 * g);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                sumi[i] += scj * (int)C[i];
                                summ[i] += mnj * Bs[i];
                            }
                            if constexpr (EMIT) {
                                if (col < N)
#pragma unroll
                                    for (int i = 0; i < 4; ++i)
                                        if (m0 + 4 * g + i < M)
                                            a.sums[(((int64_t)(m0 + 4 * g + i) * N + col) * nsb + u) * 10 + jj] = (int32_t)C[i];
                            }
                        }
                    }
                }
                if constexpr (MODE == MODE_B) {
                    const f32x4_t dx = *reinterpret_cast<const f32x4_t*>(dxk + u * 16 + 4 * g);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = fmaf(dx[i] * d, (float)sumi[i], fmaf(-dx[i] * dmin, (float)summ[i], acc[i]));
                    if constexpr (EMIT) {
                        if (col < N)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (m0 + 4 * g + i < M) {
                                    int32_t* o = a.sums + (((int64_t)(m0 + 4 * g + i) * N + col) * nsb + u) * 10;
                                    o[8] = sumi[i];
                                    o[9] = summ[i];
                                }
                    }
                }
            }
            continue;
        }
        const int hp = (ppp + S - 1) / S, qa = hf * hp, qb = min(ppp, qa + hp);  // this wave's pairs
        // software-pipelined over the piece's block pairs: the operands of pair q + 1
        // are read while pair q is on the matrix cores, and pair q's scales are
        // applied after pair q + 1's matrix-core steps are issued
        auto load = [&](int q, GsPair& o) {
            // pair q (dword-aligned); the even block's values start two bytes into a dword
            const uint8_t* rp = rrow + LUB * q;
            const int s0 = 2 * (p * ppp + q);
            if constexpr (FMT == FMT_Q8_0) {
                // values 8g .. 8g+7 of a block are its bytes 2 + 8g .. 9 + 8g
                o.w[0] = lds32(rp + 8 * g);
                o.w[1] = lds32(rp + 8 * g + 4);
                o.w[2] = lds32(rp + 8 * g + 8);
                o.w[3] = lds32(rp + 36 + 8 * g);
                o.w[4] = lds32(rp + 40 + 8 * g);
            } else {
                // values 8g .. 8g+7: the low (g < 2) or high nibbles of qs bytes
                // 8 (g & 1) .. +7, Q5_0 with bits 8g .. 8g+7 of qh as fifth bits
                constexpr int QS0 = FMT == FMT_Q4_0 ? 2 : 6, QS1 = HALF + QS0;
                const int qo = 8 * (g & 1);
                o.w[0] = lds32(rp + QS0 - 2 + qo);
                o.w[1] = lds32(rp + QS0 + 2 + qo);
                o.w[2] = lds32(rp + QS0 + 6 + qo);
                o.w[3] = lds32(rp + QS1 + qo);
                o.w[4] = lds32(rp + QS1 + qo + 4);
                if constexpr (FMT == FMT_Q5_0) {
                    o.w[7] = lds32(rp + 4);
                    o.w[8] = lds32(rp + HALF + 2);
                }
            }
            o.w[5] = lds32(rp);
            o.w[6] = lds32(rp + HALF - 2);
            if constexpr (MODE == MODE_A) {
#pragma unroll
                for (int c = 0; c < 4; ++c) o.a[c] = lds128(A + ((2 * s0 + c) * 64 + lane) * 16);
            } else {
                o.a[0] = lds128(A + (s0 * 64 + lane) * 16);
                o.a[1] = lds128(A + ((s0 + 1) * 64 + lane) * 16);
                o.a[2] = __builtin_bit_cast(u32x4_t, *reinterpret_cast<const f32x4_t*>(dxs + s0 * 16 + 4 * g));
                o.a[3] = __builtin_bit_cast(u32x4_t, *reinterpret_cast<const f32x4_t*>(dxs + (s0 + 1) * 16 + 4 * g));
            }
        };
        // pair sums Ce, Co (blocks s0, s0 + 1) into acc with the pair's scales
        auto apply = [&](const f32x4_t& Ce, const f32x4_t& Co, const GsPair& o, int s0) {
            const float de = f16lo(o.w[5]), dd = f16hi(o.w[6]);
            if constexpr (MODE == MODE_A) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = fmaf(Co[i], dd, fmaf(Ce[i], de, acc[i]));
            } else {
                const f32x4_t xe = __builtin_bit_cast(f32x4_t, o.a[2]), xo = __builtin_bit_cast(f32x4_t, o.a[3]);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = fmaf(Co[i], dd * xo[i], fmaf(Ce[i], de * xe[i], acc[i]));
                if constexpr (EMIT) {
                    if (col < N) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int m = m0 + 4 * g + i;
                            if (m < M) {
                                int32_t* out = a.sums + ((int64_t)m * N + col) * nb + s0;
                                out[0] = (int32_t)Ce[i];
                                out[1] = (int32_t)Co[i];
                            }
                        }
                    }
                }
            }
        };
        GsPair cur, prv;
        f32x4_t pCe = zf, pCo = zf;
        if (qa < qb) load(qa, cur);
        for (int q = qa; q < qb; ++q) {
            GsPair nxt;
            if (q + 1 < qb) load(q + 1, nxt);
            half8_t Be, Bo;
            if constexpr (FMT == FMT_Q8_0) {
                Be = i8x8_to_f16(__builtin_amdgcn_alignbyte(cur.w[1], cur.w[0], 2), __builtin_amdgcn_alignbyte(cur.w[2], cur.w[1], 2));
                Bo = i8x8_to_f16(cur.w[3], cur.w[4]);
            } else {
                const int sh = 4 * (g >> 1);
                uint32_t ce0 = (__builtin_amdgcn_alignbyte(cur.w[1], cur.w[0], 2) >> sh) & 0x0f0f0f0fu;
                uint32_t ce1 = (__builtin_amdgcn_alignbyte(cur.w[2], cur.w[1], 2) >> sh) & 0x0f0f0f0fu;
                uint32_t co0 = (cur.w[3] >> sh) & 0x0f0f0f0fu;
                uint32_t co1 = (cur.w[4] >> sh) & 0x0f0f0f0fu;
                if constexpr (FMT == FMT_Q5_0) {
                    const uint32_t he = __builtin_amdgcn_alignbyte(cur.w[7], cur.w[5], 2), ho = cur.w[8];
                    ce0 |= spread4((he >> (8 * g)) & 15u);
                    ce1 |= spread4((he >> (8 * g + 4)) & 15u);
                    co0 |= spread4((ho >> (8 * g)) & 15u);
                    co1 |= spread4((ho >> (8 * g + 4)) & 15u);
                }
                constexpr int OFF = FMT == FMT_Q4_0 ? 8 : 16;
                Be = gs_codes_f16<OFF>(ce0, ce1);
                Bo = gs_codes_f16<OFF>(co0, co1);
            }
            f32x4_t Ce, Co;
            if constexpr (MODE == MODE_A) {
                Ce = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, cur.a[0]), Be, zf, 0, 0, 0);
                Co = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, cur.a[2]), Bo, zf, 0, 0, 0);
                Ce = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, cur.a[1]), Be, Ce, 0, 0, 0);
                Co = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, cur.a[3]), Bo, Co, 0, 0, 0);
            } else {
                Ce = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, cur.a[0]), Be, zf, 0, 0, 0);
                Co = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, cur.a[1]), Bo, zf, 0, 0, 0);
            }
            if (q > qa) apply(pCe, pCo, prv, 2 * (p * ppp + q - 1));
            pCe = Ce;
            pCo = Co;
            prv = cur;
            cur = nxt;
        }
        if (qa < qb) apply(pCe, pCo, prv, 2 * (p * ppp + qb - 1));
        if (a.nbuf == 1 && p + 1 < np) {
            __syncthreads();  // both halves are done with the buffer
            issue(p + 1);
        }
    }

    {
        // the upper half's partial sums join the lower half's (in that order)
        __syncthreads();  // the activation operand's bytes take them
        f32x4_t* part = reinterpret_cast<f32x4_t*>(lds);
        if (hf == 1) part[blk * 64 + lane] = acc;
        __syncthreads();
        if (hf == 1) return;
        acc += part[blk * 64 + lane];
    }
    if (Y != nullptr && col < N) {
        const int* se = reinterpret_cast<const int*>(lds + a.off_dx);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = m0 + 4 * g + i;
            if (m < M) {
                float v = acc[i];
                if constexpr (MODE == MODE_A) v *= ldexpf(1.0f, -se[4 * g + i]);
                Y[(int64_t)m * N + col] = v;
            }
        }
    }
}

void gs_allow_lds(const void* k, int bytes)
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

// The largest multiple of 64 that divides K and is at most GS_PIECE.
int gs_piece(int64_t K)
{
    int kp = (int)(std::min<int64_t>(K, GS_PIECE) / 64) * 64;
    while (kp > 64 && K % kp != 0) kp -= 64;
    return kp;
}

}  // namespace

template <int FMT>
static const void* gs_kernel(int mode, bool traced)
{
    return mode == MODE_A ? (const void*)gemm_s_kernel<FMT, MODE_A, false>
           : traced       ? (const void*)gemm_s_kernel<FMT, MODE_B, true>
                          : (const void*)gemm_s_kernel<FMT, MODE_B, false>;
}

// LDS bytes of a launch and its buffer plan: whole rows when they fit; else
// pieces of at most 576 values, two buffers per wave where they fit (the
// largest such piece), one otherwise.
static int gs_plan(int fmt, int mode, int64_t K, GemmSArgs& a)
{
    const int nb = (int)(K / 32), lub = gs_lub(fmt);
    // the activation operand's bytes also take the upper half's partial sums (4 KB)
    const int abytes = std::max(mode == MODE_A ? nb * 2048 : nb * 1024, 4096);
    // mode (a): row exponents, the halves' row maxima; Q4_K also the sub-block sums [K/32][16]
    const int nsb = (int)(K / 256);
    const int dxbytes = mode == MODE_A ? 256 + (fmt == FMT_Q4_K ? nb * 64 : 0)
                        : fmt == FMT_Q4_K ? nsb * 64 + nb * 64  // d_x, sums of 32
                                          : nb * 64;
    a.row_bytes = (int)gs_row_bytes(fmt, K);
    a.off_dx = abytes;
    a.off_b = (abytes + dxbytes + 15) & ~15;
    const int room = 160 * 1024 - a.off_b;
    if (4 * 16 * a.row_bytes <= room || fmt == FMT_Q4_K) {  // Q4_K: whole rows only
        a.kp = (int)K;
        a.cpr = 0;
        a.nbuf = 1;
        a.bsz = 16 * a.row_bytes;
    } else {
        auto bsz = [lub](int kp) { return 16 * 16 * (((kp / 64 * lub + 15) / 16) | 1); };
        a.nbuf = 1;
        a.kp = gs_piece(K);
        for (int kp = a.kp; kp >= 64; kp -= 64)
            if (K % kp == 0 && 4 * 2 * bsz(kp) <= room) {
                a.kp = kp;
                a.nbuf = 2;
                break;
            }
        a.cpr = ((a.kp / 64 * lub + 15) / 16) | 1;
        a.bsz = bsz(a.kp);
    }
    return a.off_b + 4 * a.nbuf * a.bsz;
}

// Short rows, and a grid of at most one workgroup per compute unit: with more
// tiles the K-staged kernels, whose larger tiles reread fewer bytes, are faster
// (the 1536 x 576 gate and up pair at M = 307: 960 tiles, 17.5 us against
// 14.4 us).  The test is per problem, so a grouped run gives each problem the
// kernel of its own run.
bool gemm_s_supported(int fmt, int mode, int64_t K, int64_t Ntot, int64_t M)
{
    if (fmt == FMT_Q4_K && K % 256 != 0) return false;
    if (!((fmt == FMT_Q8_0 || fmt == FMT_Q4_0 || fmt == FMT_Q5_0 || fmt == FMT_Q4_K) && M > GEMV_MAX_M && K > 0 && K % 64 == 0 && K <= GS_KMAX && Ntot > 0 && Ntot <= GS_NMAX))
        return false;
    GemmSArgs a{};
    const int bytes = gs_plan(fmt, mode, K, a);
    const int64_t grid = ((M + GS_BM - 1) / GS_BM) * ((Ntot + GS_BN - 1) / GS_BN);
    return bytes <= 160 * 1024 && grid <= (int64_t)device_cus();
}

hipError_t launch_gemm_s(int fmt, int mode, int count, const void* const* w, const int64_t* Ns, float* const* y,
                         const float* x, int64_t K, int64_t M, hipStream_t s, const Trace* tr)
{
    if (count < 1 || count > PG_MAX || (tr && (count != 1 || mode != MODE_B))) return hipErrorInvalidValue;
    if (!(K > 0 && K % 64 == 0 && K <= GS_KMAX && M > 0) ||
        !(fmt == FMT_Q8_0 || fmt == FMT_Q4_0 || fmt == FMT_Q5_0 || (fmt == FMT_Q4_K && K % 256 == 0)))
        return hipErrorInvalidValue;
    GemmSArgs a{};
    a.g.groups = count;
    a.g.t0[0] = 0;
    for (int p = 0; p < PG_MAX; ++p) {
        const bool on = p < count;
        a.g.w[p] = on ? (const uint8_t*)w[p] : nullptr;
        a.g.y[p] = on ? y[p] : nullptr;
        a.g.n[p] = on ? (int)Ns[p] : 0;
        a.g.t0[p + 1] = a.g.t0[p] + (on ? (int)((Ns[p] + GS_BN - 1) / GS_BN) : 0);
    }
    a.x = x;
    a.sums = tr ? tr->sums : nullptr;
    a.act = tr ? tr->act : nullptr;
    a.K = (int)K;
    a.M = (int)M;
    a.nm = (int)((M + GS_BM - 1) / GS_BM);
    const int bytes = gs_plan(fmt, mode, K, a);
    const int64_t grid = (int64_t)a.nm * a.g.t0[count];
    if (grid < 1 || grid > 0x7fffffff || bytes > 160 * 1024) return hipErrorInvalidConfiguration;
    a.remap = grid % 8 == 0 ? 1 : 0;
    const void* k = fmt == FMT_Q8_0 ? gs_kernel<FMT_Q8_0>(mode, tr != nullptr)
                    : fmt == FMT_Q4_0 ? gs_kernel<FMT_Q4_0>(mode, tr != nullptr)
                    : fmt == FMT_Q5_0 ? gs_kernel<FMT_Q5_0>(mode, tr != nullptr)
                                      : gs_kernel<FMT_Q4_K>(mode, tr != nullptr);
    gs_allow_lds(k, bytes);
    void* args[] = {&a};
    return hipLaunchKernel(k, dim3((unsigned)grid), dim3(GS_NT), args, (size_t)bytes, s);
}

}  // namespace qmm
