// qmm_gemm.hip -- prefill kernel (M > 8) for y = x . W^T on GGUF blocks.
//
// 128x128 output tile per 256-thread workgroup; each wave owns 64x64 as 2x2
// v_mfma_f32_32x32x16_f16 tiles.  K advances 64 values per stage: the weight
// rows of the stage are decoded once into LDS as exact f16 integers (Q8_0: q;
// Q4_K: sc_j*q <= 945), shared by all waves; the next stage's raw bytes are
// prefetched into registers while the current one computes.
//   mode (a): activations arrive as an exact f16 hi/lo split of a power-of-two
//     scaled row (two MFMA passes); per-block f32 epilogue acc += d*C (Q8_0
//     every 32 values; Q4_K once per 256 with the mins term
//     -dmin*sum_j m_j*sum(x over sub-block j));
//   mode (b): activations arrive as their quantized integers in f16; the MFMA
//     sums are exact integers (Q8_0 block sums |S| <= 516128; Q4_K half
//     super-block sums of sc_j*q*q8 < 2^24), scaled in f32: Q8_0 acc +=
//     dw*dx*S per block, Q4_K acc += dx*d*sumi per 128 values and
//     -dx*dmin*summins per super-block (page "同一个 GGUF，CPU 和 Metal
//     生成的文字不一样", section 出处: integer dot, then the scales).
#include "qmm_device.h"

namespace qmm {

struct GemmArgs {
    const uint8_t* w;
    int64_t row_bytes;
    int N, K, M;
    const _Float16* a0;
    const _Float16* a1;
    const float* sc0;
    const void* sc1;
    float* y;
    int32_t* sums;
};

constexpr int LDA = GEMM_KS + 8;  // halves per LDS row (16-byte pad against bank conflicts)

template <int FMT, int MODE, bool EMIT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a)
{
    constexpr bool TWO = MODE == MODE_A;
    __shared__ __align__(16) _Float16 sA0[GEMM_BM * LDA];
    __shared__ __align__(16) _Float16 sA1[TWO ? GEMM_BM * LDA : 8];
    __shared__ __align__(16) _Float16 sB[GEMM_BN * LDA];
    __shared__ __align__(16) float sWd[2][GEMM_BN];   // Q8_0: weight block scales; Q4_K: [0]=d, [1]=dmin
    __shared__ __align__(16) float sXd[2][GEMM_BM];   // Q8_0 mode b: act block scales; Q4_K mode b: [0]=dx
    __shared__ __align__(16) int sQm[8][GEMM_BN];     // Q4_K sub-block mins m_j
    __shared__ __align__(16) float sXs[8][GEMM_BM];   // Q4_K: mode a sub-block sums of x*s; mode b bsum pairs

    const int M = a.M, N = a.N, K = a.K;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int m0 = blockIdx.y * GEMM_BM, n0 = blockIdx.x * GEMM_BN;
    const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
    const int nst = K / GEMM_KS;
    const int nb = K / 32;

    // ---- per-thread load roles ----
    const int br = tid >> 1, bpart = tid & 1;  // weight row and half of the stage
    const bool brow_ok = n0 + br < N;
    const uint8_t* wrow = a.w + (int64_t)(n0 + (brow_ok ? br : 0)) * a.row_bytes;

    uint4 ra0[4], ra1[TWO ? 4 : 1];
    uint32_t rb[9];
    float rx[2];

    auto load_stage = [&](int st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, row = idx >> 3, c16 = idx & 7;
            const int m = m0 + row;
            if (m < M) {
                const int64_t off = (int64_t)m * K + st * GEMM_KS + 8 * c16;
                ra0[i] = *reinterpret_cast<const uint4*>(a.a0 + off);
                if (TWO) ra1[i] = *reinterpret_cast<const uint4*>(a.a1 + off);
            } else {
                ra0[i] = make_uint4(0, 0, 0, 0);
                if (TWO) ra1[i] = make_uint4(0, 0, 0, 0);
            }
        }
        if (FMT == FMT_Q8_0) {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(wrow + 68 * st) + 8 * bpart;
#pragma unroll
            for (int i = 0; i < 9; ++i) rb[i] = brow_ok ? p[i] : 0u;
            if (MODE == MODE_B) {
                if (tid < GEMM_BM) {
                    const int m = m0 + tid;
                    const float2 v = m < M ? *reinterpret_cast<const float2*>(a.sc0 + (int64_t)m * nb + 2 * st)
                                           : make_float2(0.0f, 0.0f);
                    rx[0] = v.x;
                    rx[1] = v.y;
                }
            }
        } else {
            const int sb = st >> 2, c = st & 3;
            const uint4 hdr = brow_ok ? *reinterpret_cast<const uint4*>(wrow + 144 * sb) : make_uint4(0, 0, 0, 0);
            const uint4 qv = brow_ok ? *reinterpret_cast<const uint4*>(wrow + 144 * sb + 16 + 32 * c + 16 * bpart)
                                     : make_uint4(0, 0, 0, 0);
            rb[0] = hdr.x; rb[1] = hdr.y; rb[2] = hdr.z; rb[3] = hdr.w;
            rb[4] = qv.x; rb[5] = qv.y; rb[6] = qv.z; rb[7] = qv.w;
        }
    };

    auto store_stage = [&](int st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, row = idx >> 3, c16 = idx & 7;
            *reinterpret_cast<uint4*>(&sA0[row * LDA + 8 * c16]) = ra0[i];
            if (TWO) *reinterpret_cast<uint4*>(&sA1[row * LDA + 8 * c16]) = ra1[i];
        }
        if (FMT == FMT_Q8_0) {
            uint32_t q[8];
            float d;
            if (bpart == 0) {
                d = f16lo(rb[0]);
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_alignbyte(rb[i + 1], rb[i], 2);
            } else {
                d = f16hi(rb[0]);
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = rb[i + 1];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t t0, t1, t2, t3;
                i8x4_to_f16(q[2 * i], t0, t1);
                i8x4_to_f16(q[2 * i + 1], t2, t3);
                *reinterpret_cast<uint4*>(&sB[br * LDA + 32 * bpart + 8 * i]) = make_uint4(t0, t1, t2, t3);
            }
            sWd[bpart][br] = brow_ok ? d : 0.0f;
            if (MODE == MODE_B && tid < GEMM_BM) {
                sXd[0][tid] = rx[0];
                sXd[1][tid] = rx[1];
            }
        } else {
            const int c = st & 3;
            int sc0, mn0, sc1, mn1;
            q4k_scale_min(rb[1], rb[2], rb[3], 2 * c, sc0, mn0);
            q4k_scale_min(rb[1], rb[2], rb[3], 2 * c + 1, sc1, mn1);
            const _Float16 f0 = (_Float16)(float)sc0, f1 = (_Float16)(float)sc1;
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // 8 bytes at a time
                half8_t lo, hi;
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const uint32_t byte = (rb[4 + 2 * h + (b >> 2)] >> (8 * (b & 3))) & 0xffu;
                    lo[b] = (_Float16)(float)(byte & 15u) * f0;
                    hi[b] = (_Float16)(float)(byte >> 4) * f1;
                }
                *reinterpret_cast<half8_t*>(&sB[br * LDA + 16 * bpart + 8 * h]) = lo;
                *reinterpret_cast<half8_t*>(&sB[br * LDA + 32 + 16 * bpart + 8 * h]) = hi;
            }
            if (c == 0 && bpart == 0) {
                sWd[0][br] = brow_ok ? f16lo(rb[0]) : 0.0f;
                sWd[1][br] = brow_ok ? f16hi(rb[0]) : 0.0f;
#pragma unroll
                for (int jq = 0; jq < 8; ++jq) {
                    int s_, m_;
                    q4k_scale_min(rb[1], rb[2], rb[3], jq, s_, m_);
                    sQm[jq][br] = m_;
                }
            }
            if (c == 0) {  // per-row activation data of the super-block
                const int sb = st >> 2;
                for (int idx = tid; idx < GEMM_BM * 8; idx += 256) {
                    const int row = idx >> 3, jq = idx & 7, m = m0 + row;
                    if (MODE == MODE_A) {
                        sXs[jq][row] = m < M ? reinterpret_cast<const float*>(a.sc1)[(int64_t)m * (K / 32) + 8 * sb + jq] : 0.0f;
                    } else {
                        const int v = m < M ? reinterpret_cast<const int32_t*>(a.sc1)[(int64_t)m * (K / 32) + 8 * sb + jq] : 0;
                        sXs[jq][row] = __builtin_bit_cast(float, v);
                    }
                }
                if (MODE == MODE_B)
                    for (int row = tid; row < GEMM_BM; row += 256)
                        sXd[0][row] = m0 + row < M ? a.sc0[(int64_t)(m0 + row) * (K / 256) + sb] : 0.0f;
            }
        }
    };

    f32x16_t acc[2][2], cb[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int yv = 0; yv < 2; ++yv)
#pragma unroll
            for (int r = 0; r < 16; ++r) { acc[x][yv][r] = 0.0f; cb[x][yv][r] = 0.0f; }
    int32_t half0[2][2][16];  // Q4_K mode b block-sums hook: first-half sumi

    const int li = lane & 31, lk = 8 * (lane >> 5);
    // C layout: lane column j = li; register r holds row 8*(r/4) + 4*(lane/32) + (r%4)
    auto crow = [&](int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); };

    load_stage(0);
    for (int st = 0; st < nst; ++st) {
        __syncthreads();
        store_stage(st);
        __syncthreads();
        if (st + 1 < nst) load_stage(st + 1);

#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            half8_t A0[2], A1[2], B[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                A0[t] = *reinterpret_cast<const half8_t*>(&sA0[(wm + 32 * t + li) * LDA + 16 * kk + lk]);
                if (TWO) A1[t] = *reinterpret_cast<const half8_t*>(&sA1[(wm + 32 * t + li) * LDA + 16 * kk + lk]);
                B[t] = *reinterpret_cast<const half8_t*>(&sB[(wn + 32 * t + li) * LDA + 16 * kk + lk]);
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    cb[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0[mt], B[nt], cb[mt][nt], 0, 0, 0);
                    if (TWO) cb[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1[mt], B[nt], cb[mt][nt], 0, 0, 0);
                }

            if (FMT == FMT_Q8_0 && (kk & 1)) {  // end of a 32-value block
                const int blk = kk >> 1;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const float dw = sWd[blk][wn + 32 * nt + li];
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            float s = dw;
                            if (MODE == MODE_B) s *= sXd[blk][wm + 32 * mt + crow(r)];
                            acc[mt][nt][r] += s * cb[mt][nt][r];
                            if (EMIT) {
                                const int m = m0 + wm + 32 * mt + crow(r), n = n0 + wn + 32 * nt + li;
                                if (m < M && n < N) a.sums[((int64_t)m * N + n) * nb + 2 * st + blk] = (int32_t)cb[mt][nt][r];
                            }
                            cb[mt][nt][r] = 0.0f;
                        }
                    }
            }
        }

        if (FMT == FMT_Q4_K) {
            const int c = st & 3;
            if (MODE == MODE_B && (c & 1)) {  // end of a 128-value half super-block
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const float d = sWd[0][wn + 32 * nt + li];
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float dx = sXd[0][wm + 32 * mt + crow(r)];
                            acc[mt][nt][r] += (dx * d) * cb[mt][nt][r];
                            if (EMIT) {
                                if (c == 1) half0[mt][nt][r] = (int32_t)cb[mt][nt][r];
                                else half0[mt][nt][r] += (int32_t)cb[mt][nt][r];
                            }
                            cb[mt][nt][r] = 0.0f;
                        }
                    }
            }
            if (c == 3) {  // end of the super-block: scale (mode a) and mins term
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        const int nl = wn + 32 * nt + li;
                        const float d = sWd[0][nl], dmin = sWd[1][nl];
                        int mj[8];
#pragma unroll
                        for (int jq = 0; jq < 8; ++jq) mj[jq] = sQm[jq][nl];
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int ml = wm + 32 * mt + crow(r);
                            if (MODE == MODE_A) {
                                float mins = 0.0f;
#pragma unroll
                                for (int jq = 0; jq < 8; ++jq) mins += (float)mj[jq] * sXs[jq][ml];
                                acc[mt][nt][r] += d * cb[mt][nt][r] - dmin * mins;
                                cb[mt][nt][r] = 0.0f;
                            } else {
                                int summ = 0;
#pragma unroll
                                for (int jq = 0; jq < 8; ++jq) summ += mj[jq] * __builtin_bit_cast(int, sXs[jq][ml]);
                                acc[mt][nt][r] -= sXd[0][ml] * dmin * (float)summ;
                                if (EMIT) {
                                    const int m = m0 + ml, n = n0 + nl;
                                    if (m < M && n < N) {
                                        int32_t* o = a.sums + (((int64_t)m * N + n) * (K / 256) + (st >> 2)) * 10;
#pragma unroll
                                        for (int jq = 0; jq < 8; ++jq) o[jq] = INT32_MIN;
                                        o[8] = half0[mt][nt][r];
                                        o[9] = summ;
                                    }
                                }
                            }
                        }
                    }
            }
        }
    }

    if (EMIT) return;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int n = n0 + wn + 32 * nt + li;
            if (n >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm + 32 * mt + crow(r);
                if (m < M) {
                    float v = acc[mt][nt][r];
                    if (MODE == MODE_A) v *= a.sc0[m];
                    a.y[(int64_t)m * N + n] = v;
                }
            }
        }
}

template <int FMT, int MODE, bool EMIT>
static void launch_one(const GemmArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.N + GEMM_BN - 1) / GEMM_BN), (unsigned)((a.M + GEMM_BM - 1) / GEMM_BM));
    hipLaunchKernelGGL((gemm_kernel<FMT, MODE, EMIT>), grid, dim3(256), 0, s, a);
}

hipError_t launch_gemm(int fmt, int mode, const void* w, int64_t N, int64_t K, int64_t M, const GemmBufs& b,
                       float* y, int32_t* sums, hipStream_t s)
{
    GemmArgs a{};
    a.w = (const uint8_t*)w;
    a.row_bytes = fmt == FMT_Q8_0 ? (K / 32) * 34 : (K / 256) * 144;
    a.N = (int)N;
    a.K = (int)K;
    a.M = (int)M;
    a.a0 = b.a0;
    a.a1 = b.a1;
    a.sc0 = b.sc0;
    a.sc1 = b.sc1;
    a.y = y;
    a.sums = sums;
    const bool emit = sums != nullptr;
    if (fmt == FMT_Q8_0) {
        if (mode == MODE_A) launch_one<FMT_Q8_0, MODE_A, false>(a, s);
        else if (emit) launch_one<FMT_Q8_0, MODE_B, true>(a, s);
        else launch_one<FMT_Q8_0, MODE_B, false>(a, s);
    } else {
        if (mode == MODE_A) launch_one<FMT_Q4_K, MODE_A, false>(a, s);
        else if (emit) launch_one<FMT_Q4_K, MODE_B, true>(a, s);
        else launch_one<FMT_Q4_K, MODE_B, false>(a, s);
    }
    return hipGetLastError();
}

}  // namespace qmm
