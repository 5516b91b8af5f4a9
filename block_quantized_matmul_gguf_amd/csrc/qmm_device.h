// qmm_device.h -- device-side helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm_internal.h"

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x32_t __attribute__((ext_vector_type(32)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define QMM_DEV __device__ __forceinline__

// Raw buffer resource over `bytes` bytes from `base`: loads at offsets past
// the end return zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
QMM_DEV rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Lane exchanges inside the vector ALU (DPP), for reductions that must not
// wait on the LDS crossbar: quad_perm [1,0,3,2] (lane ^ 1), [2,3,0,1]
// (lane ^ 2), row_half_mirror (lane i <-> 7 - i within 8 lanes), row_mirror
// (i <-> 15 - i within 16).  Applied in this order, an associative and
// commutative combine leaves the result of a 16-lane row in every lane of it.
enum { DPP_X1 = 0xB1, DPP_X2 = 0x4E, DPP_HMIRROR = 0x141, DPP_MIRROR = 0x140 };
template <int CTRL>
QMM_DEV int dpp_i(int v) { return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false); }
template <int CTRL>
QMM_DEV float dpp_f(float v) { return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v))); }
// max over the wave, the same value in every lane
QMM_DEV float wave_max(float v)
{
    v = fmaxf(v, dpp_f<DPP_X1>(v));
    v = fmaxf(v, dpp_f<DPP_X2>(v));
    v = fmaxf(v, dpp_f<DPP_HMIRROR>(v));
    v = fmaxf(v, dpp_f<DPP_MIRROR>(v));
    const int b = __builtin_bit_cast(int, v);
    return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)), __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)), __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48))));
}

// Waits until at most N of this wave's vector memory operations are
// outstanding.  They retire in issue order, so after vm_wait<k*T> every stage
// but the last k issued has landed.  The compiler does not track loads that
// write LDS directly, hence the explicit waits ("memory" keeps LDS reads after).
template <int N>
QMM_DEV void vm_wait()
{
    static_assert(N >= 0 && N <= 63, "vmcnt holds 0..63");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// vm_wait<ahead*T> for a wave-uniform ahead in [0, I].
template <int T, int I>
QMM_DEV void vm_wait_ahead(int ahead)
{
    if constexpr (I == 0) {
        vm_wait<0>();
    } else {
        if (ahead >= I) vm_wait<I * T>();
        else vm_wait_ahead<T, I - 1>(ahead);
    }
}
QMM_DEV void lgkm_wait0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Byte count for a buffer resource, saturated to its 32-bit field.
QMM_DEV uint32_t clamp_u32(int64_t v) { return v > 0xffffffffll ? 0xffffffffu : (uint32_t)v; }

QMM_DEV float f16lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu)); }
QMM_DEV float f16hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }
QMM_DEV uint16_t f16bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
QMM_DEV float f16round(float f) { return (float)(_Float16)f; }

// Four signed int8 in a dword -> four exact f16 (two half2 dwords, in order).
// f16 bit pattern 0x64XX is 1024 + XX; bias the byte by 128 first so that
// 1024 + (q + 128) - 1152 = q exactly.
QMM_DEV void i8x4_to_f16(uint32_t d, uint32_t& p01, uint32_t& p23)
{
    const uint32_t u = d ^ 0x80808080u;
    uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);
    uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x07030602u);
    const half2_t bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    p01 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) + bias);
    p23 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, b) + bias);
}

// Eight 4-bit values selected by `shift` (0: low nibbles, 4: high nibbles) of
// the bytes of (d0, d1) -> eight exact f16, element order [0,2,1,3,4,6,5,7].
// The caller keeps m = 0x000f000f and c = 0x64006400 in registers, so each
// pair of values is one bit-field insert (f16 bits 0x640N = 1024 + N) and one
// packed subtraction of 1024.
QMM_DEV half8_t nib8_to_f16(uint32_t d0, uint32_t d1, int shift, uint32_t m, uint32_t c)
{
    const half2_t bias = {(_Float16)-1024.0f, (_Float16)-1024.0f};
    const uint32_t s0 = d0 >> shift, s1 = d1 >> shift;
    const uint32_t w0 = (s0 & m) | (c & ~m);
    const uint32_t w1 = ((s0 >> 8) & m) | (c & ~m);
    const uint32_t w2 = (s1 & m) | (c & ~m);
    const uint32_t w3 = ((s1 >> 8) & m) | (c & ~m);
    half2_t h0 = __builtin_bit_cast(half2_t, w0) + bias;
    half2_t h1 = __builtin_bit_cast(half2_t, w1) + bias;
    half2_t h2 = __builtin_bit_cast(half2_t, w2) + bias;
    half2_t h3 = __builtin_bit_cast(half2_t, w3) + bias;
    half8_t r;
    r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
    r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
    return r;
}

// Within-8 element permutation produced by nib8_to_f16: register slot e holds
// element nib_perm(e) of {0,2,1,3,4,6,5,7} (the permutation is its own inverse).
QMM_DEV int nib_perm(int e) { return (e & 4) | ((e & 1) << 1) | ((e & 2) >> 1); }

// Q4_K: 6-bit scale and min of sub-block j from the 12 packed bytes held in
// three dwords s0 (bytes 0-3), s1 (4-7), s2 (8-11).
QMM_DEV void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j, int& sc, int& mn)
{
    if (j < 4) {
        sc = (s0 >> (8 * j)) & 63;
        mn = (s1 >> (8 * j)) & 63;
    } else {
        const int jj = j - 4;
        const uint32_t b8 = (s2 >> (8 * jj)) & 0xffu;
        sc = (int)(b8 & 0x0fu) | (int)(((s0 >> (8 * jj + 6)) & 3u) << 4);
        mn = (int)(b8 >> 4) | (int)(((s1 >> (8 * jj + 6)) & 3u) << 4);
    }
}

// Q4_0 / Q5_0 (page "自己量化": 18 and 22 bytes per 32 values; the public GGUF
// layout: f16 d, Q5_0's u32 of fifth bits, 16 bytes of nibbles with element
// j < 16 in the low nibble of byte j and element j + 16 in its high nibble).
// Bits 0..3 of h, one per byte, moved to bit 4 of bytes 0..3.
QMM_DEV uint32_t spread4(uint32_t h) { return ((h * 0x00204081u) & 0x01010101u) << 4; }

// Codes (0..15 or 0..31), one per byte, of one 32-value block: v[t] holds
// elements 4t..4t+3.  qs: the 16 nibble bytes; qh: Q5_0's fifth bits.
template <int FMT>
QMM_DEV void block_codes(const uint32_t qs[4], uint32_t qh, uint32_t v[8])
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        v[t] = qs[t] & 0x0f0f0f0fu;
        v[4 + t] = (qs[t] >> 4) & 0x0f0f0f0fu;
    }
    if constexpr (FMT == qmm::FMT_Q5_0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] |= spread4((qh >> (4 * t)) & 15u);
    }
}

// Codes and scales of a 4-byte-aligned pair of Q4_0 (9 dwords) or Q5_0 (11
// dwords) blocks held in r: the first block's fields start two bytes into a
// dword and are realigned by a byte shift, the second block's nibbles are
// dword-aligned.
template <int FMT>
QMM_DEV void pair_codes(const uint32_t* r, uint32_t v[2][8], float d[2])
{
    uint32_t a[4], b[4];
    if constexpr (FMT == qmm::FMT_Q4_0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            a[t] = __builtin_amdgcn_alignbyte(r[t + 1], r[t], 2);  // bytes 2..17
            b[t] = r[5 + t];                                       // bytes 20..35
        }
        d[0] = f16lo(r[0]);
        d[1] = f16hi(r[4]);
        block_codes<FMT>(a, 0u, v[0]);
        block_codes<FMT>(b, 0u, v[1]);
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            a[t] = __builtin_amdgcn_alignbyte(r[t + 2], r[t + 1], 2);  // bytes 6..21
            b[t] = r[7 + t];                                           // bytes 28..43
        }
        d[0] = f16lo(r[0]);
        d[1] = f16hi(r[5]);
        block_codes<FMT>(a, __builtin_amdgcn_alignbyte(r[1], r[0], 2), v[0]);  // bytes 2..5
        block_codes<FMT>(b, r[6], v[1]);                                        // bytes 24..27
    }
}

// Grouped prefill launches: up to PG_MAX problems sharing K, the mode and the
// activations (a layer's q/k/v or gate/up projections), each with its own
// weights, outputs and rows; problem p owns column tiles t0[p] .. t0[p+1]-1
// of the launch, so every output tile belongs to one problem and computes
// what that problem's own launch computes.
constexpr int PG_MAX = 4;
struct PrefillGroup {
    const uint8_t* w[PG_MAX];
    float* y[PG_MAX];
    int n[PG_MAX];       // rows (outputs) of each problem
    int t0[PG_MAX + 1];  // first column tile of each problem; t0[groups] = all column tiles
    int groups;
};
// The problem of column tile nt (a chain of selects: no indexed access to the
// kernel arguments): its weights, outputs, rows and first column tile.
QMM_DEV void pg_locate(const PrefillGroup& g, int nt, const uint8_t*& w, float*& y, int& n, int& tile0)
{
    w = g.w[0];
    y = g.y[0];
    n = g.n[0];
    tile0 = 0;
#pragma unroll
    for (int q = 1; q < PG_MAX; ++q) {
        const bool in = q < g.groups && nt >= g.t0[q];
        w = in ? g.w[q] : w;
        y = in ? g.y[q] : y;
        n = in ? g.n[q] : n;
        tile0 = in ? g.t0[q] : tile0;
    }
}

// Q8_0 GEMV block-pair k permutation.  Inside a 4-byte-aligned pair of
// blocks (68 bytes), lane group g (0..3) of the MFMA operand takes the 8
// weight bytes at dwords (1+2g, 2+2g) of the even block; group 3 takes dword
// 7 and the four bytes q0, q1, q30, q31.  The odd block's weights are
// dword-aligned and go in natural order.  Returns the weight index (0..31)
// held in slot t (0..7) of group g.
QMM_DEV int q8_even_k(int g, int t)
{
    if (g < 3) return 2 + 8 * g + t;
    if (t < 4) return 26 + t;
    const int tail[4] = {0, 1, 30, 31};
    return tail[t - 4];
}
