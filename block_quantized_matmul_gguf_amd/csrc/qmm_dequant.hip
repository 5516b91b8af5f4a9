// qmm_dequant.hip -- the dequantize-all form (QMM_MODE_DEQUANT).
//
// The page "同一个 GGUF，CPU 和 Metal 生成的文字不一样" (section 修法, and the
// comparison before it) describes a third form besides (a) and (b):
// CANDLE_DEQUANTIZE_ALL turns every quantized weight into f32 when the model
// is loaded, after which both devices run a plain f32 matmul; it removes the
// activation quantization at the cost of f32-sized weights and slower decode.
// Here the GGUF blocks are decoded to f32 [N][K] by the kernels below (every
// value is the exact dequantized weight rounded once to f32), and y = x . W^T
// is a plain f32 matmul: for decode sizes a weight-streaming kernel, else the
// library f32 GEMM (rocBLAS).
#include <rocblas/rocblas.h>

#include <mutex>
#include <set>
#include <utility>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// Q8_0, one thread per quarter block (8 values): w = f16(d) * q, exact in f32.
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const uint8_t* __restrict__ w, int64_t quarters,
                                                           float* __restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= quarters) return;
    const uint8_t* blk = w + (i >> 2) * 34;
    const uint8_t* q = blk + 2 + 8 * (i & 3);
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(blk[0] | (blk[1] << 8)));
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = d * (float)(int8_t)q[j];
    float4* o = reinterpret_cast<float4*>(out + 8 * i);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// Q4_K, one thread per 32-value sub-block j of a super-block: element 64c + l
// is the low (l < 32) or high nibble of byte 16 + 32c + l % 32, and
// w = d*sc_j*q - dmin*m_j.  d*sc_j and dmin*m_j are exact in f32, so the
// single rounding of the fused multiply-add gives the exact value rounded once.
__global__ __launch_bounds__(256) void dequant_q4_k_kernel(const uint8_t* __restrict__ w, int64_t subs,
                                                           float* __restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= subs) return;
    const int j = (int)(i & 7);
    const uint8_t* blk = w + (i >> 3) * 144;
    const uint32_t* hd = reinterpret_cast<const uint32_t*>(blk);
    int sc, mn;
    q4k_scale_min(hd[1], hd[2], hd[3], j, sc, mn);
    const float ds = f16lo(hd[0]) * (float)sc, dm = f16hi(hd[0]) * (float)mn;
    const uint4* qs = reinterpret_cast<const uint4*>(blk + 16 + 32 * (j >> 1));
    const int shift = 4 * (j & 1);
    float4* o = reinterpret_cast<float4*>(out + 32 * i);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint4 b = qs[h];
        const uint32_t wd[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(ds, (float)((wd[k] >> (8 * e + shift)) & 15u), -dm);
            o[4 * h + k] = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

hipError_t launch_dequantize(int fmt, const void* w, int64_t N, int64_t K, float* out, hipStream_t s)
{
    const int64_t units = fmt == FMT_Q8_0 ? N * (K / 32) * 4 : N * (K / 256) * 8;
    const unsigned grid = (unsigned)((units + 255) / 256);
    if (fmt == FMT_Q8_0)
        hipLaunchKernelGGL(dequant_q8_0_kernel, dim3(grid), dim3(256), 0, s, (const uint8_t*)w, units, out);
    else
        hipLaunchKernelGGL(dequant_q4_k_kernel, dim3(grid), dim3(256), 0, s, (const uint8_t*)w, units, out);
    return hipGetLastError();
}

// ------------------------------------------------- the plain f32 matmul ----

// Decode sizes (M <= 8, M*K*4 bytes of x within LDS): an HBM stream of the f32
// weights.  x is staged in LDS once per workgroup; each wave takes RR rows at a
// time (RR = 4 for several activation rows, so that one LDS read of x serves
// four weight loads), 16 bytes per lane per load, and reduces its sums across
// the wave.
constexpr int DG_THREADS = 512;
constexpr int DG_LDS_MAX = 128 * 1024;

template <int MM, int RR>
__global__ __launch_bounds__(DG_THREADS) void dense_gemv_kernel(const float* __restrict__ w, const float* __restrict__ x,
                                                                float* __restrict__ y, int N, int K, int M)
{
    extern __shared__ __align__(16) float sx[];  // [M][K]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < M * K / 4; i += DG_THREADS)
        reinterpret_cast<float4*>(sx)[i] = reinterpret_cast<const float4*>(x)[i];
    __syncthreads();
    const int waves = (int)gridDim.x * (DG_THREADS / 64);
    const int kq = K / 4;
    for (int n0 = ((int)blockIdx.x * (DG_THREADS / 64) + wave) * RR; n0 < N; n0 += waves * RR) {
        const float4* wr[RR];
#pragma unroll
        for (int r = 0; r < RR; ++r) wr[r] = reinterpret_cast<const float4*>(w + (int64_t)(n0 + r < N ? n0 + r : n0) * K);
        float acc[RR][MM];
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int m = 0; m < MM; ++m) acc[r][m] = 0.0f;
#pragma unroll 4
        for (int q = lane; q < kq; q += 64) {
            float4 v[RR];
#pragma unroll
            for (int r = 0; r < RR; ++r) v[r] = wr[r][q];
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                if (m < M) {
                    const float4 xv = reinterpret_cast<const float4*>(sx + m * K)[q];
#pragma unroll
                    for (int r = 0; r < RR; ++r)
                        acc[r][m] = __builtin_fmaf(v[r].x, xv.x, __builtin_fmaf(v[r].y, xv.y,
                                    __builtin_fmaf(v[r].z, xv.z, __builtin_fmaf(v[r].w, xv.w, acc[r][m]))));
                }
            }
        }
#pragma unroll
        for (int r = 0; r < RR; ++r)
#pragma unroll
            for (int m = 0; m < MM; ++m) {
                float t = acc[r][m];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
                if (lane == 0 && m < M && n0 + r < N) y[(int64_t)m * N + n0 + r] = t;
            }
    }
}

static int cu_count_d()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    (void)hipGetLastError();
    return cus;
}

static hipError_t dense_gemv(const float* w, const float* x, float* y, int64_t M, int64_t N, int64_t K, hipStream_t s)
{
    const size_t lds = (size_t)M * K * 4;
    const int rows_per_wg = (DG_THREADS / 64) * (M == 1 ? 1 : 4);
    const int64_t want = (N + rows_per_wg - 1) / rows_per_wg;
    const int grid = (int)(want < 8LL * cu_count_d() ? want : 8LL * cu_count_d());
    const void* k = M == 1 ? (const void*)dense_gemv_kernel<1, 1> : (const void*)dense_gemv_kernel<8, 4>;
    {  // raise the kernel's dynamic LDS limit, once per device
        static std::set<std::pair<int, const void*>> done;
        static std::mutex mu;
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) dev = 0;
        std::lock_guard<std::mutex> lock(mu);
        if (done.insert(std::make_pair(dev, k)).second) {
            (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, DG_LDS_MAX);
            (void)hipGetLastError();
        }
    }
    int n_ = (int)N, k_ = (int)K, m_ = (int)M;
    void* args[] = {(void*)&w, (void*)&x, (void*)&y, &n_, &k_, &m_};
    return hipLaunchKernel(k, dim3((unsigned)grid), dim3(DG_THREADS), args, lds, s);
}

int dense_create(void** handle)
{
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return -1;
    // the same inputs give the same bits on every run
    if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success) {
        rocblas_destroy_handle(h);
        return -1;
    }
    *handle = h;
    return 0;
}

void dense_destroy(void* handle)
{
    if (handle) rocblas_destroy_handle((rocblas_handle)handle);
}

// y[M x N] = x[M x K] . W[N x K]^T, all row-major f32.  Decode sizes take the
// stream kernel above; otherwise rocBLAS, in whose column-major terms
// y^T (N x M) = W (N x K, stored as its K x N transpose) . x^T (K x M).
int dense_gemm(void* handle, const float* w, const float* x, float* y, int64_t M, int64_t N, int64_t K,
               hipStream_t s)
{
    if (M <= 8 && (size_t)M * K * 4 <= (size_t)DG_LDS_MAX && K % 4 == 0) {
        const hipError_t e = dense_gemv(w, x, y, M, N, K, s);
        return e == hipSuccess ? 0 : -2;
    }
    rocblas_handle h = (rocblas_handle)handle;
    if (rocblas_set_stream(h, s) != rocblas_status_success) return -1;
    const float one = 1.0f, zero = 0.0f;
    const rocblas_status st = rocblas_sgemm(h, rocblas_operation_transpose, rocblas_operation_none, (rocblas_int)N,
                                            (rocblas_int)M, (rocblas_int)K, &one, w, (rocblas_int)K, x,
                                            (rocblas_int)K, &zero, y, (rocblas_int)N);
    return st == rocblas_status_success ? 0 : (int)st;
}

}  // namespace qmm
