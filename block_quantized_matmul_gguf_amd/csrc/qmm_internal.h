// qmm_internal.h -- interface between the host plan/dispatch code and the
// kernel launchers.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

enum { FMT_Q4_0 = 2, FMT_Q5_0 = 6, FMT_Q8_0 = 8, FMT_Q4_K = 12, FMT_Q6_K = 14, FMT_Q8_K = 15 };
enum { MODE_A = 0, MODE_B = 1, MODE_DEQ = 2 };

// Decode (GEMV) path: M <= 8 rows; 512-thread workgroups of eight waves,
// each wave streaming 16-row tiles over one slice of K.
constexpr int GEMV_MAX_M = 8;

struct GemvGeom {
    int nlu;          // load units per row (Q8_0 block pairs or Q4_K super-blocks)
    int64_t row_bytes;
    int tiles;        // 16-row tiles
    int ks;           // K splits across workgroups
    int lus_split;    // load units per split
    int kw;           // waves per tile (K slices inside a workgroup)
    int slice;        // load units per wave slice
    int P;            // load units per stage
    int R;            // activation rows per lane the arithmetic covers (1 or 4)
    int G;            // tiles per workgroup step
    int groups;       // tile groups per split
    int gpw;          // tile groups per workgroup
    int rs;           // LDS row stride of the per-wave weight stage buffer (bytes)
    int D;            // stage buffers per wave filled by LDS-direct loads (0: register staging)
    int sc_off, red_off, misc_off, stg_off, lds;  // LDS layout (bytes)
    int grid;         // workgroups
};

// Device buffers of the decode path inside a plan's workspace.
struct GemvBufs {
    float* part;   // split-K partials [ks][8][N]
};

// Device buffers of the prefill path.
struct GemmBufs {
    _Float16* a0;   // mode (a): hi part of the scaled activation rows [M][K]; mode (b): the quantized
                    // activations as int8 [M][K]
    _Float16* a1;   // lo part [M][K]
    float* rs;      // 1/s per row [M]
    _Float16* xs;   // Q4_K mode (a): hi and lo of s * (sub-block sums) / 32; mode (b): the Q8K
                    // sub-block sums as multiples of 64 and remainders; [M][K/256][16]
    float* sd;      // mode (b): activation block scales, block-major [K/32 or K/256][M]
};

// Outputs of a traced run (mode (b)): the kernels that compute y also write
// the integer block sums they form and the quantized activations they use.
struct Trace {
    int32_t* sums;  // [M][N][block sums per row], see qmatmul_run_traced
    uint8_t* act;   // canonical Q8_0 / Q8K blocks of x [M][row bytes], or null
};

GemvGeom gemv_geom(int fmt, int mode, int64_t N, int64_t K, int M, bool emit);
int device_cus();  // compute units of the current device (cached per device)

// Decode with one activation row, weights streamed row by row.
bool gemv_row_supported(int fmt, int mode, int M, int64_t N, int64_t K, bool emit);
hipError_t launch_gemv_row(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, float* y, hipStream_t s,
                           const Trace* tr = nullptr);
// Several problems sharing x and K (their rows end to end) in one launch; at
// most gemv_row_group_max() of them.
int gemv_row_group_max();
hipError_t launch_gemv_row_group(int fmt, int mode, int count, const void* const* w, const int64_t* Ns, float* const* y,
                                 const float* x, int64_t K, hipStream_t s, const Trace* tr = nullptr);
bool gemv_supported(int fmt, int64_t K);
int gemv_max_splits(int fmt, int64_t K);

hipError_t launch_quantize_act(int act_fmt, const float* x, int64_t M, int64_t K, void* out, hipStream_t s);
hipError_t launch_quantize_weights(int fmt, const float* w, int64_t N, int64_t K, void* out, hipStream_t s);
hipError_t launch_quantize_q4_k_search(const float* w, int64_t N, int64_t K, void* out, hipStream_t s);

// Decode with 2..8 f32 activation rows (mode (a), Q8_0 and Q4_K, K <= 4096):
// the activation operand in registers, K split over the eight waves.
bool gemv_reg_supported(int fmt, int mode, int M, int64_t N, int64_t K);
hipError_t launch_gemv_reg(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, int M, float* y,
                           hipStream_t s, const Trace* tr);

hipError_t launch_gemv(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, int M,
                       const GemvBufs& b, float* y, hipStream_t s, const Trace* tr = nullptr);

// act != null (mode (b), traced runs): the canonical activation blocks as well
hipError_t launch_gemm_prep(int fmt, int mode, const float* x, int64_t M, int64_t K, const GemmBufs& b, hipStream_t s,
                            uint8_t* act = nullptr);
// sums (mode (b) only): the traced run, see launch_gemm_q
hipError_t launch_gemm(int fmt, int mode, const void* w, int64_t N, int64_t K, int64_t M, const GemmBufs& b,
                       float* y, hipStream_t s, int32_t* sums = nullptr);
// sums != null: the same kernel also writes its int32 block sums (Q8_0: S per
// block; Q4_K: S_0..S_7, sumi (from the S_j and the weight scales) and summins
// per super-block); y may then be null.
hipError_t launch_gemm_q(int fmt, const void* w, int64_t N, int64_t K, int64_t M, const GemmBufs& b, float* y,
                         hipStream_t s, int32_t* sums = nullptr);
// Grouped prefill: count (<= 4) problems sharing K, the mode and the prepared
// activations b in one launch, each output computed as its own launch would.
hipError_t launch_gemm_group(int fmt, int mode, int count, const void* const* w, const int64_t* Ns, float* const* y,
                             int64_t K, int64_t M, const GemmBufs& b, hipStream_t s, int32_t* sums = nullptr);
hipError_t launch_gemm_q_group(int fmt, int count, const void* const* w, const int64_t* Ns, float* const* y,
                               int64_t K, int64_t M, const GemmBufs& b, hipStream_t s, int32_t* sums = nullptr);
int gemm_group_max();
// Q8_0, Q4_0 and Q5_0 prefill with short rows (M > 8, K % 64 == 0, K <= 1536,
// at most 8192 output columns, a grid of one round per problem): one launch that prepares its own
// activations (no preparation launch, no workspace); count (<= 4) problems
// share K, the mode and x; a traced run (tr, mode (b), count == 1) also writes
// the block sums [M][N][K/32] and the canonical activation blocks.
bool gemm_s_supported(int fmt, int mode, int64_t K, int64_t Ntot, int64_t M);
hipError_t launch_gemm_s(int fmt, int mode, int count, const void* const* w, const int64_t* Ns, float* const* y,
                         const float* x, int64_t K, int64_t M, hipStream_t s, const Trace* tr = nullptr);

// Q4_0, Q5_0 and Q6_K weights.  Decode runs (and every Q6_K run) take the
// ext kernels; Q4_0/Q5_0 prefill transcodes the weights to Q8_0 blocks (same
// dequantized values, same integer block sums) and runs the Q8_0 kernels.
struct ExtBufs {
    int8_t* xq;   // mode (b): quantized activations int8 [M][K]
    float* xd;    // their scales [M][K/32] or [M][K/256]
    int32_t* xs;  // sums of their values [M][K/32] or [M][K/16]
    uint8_t* tw;  // Q4_0/Q5_0 prefill: the weights as Q8_0 blocks [N][K/32][34]
};
bool is_ext_format(int fmt);
int64_t ext_block_bytes(int fmt);
hipError_t launch_ext_prep(int fmt, const float* x, int64_t M, int64_t K, const ExtBufs& b, hipStream_t s,
                           uint8_t* act = nullptr);
// tr != null (mode (b)): the traced run, y may then be null
hipError_t launch_ext_run(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, int64_t M,
                          const ExtBufs& b, float* y, hipStream_t s, const Trace* tr = nullptr);
// Grouped decode (M <= 8): up to ext_group_max() problems sharing K, mode and
// x in one launch; b is the first problem's workspace.
int ext_group_max();
bool ext_group_supported(int fmt, int mode, int64_t K, int64_t M);  // the activations fit in LDS
hipError_t launch_ext_group(int fmt, int mode, int count, const void* const* w, const int64_t* Ns, float* const* y,
                            const float* x, int64_t K, int64_t M, const ExtBufs& b, hipStream_t s);
hipError_t launch_ext_to_q8_0(int fmt, const void* w, int64_t N, int64_t K, void* out, hipStream_t s);
hipError_t launch_ext_dequantize(int fmt, const void* w, int64_t N, int64_t K, float* out, hipStream_t s);
hipError_t launch_ext_quantize_weights(int fmt, const float* w, int64_t N, int64_t K, void* out, hipStream_t s);

// Dequantize-all form: GGUF blocks -> f32 [N][K], and the plain f32 GEMM
// (rocBLAS) behind an opaque handle; dense_* return 0 on success.
hipError_t launch_dequantize(int fmt, const void* w, int64_t N, int64_t K, float* out, hipStream_t s);
int dense_create(void** handle);
void dense_destroy(void* handle);
int dense_gemm(void* handle, const float* w, const float* x, float* y, int64_t M, int64_t N, int64_t K,
               hipStream_t s);

// Odd block counts of the 32-value formats: rows copied one all-zero block
// longer (src/dst row bytes), x copied with K..Kp-1 zero; and the traced
// outputs of such a run cut back (of every `from` items of `unit` bytes keep
// the first `keep`).
hipError_t launch_pad(const void* w, int64_t N, int src_row_bytes, int dst_row_bytes, void* wpad, const float* x,
                      int64_t M, int64_t K, int64_t Kp, float* xpad, hipStream_t s);
hipError_t launch_unpad(const void* src, int64_t groups, int from, int keep, int unit, void* dst, hipStream_t s);

// Plan-free run on caller-provided device memory (the no-allocation entry
// point; dry_run: the argument checks only, no HIP call), and setting the
// calling thread's error message.
int run_on_scratch(int format, int64_t N, int64_t K, int64_t M, int mode, const void* w, const float* x, float* y,
                   void* scratch, size_t scratch_bytes, void* stream, bool dry_run);
int set_error(int code, const char* msg);

}  // namespace qmm
