// qmm_internal.h -- interface between the host plan/dispatch code and the
// kernel launchers.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

enum { FMT_Q8_0 = 8, FMT_Q4_K = 12, FMT_Q8_K = 15 };
enum { MODE_A = 0, MODE_B = 1 };

// Decode (GEMV) path: M <= 8 rows; 256-thread workgroups of four waves, each
// wave streaming 16-row tiles of one K split.
constexpr int GEMV_MAX_M = 8;
constexpr int GEMV_MAX_SPLITS = 16;
constexpr int GEMV_STAGE_BYTES = 9792;  // per-wave weight staging buffer (16 rows)

// Prefill (GEMM) path tile.
constexpr int GEMM_BM = 128;
constexpr int GEMM_BN = 128;
constexpr int GEMM_KS = 64;

struct GemvGeom {
    int units;        // weight blocks per row (Q8_0: 32 values, Q4_K: 256)
    int unit_bytes;   // 34 or 144
    int64_t row_bytes;
    int tiles;        // 16-row tiles
    int ks;           // K splits
    int ups;          // units per K split
    int full_rows;    // 1: stage whole rows (the 16-row tile is contiguous)
    int su;           // units per stage when staging row segments
    int upw;          // tiles per wave
    int grid;         // workgroups
};

// Device buffers of the decode path inside a plan's workspace.
struct GemvBufs {
    float* part;   // split-K partials [ks][8][N]
};

// Device buffers of the prefill path.
struct GemmBufs {
    _Float16* a0;  // mode a: hi part [M][K]; mode b: quantized activations as f16 [M][K]
    _Float16* a1;  // mode a: lo part [M][K]
    float* sc0;    // mode a: 1/row scale [M]; mode b: act block scales [M][K/32 or K/256]
    void* sc1;     // mode a Q4_K: scaled sub-block sums [M][K/32] f32; mode b Q4_K: bsum pairs [M][K/32] i32
};

GemvGeom gemv_geom(int fmt, int mode, int64_t N, int64_t K, int M, int max_wgs);
bool gemv_supported(int fmt, int64_t K);
int gemv_max_splits(int fmt, int64_t K);

hipError_t launch_quantize_act(int act_fmt, const float* x, int64_t M, int64_t K, void* out, hipStream_t s);
hipError_t launch_quantize_weights(int fmt, const float* w, int64_t N, int64_t K, void* out, hipStream_t s);

hipError_t launch_gemv(int fmt, int mode, const void* w, const float* x, int64_t N, int64_t K, int M,
                       const GemvBufs& b, float* y, int32_t* sums, hipStream_t s);

hipError_t launch_gemm_prep(int fmt, int mode, const float* x, int64_t M, int64_t K, const GemmBufs& b, hipStream_t s);
hipError_t launch_gemm(int fmt, int mode, const void* w, int64_t N, int64_t K, int64_t M, const GemmBufs& b,
                       float* y, int32_t* sums, hipStream_t s);

}  // namespace qmm
