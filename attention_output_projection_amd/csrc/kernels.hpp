// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to the
// library; the public C ABI is include/oproj.h).  Arguments arrive validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oproj {

// Compute units and XCDs (chiplets with their own L2) of the current device,
// queried from the HIP runtime once per device and cached; the launchers size
// their grids and tile orders from it.
struct DeviceInfo {
    int cus;
    int xcds;
};
DeviceInfo current_device_info();

struct ActLayout {
    int64_t stride_t, stride_g;              // codes, bytes == elements
    int64_t s_stride_t, s_stride_g, s_stride_kb;  // scales, 4-byte words (fp32 or packed UE8M0)
};

struct RopeQuantArgs {
    int64_t T, G, hpg, max_pos;
    int pow2;
    int e8m0;                 // write packed UE8M0 words (one per head: 4 blocks) instead of fp32
    const uint16_t* o;        // bf16 [T][G*hpg][512]
    const float* o_f32;       // or fp32 [T][G*hpg][512] (then o is unused)
    const int64_t* positions; // [T]
    const float* cos_sin;     // [max_pos][64]
    uint8_t* codes;
    void* scales;             // fp32 per block, or uint32 UE8M0 words
    ActLayout lay;
};
hipError_t launch_inv_rope_quant(const RopeQuantArgs& a, hipStream_t s);

struct WeightQuantArgs {
    int64_t rows, K, brows;
    int pow2;
    int e8m0;  // write UE8M0 bytes (packed four per word along K) instead of fp32
    const float* w;
    uint8_t* codes;
    void* scales;
};
hipError_t launch_quantize_weight(const WeightQuantArgs& a, hipStream_t s);

struct GroupedGemmArgs {
    int64_t T, G, D, R;
    int mx;        // both scale sets are powers of two: use block-scaled MFMA
    int w_1x128;   // weight scales per row (else 128x128 tiles of the flat matrix)
    int a_e8m0;    // activation scales are packed UE8M0 words (implies mx)
    int w_e8m0;    // weight scales are packed UE8M0 words, per row (implies mx and w_1x128)
    const uint8_t* a;
    const void* sa;
    ActLayout lay;
    const uint8_t* w;
    const void* sw;  // fp32 scales or packed UE8M0 words
    uint16_t* z;   // bf16 [T][G][R]
};
hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, hipStream_t s);

// One launch for both steps at few tokens (quantisation into the default
// layout of q's buffers, then the grouped GEMM reading them).  *launched is
// false, and nothing is enqueued, when the shape does not fit that path.
// `sync` holds one 128-byte barrier word line per group (zero before the first
// launch with it; each launch leaves it ready for the next); launches that
// overlap in time need distinct `sync` regions.
hipError_t launch_fused_decode(const RopeQuantArgs& q, const GroupedGemmArgs& a, uint64_t* sync, hipStream_t s,
                               bool* launched);
constexpr size_t kFusedDecodeSyncBytesPerGroup = 128;
// Why that path cannot take a call of this shape on the current device
// (static text), or nullptr when it can.
const char* fused_decode_unfit(int64_t T, int64_t G, int64_t hpg, int64_t R);

struct RopeBf16Args {
    int64_t T, G, hpg, max_pos;
    const uint16_t* o;         // bf16 [T][G*hpg][512]
    const int64_t* positions;  // [T]
    const float* cos_sin;      // [max_pos][64]
    uint16_t* x;               // bf16 x(t, g, k) at x[t*stride_t + g*stride_g + k]
    int64_t stride_t, stride_g;
};
hipError_t launch_inv_rope_bf16(const RopeBf16Args& a, hipStream_t s);

// Grouped bf16 GEMM: for g < G, y_g[m][n] = sum_k x_g[m][k] * w_g[n][k] with
// x_g = x + g*gx (row stride sx), w_g = w + g*gw (rows of K), y_g = y + g*gy
// (row stride sy); all in elements.
struct Bf16GemmArgs {
    int64_t G, M, N, K;
    const uint16_t* x;
    const uint16_t* w;
    uint16_t* y;
    int64_t sx, sy, gx, gw, gy;
};
hipError_t launch_bf16_gemm(const Bf16GemmArgs& a, hipStream_t s);

struct DenseGemmArgs {
    int64_t M, N, K;
    const uint16_t* x;  // bf16 [M][K]
    const uint16_t* w;  // bf16 [N][K]
    uint16_t* y;        // bf16 [M][N]
};
hipError_t launch_dense_bf16_gemm(const DenseGemmArgs& a, hipStream_t s);

}  // namespace oproj
