// gemm_bf16.hip -- step a4 on gfx950: the dense wo_b GEMM over the flattened
// z (sglang source page "python/sglang/srt/models/deepseek_v4.py",
// MQALayer.forward: wo_b is applied to z.flatten(1); wo_b is a linear layer
// from G*R to hidden, weight [hidden, G*R]):
//   y[m][j] = sum_c x[m][c] * w[j][c],  bf16 in, fp32 accumulate, bf16 out.
//
// v_mfma_f32_16x16x32_bf16, 128x128 output tile per 256-thread workgroup
// (2x2 waves of 64x64), K staged 64 deep (128 bytes per row) through
// double-buffered LDS with rows padded to 144 bytes; the accumulators stay in
// the matrix-core result registers for the whole K loop.
#include "device_common.hpp"
#include "kernels.hpp"

namespace oproj {

namespace {

constexpr int BM = 128, BN = 128, BKB = 128 /* bytes of K per stage */, LROW = 144;

struct DParams {
    const uint16_t* x;
    const uint16_t* w;
    uint16_t* y;
    int64_t M, N, K;
    int64_t mtiles, ntiles;
};

__device__ __forceinline__ int64_t xcd_remap_d(int64_t bid, int64_t nblocks) {
    if (nblocks % 8 != 0) return bid;
    return (bid % 8) * (nblocks / 8) + bid / 8;
}

__global__ __launch_bounds__(256) void gemm_bf16_kernel(DParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * LROW];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * LROW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nblocks = p.mtiles * p.ntiles;
    const int64_t tile = xcd_remap_d(blockIdx.x, nblocks);
    const int64_t mt = tile / p.ntiles, nt = tile % p.ntiles;
    const int64_t m0 = mt * BM, n0 = nt * BN;
    const int64_t kbytes = p.K * 2;
    const int64_t nstage = kbytes / BKB;

    const int crow = tid >> 3;
    const int ccol = (tid & 7) * 16;
    const uint8_t* aptr[4];
    const uint8_t* bptr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t m = m0 + crow + 32 * i;
        m = m < p.M ? m : p.M - 1;
        aptr[i] = reinterpret_cast<const uint8_t*>(p.x) + m * kbytes + ccol;
        int64_t n = n0 + crow + 32 * i;
        n = n < p.N ? n : p.N - 1;
        bptr[i] = reinterpret_cast<const uint8_t*>(p.w) + n * kbytes + ccol;
    }
    uint4 ra[4], rb[4];
#define OPROJ_GLOAD(ks)                                                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                \
        ra[i] = *reinterpret_cast<const uint4*>(aptr[i] + (ks) * BKB);             \
        rb[i] = *reinterpret_cast<const uint4*>(bptr[i] + (ks) * BKB);             \
    }
#define OPROJ_SWRITE(buf)                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                \
        *reinterpret_cast<uint4*>(&sA[buf][(crow + 32 * i) * LROW + ccol]) = ra[i]; \
        *reinterpret_cast<uint4*>(&sB[buf][(crow + 32 * i) * LROW + ccol]) = rb[i]; \
    }

    v4f acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    const int fk = (lane >> 4) * 16;

    OPROJ_GLOAD(0);
    OPROJ_SWRITE(0);
    __syncthreads();
    for (int64_t ks = 0; ks < nstage; ++ks) {
        const int buf = (int)(ks & 1);
        // unconditional (clamped) prefetch keeps the staging registers out of scratch
        OPROJ_GLOAD(ks + 1 < nstage ? ks + 1 : ks);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v8bf af[4], bfr[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                af[mi] = *reinterpret_cast<const v8bf*>(&sA[buf][(wm * 64 + mi * 16 + frow) * LROW + h * 64 + fk]);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                bfr[ni] = *reinterpret_cast<const v8bf*>(&sB[buf][(wn * 64 + ni * 16 + frow) * LROW + h * 64 + fk]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
        }
        if (ks + 1 < nstage) { OPROJ_SWRITE(buf ^ 1); }
        __syncthreads();
    }

#undef OPROJ_GLOAD
#undef OPROJ_SWRITE
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = m0 + wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
                const int64_t col = n0 + wn * 64 + ni * 16 + frow;
                if (row < p.M && col < p.N) p.y[row * p.N + col] = (uint16_t)f32_to_bf16_bits(acc[mi][ni][i]);
            }
}

}  // namespace

hipError_t launch_dense_bf16_gemm(const DenseGemmArgs& a, hipStream_t stream) {
    DParams p;
    p.x = a.x;
    p.w = a.w;
    p.y = a.y;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.mtiles = (a.M + BM - 1) / BM;
    p.ntiles = (a.N + BN - 1) / BN;
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3((unsigned)(p.mtiles * p.ntiles)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace oproj
