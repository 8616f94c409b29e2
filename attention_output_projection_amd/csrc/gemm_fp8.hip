// gemm_fp8.hip -- step a3 on gfx950: the grouped wo_a contraction
//   z[t][g][n] = sum_k (a[t,g,k] * sa[t,g,k/128]) * (w[g*R+n][k] * sw(g*R+n, k/128))
// (vLLM API page "vllm.models.deepseek_v4.nvidia.ops.o_proj",
// deep_gemm_fp8_o_proj: einsum "bhr,hdr->bhd" over wo_a viewed [G, R, D];
// vLLM API page "vllm.models.deepseek_v4.common.grouped_wo_a": group g meets
// only weight rows g*R .. g*R+R-1; sglang source page
// "python/sglang/srt/models/deepseek_v4.py", _dequant_fp8: weight scales
// multiply 128x128 blocks).
//
// Matrix cores: v_mfma_f32_16x16x128_f8f6f4 (one instruction spans a whole
// 128-deep quantisation block).  Operand fragments: lane l holds row l%16 of
// the 16-row A (or B) slab and the 32 K-bytes 32*(l/16)..+31 of the block;
// A and B use the same K assignment, so the sum over K is the block's dot
// product.  Result: lane l holds C[4*(l/16)+i][l%16], i = 0..3.
//
// Block scales:
//  * fp32 recipe: each 128-deep MFMA writes a fresh fp32 partial P, folded
//    into the accumulator as acc = fma(P, sa[row]*sw[col], acc) (sw is one
//    value per 128 output columns in the 128x128 weight recipe, so the
//    product sa*sw is formed once per row and K-block and reused across the
//    wave's column subtiles);
//  * pow2 recipe (both scale sets are powers of two): the block-scaled MFMA
//    v_mfma_scale_f32_16x16x128_f8f6f4 applies the E8M0 exponents of sa and
//    sw in the matrix core and accumulates directly; no VALU work per block.
//
// Two kernels share this machinery:
//  * tile kernel (large T): 128x128 output tile per 256-thread workgroup,
//    2x2 waves of 64x64, A/B K-blocks staged through double-buffered LDS
//    (rows padded to 144 bytes so the 16-lane fragment reads hit distinct
//    banks), one barrier per K-block;
//  * decode kernel (small T): 64x64 output tile per workgroup, the four waves
//    split the K-blocks (interleaved, so their loads of one weight row are
//    adjacent), fragments loaded straight from global memory into registers
//    with a one-block register prefetch, partials summed through LDS.  The
//    weight stream is the cost at small T; no LDS staging is needed.
// Both remap workgroups so that tiles of one group land on one XCD (a group's
// activations and weights then stay in that XCD's L2).
#include "device_common.hpp"
#include "kernels.hpp"

namespace oproj {

namespace {

struct GParams {
    const uint8_t* a;
    const float* sa;
    const uint8_t* w;
    const float* sw;
    uint16_t* z;
    int64_t T, G, D, R, KB;
    int64_t st, sg, sst, ssg, sskb;
    int64_t mtiles, ntiles;
    int w_shift;  // 7: 128x128 weight scales; 0: per row
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_fp8_mx(const v8i& a, const v8i& b, const v4f& c, int ea,
                                           int eb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// Spread consecutive workgroup ids over the 8 XCDs so that a contiguous range
// of tiles (same group) runs on one XCD.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks) {
    if (nblocks % 8 != 0) return bid;
    return (bid % 8) * (nblocks / 8) + bid / 8;
}

__device__ __forceinline__ int64_t wscale_index(const GParams& p, int64_t wrow, int64_t kb) {
    return (wrow >> p.w_shift) * p.KB + kb;
}

// ---------------------------------------------------------------------------
// Tile kernel
constexpr int TBM = 128, TBN = 128, LROW = 144;

template <bool MX, bool W1>
__global__ __launch_bounds__(256) void gemm_fp8_tile_kernel(GParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][TBM * LROW];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][TBN * LROW];
    __shared__ __attribute__((aligned(16))) float sSA[2][TBM];
    __shared__ __attribute__((aligned(16))) float sSW[2][TBN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nblocks = p.G * p.mtiles * p.ntiles;
    const int64_t tile = xcd_remap(blockIdx.x, nblocks);
    const int64_t g = tile / (p.mtiles * p.ntiles);
    const int64_t mt = (tile / p.ntiles) % p.mtiles;
    const int64_t nt = tile % p.ntiles;
    const int64_t m0 = mt * TBM, n0 = nt * TBN;

    // global -> register staging: 1024 16-byte chunks per operand, 4 per thread
    const int crow = tid >> 3;       // + 32*i
    const int ccol = (tid & 7) * 16; // byte offset in the 128-byte K-block row
    const uint8_t* aptr[4];
    const uint8_t* bptr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t m = m0 + crow + 32 * i;
        m = m < p.T ? m : p.T - 1;  // rows past T are computed but never stored
        aptr[i] = p.a + m * p.st + g * p.sg + ccol;
        int64_t n = n0 + crow + 32 * i;
        n = n < p.R ? n : p.R - 1;
        bptr[i] = p.w + (g * p.R + n) * p.D + ccol;
    }
    const float* saptr = nullptr;
    const float* swptr = nullptr;
    if (tid < TBM) {
        int64_t m = m0 + tid;
        m = m < p.T ? m : p.T - 1;
        saptr = p.sa + m * p.sst + g * p.ssg;
    } else {
        int64_t n = n0 + (tid - TBM);
        n = n < p.R ? n : p.R - 1;
        swptr = p.sw + wscale_index(p, g * p.R + n, 0);
    }

    // staging registers; macros (not lambdas) keep them out of scratch
    uint4 ra[4], rb[4];
    float rs;
#define OPROJ_GLOAD(kb)                                                            \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                \
        ra[i] = *reinterpret_cast<const uint4*>(aptr[i] + (kb) * 128);             \
        rb[i] = *reinterpret_cast<const uint4*>(bptr[i] + (kb) * 128);             \
    }                                                                              \
    rs = (tid < TBM) ? saptr[(kb) * p.sskb] : swptr[(kb)];
#define OPROJ_SWRITE(buf)                                                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                \
        *reinterpret_cast<uint4*>(&sA[buf][(crow + 32 * i) * LROW + ccol]) = ra[i]; \
        *reinterpret_cast<uint4*>(&sB[buf][(crow + 32 * i) * LROW + ccol]) = rb[i]; \
    }                                                                              \
    if (tid < TBM)                                                                 \
        sSA[buf][tid] = rs;                                                        \
    else                                                                           \
        sSW[buf][tid - TBM] = rs;

    v4f acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    const int fk = (lane >> 4) * 32;

    OPROJ_GLOAD(0);
    OPROJ_SWRITE(0);
    __syncthreads();

    for (int64_t kb = 0; kb < p.KB; ++kb) {
        const int buf = (int)(kb & 1);
        // unconditional (clamped) prefetch keeps the staging registers out of scratch
        OPROJ_GLOAD(kb + 1 < p.KB ? kb + 1 : kb);

        v8i af[4], bfr[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const uint8_t* src = &sA[buf][(wm * 64 + mi * 16 + frow) * LROW + fk];
            const uint4 lo = *reinterpret_cast<const uint4*>(src);
            const uint4 hi = *reinterpret_cast<const uint4*>(src + 16);
            af[mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const uint8_t* src = &sB[buf][(wn * 64 + ni * 16 + frow) * LROW + fk];
            const uint4 lo = *reinterpret_cast<const uint4*>(src);
            const uint4 hi = *reinterpret_cast<const uint4*>(src + 16);
            bfr[ni] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }

        if constexpr (MX) {
            int ea[4], eb[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) ea[mi] = e8m0_of(sSA[buf][wm * 64 + mi * 16 + frow]);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) eb[ni] = e8m0_of(sSW[buf][wn * 64 + ni * 16 + frow]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = mfma_fp8_mx(af[mi], bfr[ni], acc[mi][ni], ea[mi], eb[ni]);
        } else {
            float sa4[4][4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const float4 t4 = *reinterpret_cast<const float4*>(
                    &sSA[buf][wm * 64 + mi * 16 + 4 * (lane >> 4)]);
                sa4[mi][0] = t4.x;
                sa4[mi][1] = t4.y;
                sa4[mi][2] = t4.z;
                sa4[mi][3] = t4.w;
            }
            if constexpr (W1) {
                float swv[4];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) swv[ni] = sSW[buf][wn * 64 + ni * 16 + frow];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const v4f pp = mfma_fp8(af[mi], bfr[ni], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[mi][ni][i] = __builtin_fmaf(pp[i], sa4[mi][i] * swv[ni], acc[mi][ni][i]);
                    }
            } else {
                const float sws = sSW[buf][wn * 64];  // one weight scale per 64-column span
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    float cmb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) cmb[i] = sa4[mi][i] * sws;
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const v4f pp = mfma_fp8(af[mi], bfr[ni], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[mi][ni][i] = __builtin_fmaf(pp[i], cmb[i], acc[mi][ni][i]);
                    }
                }
            }
        }

        if (kb + 1 < p.KB) { OPROJ_SWRITE(buf ^ 1); }
        __syncthreads();
    }

#undef OPROJ_GLOAD
#undef OPROJ_SWRITE
    // epilogue: bf16 (nearest even), z[t][g][n]
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = m0 + wm * 64 + mi * 16 + 4 * (lane >> 4) + i;
                const int64_t col = n0 + wn * 64 + ni * 16 + frow;
                if (row < p.T && col < p.R)
                    p.z[(row * p.G + g) * p.R + col] = (uint16_t)f32_to_bf16_bits(acc[mi][ni][i]);
            }
}

// ---------------------------------------------------------------------------
// Decode kernel
constexpr int DBM = 64, DBN = 64, kMaxKB = 64;

template <bool MX, bool W1>
__global__ __launch_bounds__(256) void gemm_fp8_decode_kernel(GParams p) {
    // scale staging during the K loop, partial-sum exchange afterwards
    __shared__ __attribute__((aligned(16))) float smem[4 * DBM * DBN];  // 64 KiB
    float* sSA = smem;                      // [KB][64 rows]
    float* sSW = smem + kMaxKB * DBM;       // [KB][64 cols]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t nblocks = p.G * p.mtiles * p.ntiles;
    const int64_t tile = xcd_remap(blockIdx.x, nblocks);
    const int64_t g = tile / (p.mtiles * p.ntiles);
    const int64_t mt = (tile / p.ntiles) % p.mtiles;
    const int64_t nt = tile % p.ntiles;
    const int64_t m0 = mt * DBM, n0 = nt * DBN;

    // stage all scales of the tile: 64 rows x KB and 64 columns x KB
    for (int64_t i = tid; i < p.KB * DBM; i += 256) {
        const int64_t kb = i / DBM, r = i % DBM;
        int64_t m = m0 + r;
        m = m < p.T ? m : p.T - 1;
        sSA[i] = p.sa[m * p.sst + g * p.ssg + kb * p.sskb];
        int64_t n = n0 + r;
        n = n < p.R ? n : p.R - 1;
        sSW[i] = p.sw[wscale_index(p, g * p.R + n, kb)];
    }
    __syncthreads();

    const int frow = lane & 15;
    const int fk = (lane >> 4) * 32;
    const uint8_t* abase[4];
    const uint8_t* bbase[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        int64_t m = m0 + s * 16 + frow;
        m = m < p.T ? m : p.T - 1;
        abase[s] = p.a + m * p.st + g * p.sg + fk;
        int64_t n = n0 + s * 16 + frow;
        n = n < p.R ? n : p.R - 1;
        bbase[s] = p.w + (g * p.R + n) * p.D + fk;
    }

    v4f acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

    auto load_frag = [](const uint8_t* ptr) {
        const uint4 lo = *reinterpret_cast<const uint4*>(ptr);
        const uint4 hi = *reinterpret_cast<const uint4*>(ptr + 16);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    v8i ca[4], cb[4], na[4], nb[4];
    int64_t kb = wave;
    if (kb < p.KB) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            ca[s] = load_frag(abase[s] + kb * 128);
            cb[s] = load_frag(bbase[s] + kb * 128);
        }
    }
    for (; kb < p.KB; kb += 4) {
        const int64_t kn = kb + 4;
        if (kn < p.KB) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                na[s] = load_frag(abase[s] + kn * 128);
                nb[s] = load_frag(bbase[s] + kn * 128);
            }
        }
        const float* sak = sSA + kb * DBM;
        const float* swk = sSW + kb * DBN;
        if constexpr (MX) {
            int ea[4], eb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                ea[s] = e8m0_of(sak[s * 16 + frow]);
                eb[s] = e8m0_of(swk[s * 16 + frow]);
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = mfma_fp8_mx(ca[mi], cb[ni], acc[mi][ni], ea[mi], eb[ni]);
        } else {
            float sa4[4][4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const float4 t4 = *reinterpret_cast<const float4*>(&sak[mi * 16 + 4 * (lane >> 4)]);
                sa4[mi][0] = t4.x;
                sa4[mi][1] = t4.y;
                sa4[mi][2] = t4.z;
                sa4[mi][3] = t4.w;
            }
            if constexpr (W1) {
                float swv[4];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) swv[ni] = swk[ni * 16 + frow];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const v4f pp = mfma_fp8(ca[mi], cb[ni], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[mi][ni][i] = __builtin_fmaf(pp[i], sa4[mi][i] * swv[ni], acc[mi][ni][i]);
                    }
            } else {
                const float sws = swk[0];
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    float cmb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) cmb[i] = sa4[mi][i] * sws;
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const v4f pp = mfma_fp8(ca[mi], cb[ni], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[mi][ni][i] = __builtin_fmaf(pp[i], cmb[i], acc[mi][ni][i]);
                    }
                }
            }
        }
        if (kn < p.KB) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                ca[s] = na[s];
                cb[s] = nb[s];
            }
        }
    }

    // sum the four K-slices: every wave parks its partial tile in LDS
    __syncthreads();  // scale staging is dead from here on
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                smem[wave * (DBM * DBN) + (((mi * 4 + ni) * 4 + i) * 64) + lane] = acc[mi][ni][i];
    __syncthreads();
    const int col = tid & 63;
#pragma unroll 4
    for (int rr = 0; rr < 16; ++rr) {
        const int row = (tid >> 6) + 4 * rr;
        const int mi = row >> 4, i = row & 3, ln = 16 * ((row & 15) >> 2) + (col & 15), ni = col >> 4;
        const int idx = ((mi * 4 + ni) * 4 + i) * 64 + ln;
        const float s = smem[idx] + smem[DBM * DBN + idx] + smem[2 * DBM * DBN + idx] +
                        smem[3 * DBM * DBN + idx];
        const int64_t t = m0 + row, n = n0 + col;
        if (t < p.T && n < p.R) p.z[(t * p.G + g) * p.R + n] = (uint16_t)f32_to_bf16_bits(s);
    }
}

}  // namespace

hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, hipStream_t stream) {
    GParams p;
    p.a = a.a;
    p.sa = a.sa;
    p.w = a.w;
    p.sw = a.sw;
    p.z = a.z;
    p.T = a.T;
    p.G = a.G;
    p.D = a.D;
    p.R = a.R;
    p.KB = a.D / 128;
    p.st = a.lay.stride_t;
    p.sg = a.lay.stride_g;
    p.sst = a.lay.s_stride_t;
    p.ssg = a.lay.s_stride_g;
    p.sskb = a.lay.s_stride_kb;
    p.w_shift = a.w_1x128 ? 0 : 7;
    const bool decode = a.T <= 128 && p.KB <= kMaxKB;
    if (decode) {
        p.mtiles = (a.T + DBM - 1) / DBM;
        p.ntiles = (a.R + DBN - 1) / DBN;
        const dim3 grid((unsigned)(p.G * p.mtiles * p.ntiles));
        if (a.mx) {
            if (a.w_1x128)
                hipLaunchKernelGGL((gemm_fp8_decode_kernel<true, true>), grid, dim3(256), 0, stream, p);
            else
                hipLaunchKernelGGL((gemm_fp8_decode_kernel<true, false>), grid, dim3(256), 0, stream, p);
        } else {
            if (a.w_1x128)
                hipLaunchKernelGGL((gemm_fp8_decode_kernel<false, true>), grid, dim3(256), 0, stream, p);
            else
                hipLaunchKernelGGL((gemm_fp8_decode_kernel<false, false>), grid, dim3(256), 0, stream, p);
        }
    } else {
        p.mtiles = (a.T + TBM - 1) / TBM;
        p.ntiles = (a.R + TBN - 1) / TBN;
        const dim3 grid((unsigned)(p.G * p.mtiles * p.ntiles));
        if (a.mx) {
            if (a.w_1x128)
                hipLaunchKernelGGL((gemm_fp8_tile_kernel<true, true>), grid, dim3(256), 0, stream, p);
            else
                hipLaunchKernelGGL((gemm_fp8_tile_kernel<true, false>), grid, dim3(256), 0, stream, p);
        } else {
            if (a.w_1x128)
                hipLaunchKernelGGL((gemm_fp8_tile_kernel<false, true>), grid, dim3(256), 0, stream, p);
            else
                hipLaunchKernelGGL((gemm_fp8_tile_kernel<false, false>), grid, dim3(256), 0, stream, p);
        }
    }
    return hipGetLastError();
}

}  // namespace oproj
