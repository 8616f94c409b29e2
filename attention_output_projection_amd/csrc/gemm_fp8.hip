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
//  * decode kernel (small T): 64x64 output tile per workgroup, its eight
//    waves split the K-blocks (interleaved, so their loads of one weight row
//    are adjacent), fragments loaded straight from global memory into
//    registers with a one-block register prefetch, partials summed through
//    LDS.  The weight stream is the cost at small T: eight waves per CU keep
//    enough of it in flight; no LDS staging is needed.
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
// Decode kernel (few tokens): the weight stream is the cost.
// Workgroup tile: one group, 64 tokens x 64 columns, the whole K.  Each
// K-block is one pipeline stage in LDS: the 64x128-byte activation slab, the
// 64x128-byte weight slab and the block's scales, all copied by the DMA form
// of the global loads (global_load_lds: no staging registers).  DNS stages
// form a ring, DNS-1 of them in flight; one s_waitcnt + barrier per K-block.
// Every wave issues the same five copies per stage (1 KiB x 2 activation rows
// groups, 1 KiB x 2 weight row groups, one scale gather), so the wait count is
// a constant.  Rows are 128 bytes with the 16-byte pieces XOR-swizzled by
// (row >> 1) & 7, which makes the 16-row fragment reads conflict-free.
// Waves split N (wave w owns columns 16w..16w+15): no partial-sum exchange.
constexpr int DBM = 64, DBN = 64, DNS = 4, DKS = 2;
constexpr int DSTAGE = 64 * 128 * 2 + 1024;  // activations + weights + scales

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// LDS byte offset of a __shared__ address, made wave-uniform (an SGPR).
__device__ __forceinline__ uint32_t lds_offset(const uint8_t* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_u8*)p);
}

// DMA copies global -> LDS (global_load_lds): lane i's 16 (or 4) bytes land
// at lds + 16*i (4*i); `lds` is made wave-uniform and goes to M0.  Written as
// asm: the compiler cannot tell these LDS writes from the ring slots being
// read and would otherwise wait for every copy before each LDS read; all
// waits for the copies are explicit (wait_vmcnt).  Nothing else in the
// kernels that use them keeps a value in M0.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <bool MX, bool W1>
__global__ __launch_bounds__(DKS * 256) void gemm_fp8_decode_kernel(GParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[DKS][DNS][DSTAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int kq = tid >> 8;            // K quarter/half handled by this wave group
    const int wave = (tid >> 6) & 3;    // column group within the tile
    const int64_t nblocks = p.G * p.mtiles * p.ntiles;
    const int64_t tile = xcd_remap(blockIdx.x, nblocks);
    const int64_t g = tile / (p.mtiles * p.ntiles);
    const int64_t mt = (tile / p.ntiles) % p.mtiles;
    const int64_t nt = tile % p.ntiles;
    const int64_t m0 = mt * DBM, n0 = nt * DBN;
    // this wave group's K-blocks: [kb0, kb0 + nkb)
    const int64_t kb0 = p.KB * kq / DKS;
    const int64_t nkb = p.KB * (kq + 1) / DKS - kb0;
    const int64_t klast = kb0 + (nkb > 0 ? nkb : 1) - 1;

    // ---- per-lane copy sources (the K-block offset is added per stage)
    const uint8_t* asrc[2];
    const uint8_t* wsrc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 16 * wave + 8 * j + (lane >> 3);
        const int piece = (lane & 7) ^ swz(row);
        int64_t m = m0 + row;
        m = m < p.T ? m : p.T - 1;  // rows past T are computed but never stored
        asrc[j] = p.a + m * p.st + g * p.sg + piece * 16;
        int64_t n = n0 + row;
        n = n < p.R ? n : p.R - 1;
        wsrc[j] = p.w + (g * p.R + n) * p.D + piece * 16;
    }
    // scale gather: lanes 0-15 activation scales of tokens 16w+l, lanes 16-31
    // weight scales of columns 16w+l-16; lanes 32-63 repeat them (junk slots)
    const float* ssrc;
    int64_t sstep;
    {
        const int l = lane & 31;
        if (l < 16) {
            int64_t m = m0 + 16 * wave + l;
            m = m < p.T ? m : p.T - 1;
            ssrc = p.sa + m * p.sst + g * p.ssg;
            sstep = p.sskb;
        } else {
            int64_t n = n0 + 16 * wave + (l - 16);
            n = n < p.R ? n : p.R - 1;
            ssrc = p.sw + wscale_index(p, g * p.R + n, 0);
            sstep = 1;
        }
    }
    const uint32_t ring0 = lds_offset(&ring[kq][0][0]);
    auto issue = [&](int64_t i, int slot) __attribute__((always_inline)) {
        int64_t kb = kb0 + i;
        kb = kb < klast ? kb : klast;  // tail stages re-copy the last block into a dead slot
        const uint32_t st = ring0 + (uint32_t)(slot * DSTAGE);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            dma16(asrc[j] + kb * 128, st + (16 * wave + 8 * j) * 128);
            dma16(wsrc[j] + kb * 128, st + 8192 + (16 * wave + 8 * j) * 128);
        }
        dma4(ssrc + kb * sstep, st + 16384 + 256 * wave);
    };

#pragma unroll
    for (int s = 0; s < DNS - 1; ++s) issue(s, s);

    v4f acc[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) acc[mi] = v4f{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    const int p0 = 2 * (lane >> 4);
    const int64_t nstages = p.KB / DKS + 1;  // >= nkb for every group: same barrier count
    for (int64_t i = 0; i < nstages; ++i) {
        wait_vmcnt<5 * (DNS - 2)>();  // this wave's copies of stage i have landed
        __builtin_amdgcn_s_barrier();  // ... and every other wave's (no fence: the
                                       // prefetches stay in flight)
        issue(i + DNS - 1, (int)((i + DNS - 1) % DNS));
        if (i >= nkb) continue;        // uniform per wave group
        const uint8_t* st = ring[kq][i % DNS];
        v8i bfr;
        {
            const int r = 16 * wave + frow;
            const uint4 lo = *reinterpret_cast<const uint4*>(st + 8192 + r * 128 + 16 * (p0 ^ swz(r)));
            const uint4 hi = *reinterpret_cast<const uint4*>(st + 8192 + r * 128 + 16 * ((p0 + 1) ^ swz(r)));
            bfr = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        const float* sc = reinterpret_cast<const float*>(st + 16384);
        const float swv = sc[64 * wave + 16 + (W1 || MX ? frow : 0)];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int r = 16 * mi + frow;
            const uint4 lo = *reinterpret_cast<const uint4*>(st + r * 128 + 16 * (p0 ^ swz(r)));
            const uint4 hi = *reinterpret_cast<const uint4*>(st + r * 128 + 16 * ((p0 + 1) ^ swz(r)));
            const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            if constexpr (MX) {
                acc[mi] = mfma_fp8_mx(af, bfr, acc[mi], e8m0_of(sc[64 * mi + frow]), e8m0_of(swv));
            } else {
                const float4 t4 = *reinterpret_cast<const float4*>(&sc[64 * mi + 4 * (lane >> 4)]);
                const float cmb[4] = {t4.x * swv, t4.y * swv, t4.z * swv, t4.w * swv};
                const v4f pp = mfma_fp8(af, bfr, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) acc[mi][i2] = __builtin_fmaf(pp[i2], cmb[i2], acc[mi][i2]);
            }
        }
    }
    wait_vmcnt<0>();  // no copy may still be writing LDS
    __syncthreads();

    // ---- sum the K groups through LDS (ring 0 of group 0 is free now)
    float* red = reinterpret_cast<float*>(&ring[0][0][0]);
    if constexpr (DKS > 1) {
        if (kq > 0) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[((kq - 1) * 256 + (wave * 64 + lane)) * 16 + mi * 4 + i] = acc[mi][i];
        }
        __syncthreads();
        if (kq > 0) return;
#pragma unroll
        for (int q = 1; q < DKS; ++q)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[mi][i] += red[((q - 1) * 256 + (wave * 64 + lane)) * 16 + mi * 4 + i];
    }

    // ---- bf16 results of this wave's 16 columns
    const int64_t col = n0 + 16 * wave + frow;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = m0 + mi * 16 + 4 * (lane >> 4) + i;
            if (row < p.T && col < p.R) p.z[(row * p.G + g) * p.R + col] = (uint16_t)f32_to_bf16_bits(acc[mi][i]);
        }
}

void launch_decode(const GParams& p, bool mx, bool w1, hipStream_t stream) {
    const dim3 grid((unsigned)(p.G * p.mtiles * p.ntiles)), block(DKS * 256);
    if (mx) {
        if (w1)
            hipLaunchKernelGGL((gemm_fp8_decode_kernel<true, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_fp8_decode_kernel<true, false>), grid, block, 0, stream, p);
    } else {
        if (w1)
            hipLaunchKernelGGL((gemm_fp8_decode_kernel<false, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_fp8_decode_kernel<false, false>), grid, block, 0, stream, p);
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
    // decode kernel for few tokens (the weight stream dominates), tile kernel otherwise
    const bool decode = a.T <= 128;
    if (decode) {
        p.mtiles = (a.T + DBM - 1) / DBM;
        p.ntiles = (a.R + DBN - 1) / DBN;
        launch_decode(p, a.mx != 0, a.w_1x128 != 0, stream);
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
