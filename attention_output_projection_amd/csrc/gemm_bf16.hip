// gemm_bf16.hip -- bf16 GEMMs on gfx950, y[m][j] = sum_c x[m][c] * w[j][c]
// with bf16 inputs, fp32 accumulation and bf16 output, for
//  * step a4, the dense wo_b GEMM over the flattened z (sglang source page
//    "python/sglang/srt/models/deepseek_v4.py", MQALayer.forward: wo_b is
//    applied to z.flatten(1), a linear layer from G*R to hidden with weight
//    [hidden, G*R]; vLLM API page "vllm.models.deepseek_v4.nvidia.ops.o_proj",
//    deep_gemm_fp8_o_proj ends with wo_b(z.flatten(1)));
//  * the unquantised grouped wo_a (same page, deep_gemm_fp8_o_proj without
//    FP8: a batched matmul of the bf16 groups [G, T, D] with wo_a viewed
//    [G, R, D]), one independent GEMM per group with strided operands.
//
// Same pipeline as the FP8 tile kernel: 256 x (32*NI) output tile per
// 512-thread workgroup, eight waves as 4 (M) x 2 (N) of 64 x (16*NI), one
// 64-deep K-step (128 bytes of every row) per stage, stages double-buffered in
// LDS and filled by DMA copies (global_load_lds) into XOR-swizzled 128-byte
// rows.  Waves 0-3 issue the copies (waves 0-1 right after the barrier,
// waves 2-3 in the middle of the K-step: two half-size bursts on the DMA
// path), waves 4-7 only compute.  NI = 8 gives 256x256 tiles; NI = 7 gives
// 256x224 tiles, which the launcher picks when they divide the grid into
// fuller rounds of 256 workgroups (hidden = 7168 = 32 x 224); NI = 2 gives
// 256x64 tiles for grids too small to fill the chip with wide tiles (few
// tokens).  MFMA v_mfma_f32_16x16x32_bf16: a lane's two 16-byte pieces of a
// row (pieces 2q and 2q+1 for lane group q) feed the two K=32 halves of the
// step, in the same order for both operands, so the pair of MFMAs sums the
// whole 64-deep step.  The accumulators stay in the matrix-core result
// registers for the whole K loop.  Tiles are walked in bands of four M-tiles
// (the N-tiles of a band share its activation rows) and consecutive tiles are
// kept on one XCD.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"

namespace oproj {

namespace {

constexpr int BM = 256, NW = 8;
constexpr int BAND = 4;  // M-tiles per band of the tile order

struct DParams {
    const uint16_t* x;
    const uint16_t* w;
    uint16_t* y;
    int64_t M, N, K;
    int64_t sx, sy, gx, gw, gy;  // row and group strides, elements
    int64_t G, mtiles, ntiles;   // tiles per group: mtiles x ntiles
    uint32_t tpg;                // mtiles * ntiles
    uint32_t xcd_per;            // tiles per XCD when the XCD remap applies, else 0
    int xcd_shift;               // log2 of the XCD count (a power of two) when it applies
};

// Workgroup ids are dealt to the XCDs round-robin: map them to tile numbers
// such that each XCD runs one contiguous range of tiles, and split off the
// group.  32-bit scalar arithmetic on counts the host prepares.
struct GroupTile {
    uint32_t g, id;  // group, tile within the group
};
__device__ __forceinline__ GroupTile group_tile(const DParams& p) {
    const uint32_t b = blockIdx.x;
    const uint32_t t =
        p.xcd_per ? (b & ((1u << p.xcd_shift) - 1u)) * p.xcd_per + (b >> p.xcd_shift) : b;
    const uint32_t g = t / p.tpg;
    return {g, t - g * p.tpg};
}

template <int NI>
__global__ __launch_bounds__(NW * 64) void gemm_bf16_kernel(DParams p) {
    constexpr int BN = 32 * NI;                          // tile columns
    constexpr int SA = 0, SB = BM * 128, STAGE = SB + BN * 128;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[2][STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
    const int wm = wave & 3, wn = wave >> 2;
    const GroupTile gt = group_tile(p);
    const int64_t g = gt.g;
    // band order: BAND M-tiles x all N-tiles, M fastest within the band
    const uint32_t ntl = (uint32_t)p.ntiles, mtl = (uint32_t)p.mtiles;
    const uint32_t band = gt.id / (BAND * ntl);
    const uint32_t mfirst = band * BAND;
    const uint32_t bh = (mtl - mfirst) < BAND ? (mtl - mfirst) : BAND;
    const uint32_t local = gt.id - band * BAND * ntl;
    const uint32_t nt = local / bh, mt = mfirst + (local - nt * bh);
    const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;
    const int64_t kbytes = p.K * 2, xrow = p.sx * 2;
    const int64_t nstage = kbytes / 128;

    // ---- copy plan: copying wave c (0-3) moves activation rows 64c..64c+63
    // and weight rows 8*NI*c..8*NI*c+8*NI-1, 8 rows of 128 bytes per
    // instruction; sources are uniform bases plus 32-bit lane offsets (the
    // host keeps every offset below 2^32)
    const bool copier = wave < 4;
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(p.x + g * p.gx);
    const uint8_t* wb = reinterpret_cast<const uint8_t*>(p.w + g * p.gw);
    uint32_t aoff[8], woff[NI];
    if (copier) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 64 * wave + 8 * j + (lane >> 3);
            int64_t m = m0 + row;
            m = m < p.M ? m : p.M - 1;  // rows past M are computed but never stored
            aoff[j] = (uint32_t)(m * xrow + ((lane & 7) ^ swz(row)) * 16);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int row = 8 * (NI * wave + j) + (lane >> 3);
            int64_t n = n0 + row;
            n = n < p.N ? n : p.N - 1;
            woff[j] = (uint32_t)(n * kbytes + ((lane & 7) ^ swz(row)) * 16);
        }
    }
    const uint32_t ring0 = lds_offset(&ring[0][0]);
    const uint32_t adst = ring0 + SA + 64 * (wave & 3) * 128, bdst = ring0 + SB + 8 * NI * (wave & 3) * 128;
    auto issue = [&](int64_t ks, int slot) __attribute__((always_inline)) {
        ks = ks < nstage ? ks : nstage - 1;  // past the end: re-copy the last step into a dead slot
        const uint32_t so = (uint32_t)(slot * STAGE);
#pragma unroll
        for (int j = 0; j < 8; ++j) dma16s(xb + ks * 128, aoff[j], adst + so + j * 1024);
#pragma unroll
        for (int j = 0; j < NI; ++j) dma16s(wb + ks * 128, woff[j], bdst + so + j * 1024);
    };
    if (copier) issue(0, 0);

    v4f acc[4][NI];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

    // fragment addressing: rows 16k + frow share the swizzle of frow
    const int frow = lane & 15;
    const int p0 = 2 * (lane >> 4);
    const int lo_off = frow * 128 + 16 * (p0 ^ swz(frow));
    const int hi_off = frow * 128 + 16 * ((p0 + 1) ^ swz(frow));
    auto ld = [&](const uint8_t* base, int o) __attribute__((always_inline)) {
        return *reinterpret_cast<const v8bf*>(base + o);
    };

    // The K loop, instantiated per wave role so that no branch sits among the
    // MFMAs: waves 0-1 copy their half of a step right after the barrier,
    // waves 2-3 before subtile kMid's MFMAs, waves 4-7 only compute (two
    // half-size bursts on the DMA path instead of one, as in the FP8 tile
    // kernel; kMid measured best of 1, 2, 3).
    constexpr int kCopyTop = 0, kCopyMid = 1, kComputeOnly = 2, kMid = 2;
    auto kloop = [&](auto role) __attribute__((always_inline)) {
        constexpr int ROLE = decltype(role)::value;
        for (int64_t ks = 0; ks < nstage; ++ks) {
            if (ROLE != kComputeOnly) wait_vmcnt<0>();  // this wave's copies of step ks have landed
            __builtin_amdgcn_s_barrier();  // ... and every other wave's; step ks-1 is free
            if (ROLE == kCopyTop) issue(ks + 1, (int)((ks + 1) & 1));
            const uint8_t* st = ring[ks & 1];
            const uint8_t* sta = st + SA + 64 * wm * 128;
            const uint8_t* stb = st + SB + 16 * NI * wn * 128;
            v8bf blo[NI], bhi[NI];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                blo[ni] = ld(stb + ni * 2048, lo_off);
                bhi[ni] = ld(stb + ni * 2048, hi_off);
            }
            // activation fragments of subtile mi+1 are read while subtile mi runs
            v8bf alo = ld(sta, lo_off), ahi = ld(sta, hi_off);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                if (ROLE == kCopyMid && mi == kMid) issue(ks + 1, (int)((ks + 1) & 1));
                const v8bf a0 = alo, a1 = ahi;
                if (mi < 3) {
                    alo = ld(sta + (mi + 1) * 2048, lo_off);
                    ahi = ld(sta + (mi + 1) * 2048, hi_off);
                }
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, blo[ni], acc[mi][ni], 0, 0, 0);
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bhi[ni], acc[mi][ni], 0, 0, 0);
            }
        }
    };
    if (wave < 2) kloop(std::integral_constant<int, kCopyTop>{});
    else if (copier) kloop(std::integral_constant<int, kCopyMid>{});
    else kloop(std::integral_constant<int, kComputeOnly>{});
    wait_vmcnt<0>();  // no copy may still be writing LDS when the workgroup exits

    // epilogue: bf16 (nearest even) through LDS, so that y is written as whole
    // tile rows with 16-byte stores; as many 64-row bands per pass as the ring
    // holds (rows padded by 16 bytes against bank conflicts)
    constexpr int EROW = BN + 8;                                   // bf16 per LDS row
    constexpr int BANDS = (2 * STAGE) / (64 * EROW * 2) >= 4 ? 4 : 2;  // 64-row bands per pass
    constexpr int CPR = BN / 8;                                    // 16-byte chunks per row
    static_assert(64 * BANDS * EROW * 2 <= 2 * STAGE, "a pass of the epilogue fits in the ring");
    uint16_t* stile = reinterpret_cast<uint16_t*>(&ring[0][0]);
    __builtin_amdgcn_s_barrier();  // every wave is done with the ring
#pragma unroll
    for (int pass = 0; pass < 4 / BANDS; ++pass) {
        if (wm / BANDS == pass) {
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 64 * (wm % BANDS) + 16 * mi + 4 * (lane >> 4) + i;
                        const int c = 16 * NI * wn + 16 * ni + frow;
                        stile[r * EROW + c] = (uint16_t)f32_to_bf16_bits(acc[mi][ni][i]);
                    }
        }
        __syncthreads();
        for (int idx = tid; idx < 64 * BANDS * CPR; idx += NW * 64) {
            const int r = idx / CPR, ch = idx % CPR;
            const int64_t row = m0 + 64 * BANDS * pass + r, col = n0 + 8 * ch;
            const uint4 v = *reinterpret_cast<const uint4*>(stile + r * EROW + 8 * ch);
            if (row < p.M && col < p.N) *reinterpret_cast<uint4*>(p.y + g * p.gy + row * p.sy + col) = v;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Few-token kernel (M <= 128): the weight stream is the cost, so the tile is
// 64 rows x 64 columns (no rows computed for nothing) and, as in the FP8
// decode kernel, the waves form K-groups of four that each walk their share
// of K through their own ring of XNS steps (XNS-1 in flight), one 64-element
// step (128 bytes of every row) per s_waitcnt + barrier.  Four K-groups with
// two-slot rings measured faster than two with four slots: more positions
// along K in flight at once.  In a K-group waves 0-1 copy (weights with the
// non-temporal hint: read once) and all four compute, wave w owning columns
// 16w..16w+15.  The K-groups' fp32 partial tiles are summed through LDS and
// stored as whole rows.
#ifndef OPROJ_XNS
#define OPROJ_XNS 2
#endif
#ifndef OPROJ_XKS
#define OPROJ_XKS 4
#endif
constexpr int XBM = 64, XBN = 64, XNS = OPROJ_XNS, XKS = OPROJ_XKS;
constexpr int XSTAGE = 64 * 128 * 2;  // activation slab + weight slab
constexpr int XVM = 8;                // copy instructions per copying wave per step
constexpr int XPROW = XBN + 4;        // fp32 per row of an epilogue partial tile
static_assert(XKS * XBM * XPROW * 4 <= XKS * XNS * XSTAGE, "the epilogue fits in the ring");

__global__ __launch_bounds__(XKS * 256) void gemm_bf16_decode_kernel(DParams p) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[XKS][XNS][XSTAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int kq = __builtin_amdgcn_readfirstlane(tid >> 8);           // K-group
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // row group of the tile
    const bool copier = wave < 2;
    const GroupTile gt = group_tile(p);
    const int64_t g = gt.g;
    const uint32_t mt = gt.id / (uint32_t)p.ntiles, nt = gt.id - mt * (uint32_t)p.ntiles;
    const int64_t m0 = (int64_t)mt * XBM, n0 = (int64_t)nt * XBN;
    const int64_t kbytes = p.K * 2, xrow = p.sx * 2;
    const int64_t nstep = kbytes / 128;
    const int64_t s0 = nstep * kq / XKS, ns = nstep * (kq + 1) / XKS - s0;

    // copy plan: copying wave c moves rows 32c..32c+31 of both slabs, 8 rows
    // of 128 bytes per instruction
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(p.x + g * p.gx);
    const uint8_t* wb = reinterpret_cast<const uint8_t*>(p.w + g * p.gw);
    uint32_t aoff[4], woff[4];
    if (copier) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 32 * wave + 8 * j + (lane >> 3);
            const int piece = (lane & 7) ^ swz(row);
            int64_t m = m0 + row;
            m = m < p.M ? m : p.M - 1;  // rows past M are computed but never stored
            aoff[j] = (uint32_t)(m * xrow + piece * 16);
            int64_t n = n0 + row;
            n = n < p.N ? n : p.N - 1;
            woff[j] = (uint32_t)(n * kbytes + piece * 16);
        }
    }
    const uint32_t ring0 = lds_offset(&ring[kq][0][0]);
    auto issue = [&](int64_t i, int slot) __attribute__((always_inline)) {
        const int64_t ks = s0 + i;
        const uint32_t st = ring0 + (uint32_t)(slot * XSTAGE);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16s(xb + ks * 128, aoff[j], st + (32 * wave + 8 * j) * 128);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16s_nt(wb + ks * 128, woff[j], st + 8192 + (32 * wave + 8 * j) * 128);
    };
    if (copier) {
#pragma unroll
        for (int s = 0; s < XNS - 1; ++s)
            if (s < ns) issue(s, s);
    }

    v4f acc[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) acc[mi] = v4f{0.f, 0.f, 0.f, 0.f};
    const int frow = lane & 15;
    const int p0 = 2 * (lane >> 4);
    const int64_t nst = (nstep + XKS - 1) / XKS;  // the largest share: same barrier count in both groups
    for (int64_t i = 0; i < nst; ++i) {
        if (copier) wait_ahead<XNS - 2, XVM>(ns - 1 - i);
        __builtin_amdgcn_s_barrier();
        if (copier && i + XNS - 1 < ns) issue(i + XNS - 1, (int)((i + XNS - 1) % XNS));
        if (i >= ns) continue;  // uniform per K-group
        const uint8_t* st = ring[kq][i % XNS];
        // wave w: token rows 16w..16w+15 against all 64 columns
        const int ra = 16 * wave + frow;
        const v8bf alo = *reinterpret_cast<const v8bf*>(st + ra * 128 + 16 * (p0 ^ swz(ra)));
        const v8bf ahi = *reinterpret_cast<const v8bf*>(st + ra * 128 + 16 * ((p0 + 1) ^ swz(ra)));
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int r = 16 * ni + frow;
            const v8bf blo = *reinterpret_cast<const v8bf*>(st + 8192 + r * 128 + 16 * (p0 ^ swz(r)));
            const v8bf bhi = *reinterpret_cast<const v8bf*>(st + 8192 + r * 128 + 16 * ((p0 + 1) ^ swz(r)));
            acc[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, blo, acc[ni], 0, 0, 0);
            acc[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bhi, acc[ni], 0, 0, 0);
        }
    }
    wait_vmcnt<0>();  // (already true: the last step was waited for in full)
    __syncthreads();

    float* part = reinterpret_cast<float*>(&ring[0][0][0]);  // [XKS][64][XPROW]
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            part[(kq * XBM + 16 * wave + 4 * (lane >> 4) + i) * XPROW + 16 * ni + frow] = acc[ni][i];
    __syncthreads();
    for (int idx = tid; idx < XBM * (XBN / 8); idx += XKS * 256) {
        const int r = idx / (XBN / 8), ch = idx % (XBN / 8);
        float4 s0v = *reinterpret_cast<const float4*>(part + r * XPROW + 8 * ch);
        float4 s1v = *reinterpret_cast<const float4*>(part + r * XPROW + 8 * ch + 4);
#pragma unroll
        for (int q = 1; q < XKS; ++q) {
            const float4 u0 = *reinterpret_cast<const float4*>(part + (q * XBM + r) * XPROW + 8 * ch);
            const float4 u1 = *reinterpret_cast<const float4*>(part + (q * XBM + r) * XPROW + 8 * ch + 4);
            s0v.x += u0.x; s0v.y += u0.y; s0v.z += u0.z; s0v.w += u0.w;
            s1v.x += u1.x; s1v.y += u1.y; s1v.z += u1.z; s1v.w += u1.w;
        }
        const uint4 v = {f32_to_bf16_bits(s0v.x) | (f32_to_bf16_bits(s0v.y) << 16),
                         f32_to_bf16_bits(s0v.z) | (f32_to_bf16_bits(s0v.w) << 16),
                         f32_to_bf16_bits(s1v.x) | (f32_to_bf16_bits(s1v.y) << 16),
                         f32_to_bf16_bits(s1v.z) | (f32_to_bf16_bits(s1v.w) << 16)};
        const int64_t row = m0 + r, col = n0 + 8 * ch;
        if (row < p.M && col < p.N) *reinterpret_cast<uint4*>(p.y + g * p.gy + row * p.sy + col) = v;
    }
}

// Fills p's tile map for a grid of G x mtiles x ntiles workgroups of `threads`
// work-items on a device of nx XCDs; false when the grid is beyond one launch
// (more than 2^32 - 1 work-items in all).
bool set_tile_map(DParams& p, int threads, int nx) {
    const int64_t nblocks = p.G * p.mtiles * p.ntiles;
    if (nblocks < 1 || nblocks > (int64_t)UINT32_MAX / threads) return false;
    p.tpg = (uint32_t)(p.mtiles * p.ntiles);
    p.xcd_per = 0;
    p.xcd_shift = 0;
    if (nx > 1 && (nx & (nx - 1)) == 0 && nblocks % nx == 0) {
        p.xcd_shift = __builtin_ctz((unsigned)nx);
        p.xcd_per = (uint32_t)(nblocks / nx);
    }
    return true;
}

}  // namespace

hipError_t launch_bf16_gemm(const Bf16GemmArgs& a, hipStream_t stream) {
    DParams p;
    p.x = a.x;
    p.w = a.w;
    p.y = a.y;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.sx = a.sx;
    p.sy = a.sy;
    p.gx = a.gx;
    p.gw = a.gw;
    p.gy = a.gy;
    p.G = a.G;
    const DeviceInfo dev = current_device_info();
    if (a.M <= 128) {  // few tokens: 64x64 tiles, K split over two wave groups
        p.mtiles = (a.M + XBM - 1) / XBM;
        p.ntiles = (a.N + XBN - 1) / XBN;
        if (!set_tile_map(p, XKS * 256, dev.xcds)) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(gemm_bf16_decode_kernel, dim3(p.tpg * (uint32_t)p.G), dim3(XKS * 256), 0,
                           stream, p);
        return hipGetLastError();
    }
    p.mtiles = (a.M + BM - 1) / BM;
    // 64-column tiles when 256-column tiles leave most of the chip idle;
    // otherwise 224-column tiles when they fill the last round of workgroups
    // (one per compute unit) better than 256-column tiles
    const int64_t t256 = a.G * p.mtiles * ((a.N + 255) / 256), t224 = a.G * p.mtiles * ((a.N + 223) / 224);
    const int64_t cus = dev.cus;
    auto fill = [cus](int64_t tiles) { return (double)tiles / (double)(((tiles + cus - 1) / cus) * cus); };
    int ni = 8;
    if (t256 < cus / 2)
        ni = 2;
    else if (fill(t224) > fill(t256) + 0.02)
        ni = 7;
    p.ntiles = (a.N + 32 * ni - 1) / (32 * ni);
    if (!set_tile_map(p, NW * 64, dev.xcds)) return hipErrorInvalidConfiguration;
    const dim3 grid(p.tpg * (uint32_t)p.G), block(NW * 64);
    if (ni == 2)
        hipLaunchKernelGGL(gemm_bf16_kernel<2>, grid, block, 0, stream, p);
    else if (ni == 7)
        hipLaunchKernelGGL(gemm_bf16_kernel<7>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(gemm_bf16_kernel<8>, grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_dense_bf16_gemm(const DenseGemmArgs& a, hipStream_t stream) {
    Bf16GemmArgs b;
    b.G = 1;
    b.M = a.M;
    b.N = a.N;
    b.K = a.K;
    b.x = a.x;
    b.w = a.w;
    b.y = a.y;
    b.sx = a.K;
    b.sy = a.N;
    b.gx = b.gw = b.gy = 0;
    return launch_bf16_gemm(b, stream);
}

}  // namespace oproj
