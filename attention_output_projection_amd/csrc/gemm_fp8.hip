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
//    into the accumulator as acc = fma(P, sa[token]*sw[row], acc).  In the
//    128x128 weight recipe sw is one value per 128 weight rows, and the tile
//    kernel makes the weights the MFMA's row operand: a lane's four partials
//    then belong to one token, and one product sa*sw serves all of them
//    (four fma and a quarter multiply per MFMA, which the SIMD overlaps with
//    the matrix core; five per MFMA measured 2-3% slower);
//  * pow2 recipe (both scale sets are powers of two): the block-scaled MFMA
//    v_mfma_scale_f32_16x16x128_f8f6f4 applies the E8M0 exponents of sa and
//    sw in the matrix core and accumulates directly; no VALU work per block.
//
// The kernels share this machinery, all fed by direct global->LDS copies
// (global_load_lds) into rings of 128-byte rows whose 16-byte pieces are
// XOR-swizzled so fragment reads hit distinct banks:
//  * tile kernel (large T): 256x256 output tiles, 512-thread workgroups of
//    eight waves of 128x64, one K-block per stage, double-buffered; one
//    workgroup per CU walks its tiles, the next tile's first stage copied
//    during the last K-block;
//  * decode kernel (small T): 64x64 output tile per workgroup, two K-groups
//    of four waves (16 columns each) with a four-stage ring each, the two
//    partial tiles summed through LDS at the end.  The weight stream is the
//    cost at small T; the deep ring keeps enough of it in flight.
// All of them take the tiles of one group on one XCD (a group's activations
// and weights then stay in that XCD's L2).  A further kernel runs the decode
// kernel's grid with the quantisation (steps a1 + a2) in front: each
// workgroup quantises its share of its group into a workspace, the group's
// workgroups meet at a barrier of their own, then each runs its tile.
#include <cstdlib>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_dma.hpp"
#include "rq_item.hpp"

#ifndef OPROJ_DEC_W_NT
#define OPROJ_DEC_W_NT 1
#endif

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
    int64_t kbw;  // weight scale words per scale row (KB, or KB/4 for packed UE8M0)
    int wkshift;  // weight scale words hold 1 << wkshift K-blocks (0: fp32, 2: packed UE8M0)
    int we8;      // weight scales are packed UE8M0 words (block scaled MFMA only)
    int kshift;   // activation scale words hold 1 << kshift K-blocks (0: fp32, 2: packed UE8M0)
    int e8;       // activation scales are packed UE8M0 words (block scaled MFMA only)
    int spin = 0;  // one-launch path: polls of a group barrier before the fallback
    uint64_t* sync = nullptr;  // one-launch path: the groups' barrier words (caller's workspace)
    uint32_t tpg = 1;      // tiles per group (mtiles * ntiles)
    uint32_t nt32 = 1;     // ntiles
    uint32_t xcd_per = 0;  // tiles per XCD when the XCD remap applies, else 0
    int xcd_shift = 0;     // log2 of the XCD count (a power of two) when it applies
    int pfd = 0;   // tile kernels: L2 prefetch distance in K-blocks (0: none)
    uint32_t ntot = 0;  // persistent tile kernel: tiles in all
    int xnext = 0;      // persistent tile kernel: every N-tile is whole (R a multiple of 256)
};

// Exponent byte (E8M0) of activation scale word `raw` for K-block kb: the
// exponent field of a power-of-two fp32 scale, or byte kb % 4 of a packed
// UE8M0 word.
__device__ __forceinline__ int act_e8m0(const GParams& p, uint32_t raw, int64_t kb) {
    const int sh = p.e8 ? 8 * (int)(kb & 3) : 23;
    return (int)((raw >> sh) & 0xFFu);
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_fp8_mx(const v8i& a, const v8i& b, const v4f& c, int ea,
                                           int eb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// Workgroup ids are dealt to the XCDs round-robin: remap them so that each XCD
// runs one contiguous range of tiles (the same group), then split the tile
// number into (group, M-tile, N-tile).  The host prepares the shift and the
// counts (set_tile_map), so this is a handful of 32-bit scalar operations.
struct TileCoord {
    int64_t g, mt, nt;
};
__device__ __forceinline__ TileCoord tile_coord(const GParams& p) {
    const uint32_t b = blockIdx.x;
    const uint32_t t =
        p.xcd_per ? (b & ((1u << p.xcd_shift) - 1u)) * p.xcd_per + (b >> p.xcd_shift) : b;
    const uint32_t g = t / p.tpg, r = t - g * p.tpg;
    const uint32_t mt = r / p.nt32;
    return {(int64_t)g, (int64_t)mt, (int64_t)(r - mt * p.nt32)};
}

__device__ __forceinline__ int64_t wscale_index(const GParams& p, int64_t wrow, int64_t kb) {
    return (wrow >> p.w_shift) * p.kbw + (kb >> p.wkshift);
}

// Exponent byte (E8M0) of weight scale word `raw` for K-block kb (as act_e8m0).
__device__ __forceinline__ int w_e8m0(const GParams& p, uint32_t raw, int64_t kb) {
    const int sh = p.we8 ? 8 * (int)(kb & 3) : 23;
    return (int)((raw >> sh) & 0xFFu);
}

// ---------------------------------------------------------------------------
// Tile kernel (large T): 256x256 output tiles, one 512-thread workgroup per
// CU walking a sequence of tiles (below), eight waves as 2 (M) x 4 (N) of
// 128x64 (32 MFMAs per K-block per wave, 128 fp32 accumulators in VGPRs),
// two waves per SIMD.  (Batches whose 256-row tiles would leave half the CUs
// idle take 128x256 tiles instead: waves of 64x64, the same pipeline.)  The tile and wave shapes keep
// LDS reads per MFMA low: per K-block the workgroup reads 192 KiB of
// fragments and copies 64 KiB for 2048 MFMA cycles per SIMD.  Each K-block is
// one pipeline stage (256x128-byte activation slab, 256x128-byte weight slab,
// the block's scales), DMA-copied into a double-buffered LDS ring with
// XOR-swizzled 128-byte rows; one s_waitcnt + bare barrier per K-block.
//
// Waves 0-3 issue all copies of a stage (18 each), one per SIMD; waves 4-7
// only compute.  A copy waits at issue until the CU's DMA path (about 64
// bytes per clock) accepts it, so a copying wave is held while the path
// drains the copies ahead of its own, and starts its MFMAs late; its SIMD
// partner (a wave that never copies) keeps the matrix core busy meanwhile.
// The copies go in two bursts of half the stage: waves 0-1 right after the
// barrier, waves 2-3 in the middle of the K-block, which still leaves their
// copies half a K-block to land.  Each burst holds its waves about half as
// long as one burst of all four.  Copies spread thinner (four bursts, or a
// few copies after every subtile, or by all eight waves) delay more MFMAs
// than they free, or land too late.
//
// The CU's memory pipeline holds a fixed number of outstanding lines, so the
// copy rate is set by their latency: lines that miss in L2 cost several times
// a hit.  The tiles that run together on one XCD share slabs (the 4 N-tiles of
// an M-tile its activation rows, 8 M-tiles a weight slab), so each tile also
// touches its share of the shared slabs a few K-blocks ahead (one 4-byte load
// per 128-byte line): one CU takes each miss, early, and the copies of every
// CU then hit in L2.
//
// fp32 recipe: a subtile's fresh partials are folded into the accumulators
// one subtile later (the last subtile of a K-block after the next barrier),
// so the matrix core runs the next MFMAs while the promotion waits for them.
constexpr int TBM = 256, TBN = 256, TNS = 2, TNW = 8;
// Stage layout for tiles of bm rows (256, or 128 when 256-row tiles would
// leave CUs idle): activation slab, weight slab, 256 activation scale slots
// (64 per copying wave), 256 weight scales.
constexpr int tsb(int bm) { return bm * 128; }
constexpr int tss(int bm) { return tsb(bm) + TBN * 128; }
constexpr int tsw(int bm) { return tss(bm) + 1024; }
constexpr int tstage(int bm) { return tsw(bm) + 1024; }  // 67584 bytes at 256 rows
constexpr int kTilePrefetch = 2;    // L2 prefetch distance in K-blocks (measured best of 2, 3, 4, 6)
constexpr int kCopyTop = 0, kCopyMid = 1, kComputeOnly = 2;  // wave roles in the K loop
constexpr int kMidSubtile = 4;  // waves 2-3 copy before this subtile's MFMAs (2, 3, 4 measured alike; 6 slower)

// Persistent grid: one workgroup per CU (the same number on every XCD) walks
// a sequence of tiles.  The tiles of an XCD are taken in order of tile id
// (at any time an XCD's workgroups run consecutive tile ids: the N-tiles of
// 8 M-tiles of one group), and:
//  * the last K-block of a tile copies the next tile's first stage into the
//    free ring slot (in place of a re-copy of the last block), so that stage
//    lands while the tile's results are written;
//  * each wave writes its own 128x64 results, one 16-row subtile at a time,
//    through a private 16-row LDS buffer as whole 128-byte z row segments:
//    no workgroup barrier between the K loop and the stores, and the ring
//    stays free for the next tile's copies.
// The copy offsets are lane constants plus per-tile scalar bases; a tile cut
// short by T or R clamps its rows, so its first stage is copied by itself
// (after the previous tile's re-copy has landed).
constexpr int PEROW = 64 + 8;  // bf16 per row of a wave's epilogue subtile (16-byte pad)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> two bf16 (round to nearest even) in one word, low half first.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Tiles of this workgroup: base + first + i * step while first + i * step < limit.
struct TileSeq {
    uint32_t base, first, step, limit;
};
__device__ __forceinline__ TileSeq tile_seq(const GParams& p) {
    const uint32_t b = blockIdx.x, n = gridDim.x;
    if (p.xcd_per) {
        const uint32_t x = b & ((1u << p.xcd_shift) - 1u);
        return {x * p.xcd_per, b >> p.xcd_shift, n >> p.xcd_shift, p.xcd_per};
    }
    return {0u, b, n, p.ntot};
}

// Scalar description of one tile: operand bases at K-block 0 and the last
// valid tile-local row (mlim) and weight row (nlim).
struct TilePlan {
    const uint8_t* ab;   // activation row m0 of group g
    const uint8_t* wb;   // weight row g*R + n0
    const uint8_t* sab;  // activation scale word of row m0
    const uint8_t* swb;  // weight scale word of the block holding row g*R + n0
    int32_t mlim, nlim;
    int32_t wphase;      // (g*R + n0) mod the weight scale block height
    int32_t mt, nt;
    int64_t g, m0, n0;
    bool full;
};
template <int BM, typename PP>
__device__ __forceinline__ TilePlan tile_plan(const PP& p, uint32_t t) {
    const uint32_t g = t / p.tpg, r = t - g * p.tpg, mt = r / p.nt32, nt = r - mt * p.nt32;
    TilePlan q;
    q.g = g;
    q.mt = (int32_t)mt;
    q.nt = (int32_t)nt;
    q.m0 = (int64_t)mt * BM;
    q.n0 = (int64_t)nt * TBN;
    const int64_t ml = p.T - 1 - q.m0, nl = p.R - 1 - q.n0;
    q.mlim = (int32_t)(ml < BM ? ml : BM);
    q.nlim = (int32_t)(nl < TBN ? nl : TBN);
    const int64_t wrow = (int64_t)g * p.R + q.n0;
    q.wphase = (int32_t)(wrow & ((1 << p.w_shift) - 1));
    q.ab = p.a + (int64_t)g * p.sg + q.m0 * p.st;
    q.wb = p.w + wrow * p.D;
    q.sab = reinterpret_cast<const uint8_t*>(p.sa + (int64_t)g * p.ssg + q.m0 * p.sst);
    q.swb = reinterpret_cast<const uint8_t*>(p.sw + (wrow >> p.w_shift) * p.kbw);
    q.full = q.mlim >= BM - 1 && q.nlim >= TBN - 1;
    return q;
}

// The kernel's parameters re-read from the kernel-argument segment through a
// pointer the compiler cannot see through: values a tile transition needs are
// then loaded again at each transition instead of being held in scalar
// registers across the K loop (which has none to spare).  GParams is the
// kernel's only argument, at offset 0 of the segment.
typedef __attribute__((address_space(4))) const GParams KGParams;
__device__ __forceinline__ KGParams& params_reloaded() {
    uint64_t v = reinterpret_cast<uint64_t>(__builtin_amdgcn_kernarg_segment_ptr());
    asm volatile("" : "+s"(v));
    return *reinterpret_cast<KGParams*>(v);
}

// MS: 16-row M-subtiles per wave; the tile has 32 * MS rows (8: 256 rows, 4:
// 128 rows, for batches whose 256-row tiles would not fill the CUs).
template <bool MX, bool W1, int MS>
__global__ __launch_bounds__(TNW * 64) void gemm_fp8_ptile_kernel(GParams p) {
    constexpr bool kTight = W1 && !MX && MS == 8;  // the instantiation with the most live registers
    constexpr int BM = 32 * MS;                     // tile rows
    constexpr int CRA = BM / 4;                     // activation rows per copying wave
    constexpr int TSB = tsb(BM), TSS = tss(BM), TSW = tsw(BM), TSTAGE = tstage(BM);
    constexpr int MID = MS == 8 ? kMidSubtile : MS / 2;  // the mid copiers' subtile
    // activation scale slot of tile row r: 64 slots per copying wave, CRA used
    auto asl = [](int r) __attribute__((always_inline)) { return MS == 8 ? r : 64 * (r / CRA) + r % CRA; };
    __shared__ __attribute__((aligned(1024))) uint8_t ring[TNS][TSTAGE];
    __shared__ __attribute__((aligned(16))) uint16_t epi[TNW][16 * PEROW];
    __shared__ __attribute__((aligned(256))) uint8_t pf_sink[256];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
    const int wm = wave & 1, wn = wave >> 1;
    const bool copier = wave < 4;  // wave-uniform
    const TileSeq seq = tile_seq(p);

    // ---- copy plan of copying wave c (0-3): activation rows 64c..64c+63 and
    // weight rows 64c..64c+63 of the tile (8 rows of 128 bytes per
    // instruction) and the scales of those rows; lane offsets relative to the
    // tile's scalar bases, rows clamped to the tile's last valid row.
    uint32_t off[MS + 8], soffa = 0, soffw = 0;
    auto plan_lanes = [&](KGParams& pr, const TilePlan& q) __attribute__((always_inline)) {
        if (copier) {
            // fp32 with per-row weight scales (the instantiation with the most
            // live registers): lane-derived values formed here, not held
            // across the tile loop
            int el = lane;
            if constexpr (kTight) asm volatile("" : "+v"(el));
#pragma unroll
            for (int j = 0; j < MS; ++j) {
                const int row = CRA * wave + 8 * j + (el >> 3);
                const uint32_t piece = (uint32_t)(((el & 7) ^ swz(row)) * 16);
                off[j] = (uint32_t)(row < q.mlim ? row : q.mlim) * (uint32_t)pr.st + piece;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = 64 * wave + 8 * j + (el >> 3);
                const uint32_t piece = (uint32_t)(((el & 7) ^ swz(row)) * 16);
                off[MS + j] = (uint32_t)(row < q.nlim ? row : q.nlim) * (uint32_t)pr.D + piece;
            }
            // (128-row tiles: lanes 32-63 repeat lanes 0-31 into unused slots)
            const int arow = CRA * wave + (MS == 8 ? el : (el & 31));
            soffa = (uint32_t)(arow < q.mlim ? arow : q.mlim) * (uint32_t)pr.sst * 4u;
            const int row = 64 * wave + el;
            soffw = (uint32_t)(((q.wphase + (row < q.nlim ? row : q.nlim)) >> pr.w_shift) * pr.kbw) * 4u;
        }
    };
    const uint32_t ring0 = lds_offset(&ring[0][0]);
    const uint32_t adst = ring0 + CRA * (wave & 3) * 128, wdst = ring0 + TSB + 64 * (wave & 3) * 128;
    auto issue = [&](const uint8_t* ab, const uint8_t* wb, const uint8_t* sab, const uint8_t* swb, int64_t kb,
                     int slot) __attribute__((always_inline)) {
        const uint32_t so = (uint32_t)(slot * TSTAGE);
        ab += kb * 128;
        wb += kb * 128;
#pragma unroll
        for (int j = 0; j < MS; ++j) dma16s(ab, off[j], adst + so + j * 1024);
#pragma unroll
        for (int j = 0; j < 8; ++j) dma16s(wb, off[MS + j], wdst + so + j * 1024);
        dma4s(sab + (kb >> p.kshift) * p.sskb * 4, soffa, ring0 + so + TSS + 256 * (wave & 3));
        dma4s(swb + (kb >> p.wkshift) * 4, soffw, ring0 + so + TSW + 256 * (wave & 3));
    };

    // L2 prefetch shared out among an XCD's co-running tiles, as in the tile
    // kernel: N-tile nt < 4 touches activation rows 64*nt..64*nt+63 of its
    // M-tile's slab (wave 0), M-tile mt touches weight rows 32*(mt%8)..+31 of
    // its N-tile's slab (wave 1), pfd K-blocks ahead of the copies.  (The
    // lane offset is formed at each touch from scalars: no register held
    // across the K loop.)
    const uint32_t sink = lds_offset(pf_sink);
    int32_t pf_row0 = 0, pf_lim = 0;
    uint32_t pf_stride = 0, pfoff = 0;
    auto pf_lane = [&](int el) __attribute__((always_inline)) {
        const int row = pf_row0 + (wave == 0 && MS == 8 ? el : (el & 31));
        return (uint32_t)(row < pf_lim ? row : pf_lim) * pf_stride;
    };
    auto plan_pf = [&](KGParams& pr, const TilePlan& q) __attribute__((always_inline)) {
        if (wave == 0) {
            pf_row0 = (BM / 4) * q.nt;
            pf_lim = q.mlim;
            pf_stride = (uint32_t)pr.st;
        } else if (wave == 1) {
            pf_row0 = 32 * (q.mt & 7);
            pf_lim = q.nlim;
            pf_stride = (uint32_t)pr.D;
        }
        if constexpr (!kTight) pfoff = pf_lane(lane);
    };
    auto pf_off = [&]() __attribute__((always_inline)) {
        if constexpr (kTight) {  // formed at each touch: no register held across the K loop
            int el = lane;
            asm volatile("" : "+v"(el));
            return pf_lane(el);
        } else {
            return pfoff;
        }
    };

    v4f acc[MS][4];
    // fragment addressing: rows 16k + frow share the swizzle of frow, so a
    // lane's two piece offsets are fixed and subtiles step by 2 KiB
    const int frow = lane & 15;
    const int p0 = 2 * (lane >> 4);
    const int lo_off = frow * 128 + 16 * (p0 ^ swz(frow));
    const int hi_off = frow * 128 + 16 * ((p0 + 1) ^ swz(frow));
    auto frag = [&](const uint8_t* base) __attribute__((always_inline)) {
        const uint4 lo = *reinterpret_cast<const uint4*>(base + lo_off);
        const uint4 hi = *reinterpret_cast<const uint4*>(base + hi_off);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    // fp32 recipe: the partials of the subtile issued last and their scale
    // factors, folded into the accumulators one subtile later (the last
    // subtile of a K-block across the barrier into the next K-block), so that
    // the matrix core has the next subtile's MFMAs to run while they wait.
    // With 128x128 weight blocks the weights are the MFMA's 16-row operand
    // and the tokens its 16 columns: a lane's four partials are then four
    // weight rows of one token and share one factor sa[token] * sw[block],
    // one multiply per subtile instead of one per row.  With per-row weight
    // scales the tokens stay the row operand (each partial has its own
    // factor either way, and this form holds fewer of them).
    v4f pend[4];
    float ps = 0.f;
    float psa[4] = {0.f, 0.f, 0.f, 0.f}, psw[4] = {0.f, 0.f, 0.f, 0.f};
    auto fold = [&](int mi, int ni) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc[mi][ni][i] = __builtin_fmaf(pend[ni][i], W1 ? psa[i] * psw[ni] : ps, acc[mi][ni][i]);
    };

    // Subtile mi (16 token rows x 64 columns) of this wave's results to z:
    // bf16 (nearest even) into the wave's buffer, then 8 rows of 128 bytes per
    // store.  zb points at z[m0 + 128*wm][g][n0 + 64*wn]; rows_left and
    // cols_left bound the tile by T and R.
    auto store_sub = [&](int mi, uint16_t* zb, int64_t zrs, int64_t rows_left, int64_t cols_left)
                         __attribute__((always_inline)) {
        int el = lane;  // lane-derived addresses computed here, not held across the K loop
        asm volatile("" : "+v"(el));
        const int efrow = el & 15;
        uint16_t* my = &epi[wave][0];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const uint32_t v01 = pk_bf16(acc[mi][ni][0], acc[mi][ni][1]);
            const uint32_t v23 = pk_bf16(acc[mi][ni][2], acc[mi][ni][3]);
            if constexpr (MX || W1) {  // a lane holds one column of four rows
                uint16_t* col = my + 4 * (el >> 4) * PEROW + 16 * ni + efrow;
                col[0] = (uint16_t)v01;
                col[PEROW] = (uint16_t)(v01 >> 16);
                col[2 * PEROW] = (uint16_t)v23;
                col[3 * PEROW] = (uint16_t)(v23 >> 16);
            } else {  // a lane holds four adjacent columns of one row
                *reinterpret_cast<uint2*>(my + efrow * PEROW + 16 * ni + 4 * (el >> 4)) = uint2{v01, v23};
            }
        }
        const int c8 = 8 * (el & 7);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 8 * h + (el >> 3);
            const uint4 v = *reinterpret_cast<const uint4*>(my + r * PEROW + c8);
            const int row = 16 * mi + r;
            if (row < rows_left && c8 < cols_left) *reinterpret_cast<uint4*>(zb + row * zrs + c8) = v;
        }
    };

    // The tile loop and its K loop, instantiated per wave role so that no branch sits among the
    // MFMAs: waves 0-1 copy their half of a stage right after the barrier
    // (and issue the L2 prefetch), waves 2-3 after subtile kMidSubtile-1's
    // MFMAs, waves 4-7 only compute.  Two half-size bursts on the DMA path
    // hold each copying wave about half as long as one burst of all four.
    // Not unrolled or peeled: a peeled first K-block is a second copy of the
    // loop body, and that copy spills.
    auto run = [&](auto role) __attribute__((always_inline)) {
        constexpr int ROLE = decltype(role)::value;
        constexpr bool COPY = ROLE != kComputeOnly;
        bool first = true, chained = false;
        for (uint32_t i = seq.first; i < seq.limit; i += seq.step) {
            const TilePlan q = tile_plan<BM>(params_reloaded(), seq.base + i);
            if constexpr (COPY) {
                plan_lanes(params_reloaded(), q);
                if (!chained) {
                    if (!first) wait_vmcnt<0>();  // the re-copy into slot 0 has landed
                    issue(q.ab, q.wb, q.sab, q.swb, 0, 0);
                }
            }
            if constexpr (ROLE == kCopyTop) plan_pf(params_reloaded(), q);
            first = false;
            const uint32_t inext = i + seq.step;
            const bool has_next = inext < seq.limit;
            // the next tile's first stage rides on this tile's last copies
            // when both tiles use the same lane offsets
            const uint8_t *nab = q.ab, *nwb = q.wb, *nsab = q.sab, *nswb = q.swb;
            bool chain = false;
            if (has_next && p.xnext && q.full) {
                const TilePlan qn = tile_plan<BM>(params_reloaded(), seq.base + inext);
                chain = qn.full;
                nab = qn.ab;
                nwb = qn.wb;
                nsab = qn.sab;
                nswb = qn.swb;
            }
            chained = chain;
            const bool pf = p.pfd > 0 && ROLE == kCopyTop && (wave == 1 || q.nt < 4);
#pragma unroll
            for (int mi = 0; mi < MS; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) pend[ni] = v4f{0.f, 0.f, 0.f, 0.f};
            auto issue_next = [&](int64_t kb) __attribute__((always_inline)) {
                // stage kb + 1 of this tile, or the next tile's stage 0, or
                // (neither) a re-copy of the last block into the free slot
                const bool last = kb + 1 >= p.KB;
                const bool nx = last && chain;
                const int64_t k = last ? (nx ? 0 : p.KB - 1) : kb + 1;
                issue(nx ? nab : q.ab, nx ? nwb : q.wb, nx ? nsab : q.sab, nx ? nswb : q.swb, k, (int)((kb + 1) & 1));
            };
            auto kblock = [&](int64_t kb) __attribute__((always_inline)) {
                // this wave's copies of stage kb have landed (a prefetch issued
                // after them may still be in flight: loads complete in order)
                if constexpr (ROLE == kCopyTop) {
                    if (pf && kb > 0 && kb + p.pfd < p.KB) wait_vmcnt<1>();
                    else wait_vmcnt<0>();
                } else if constexpr (ROLE == kCopyMid) {
                    wait_vmcnt<0>();
                }
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage kb-1 are done
                __builtin_amdgcn_s_barrier();  // ... and every other wave's; stage kb-1 is free
                if constexpr (ROLE == kCopyTop) {
                    issue_next(kb);
                    if (pf && kb + 1 + p.pfd < p.KB)
                        dma4s((wave == 0 ? q.ab : q.wb) + (kb + 1 + p.pfd) * 128, pf_off(), sink);
                }
                const uint8_t* st = ring[kb & 1];
                const uint8_t* sta = st + (BM / 2) * wm * 128;
                const uint8_t* stb = st + TSB + 64 * wn * 128;
                const float* sca = reinterpret_cast<const float*>(st + TSS);
                const float* scw = reinterpret_cast<const float*>(st + TSW);
                v8i bfr[4];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) bfr[ni] = frag(stb + ni * 2048);
                v8i afn = frag(sta);
                if constexpr (MX) {
                    int eb[4];
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        eb[ni] = w_e8m0(p, __float_as_uint(scw[64 * wn + 16 * ni + frow]), kb);
                    float san = sca[asl((BM / 2) * wm + frow)];
#pragma unroll
                    for (int mi = 0; mi < MS; ++mi) {
                        if constexpr (ROLE == kCopyMid) {
                            if (mi == MID) issue_next(kb);
                        }
                        const v8i af = afn;
                        const int ea = act_e8m0(p, __float_as_uint(san), kb);
                        if (mi < MS - 1) {
                            afn = frag(sta + (mi + 1) * 2048);
                            san = sca[asl((BM / 2) * wm + 16 * (mi + 1) + frow)];
                        }
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni)
                            acc[mi][ni] = mfma_fp8_mx(af, bfr[ni], acc[mi][ni], ea, eb[ni]);
                    }
                } else if constexpr (W1) {
                    float swv[4];
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) swv[ni] = scw[64 * wn + 16 * ni + frow];
                    // this lane's first token row (128-row tiles: its scale slot per subtile)
                    const int tr = (BM / 2) * wm + 4 * (lane >> 4);
                    const uint8_t* sab = reinterpret_cast<const uint8_t*>(sca) + 4 * asl(tr);
                    float4 tn = *reinterpret_cast<const float4*>(sab);
#pragma unroll
                    for (int mi = 0; mi < MS; ++mi) {
                        if constexpr (ROLE == kCopyMid) {
                            if (mi == MID) issue_next(kb);
                        }
                        const v8i af = afn;
                        const float sa4[4] = {tn.x, tn.y, tn.z, tn.w};
                        if (mi < MS - 1) {
                            afn = frag(sta + (mi + 1) * 2048);
                            tn = *reinterpret_cast<const float4*>(
                                MS == 8 ? sab + 64 * (mi + 1)
                                        : reinterpret_cast<const uint8_t*>(sca + asl(tr + 16 * (mi + 1))));
                        }
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) {
                            const v4f qv = mfma_fp8(af, bfr[ni], v4f{0.f, 0.f, 0.f, 0.f});
                            fold(mi == 0 ? MS - 1 : mi - 1, ni);
                            pend[ni] = qv;
                            if (mi == 0) psw[ni] = swv[ni];
                        }
#pragma unroll
                        for (int k = 0; k < 4; ++k) psa[k] = sa4[k];
                    }
                } else {
                    const float sws = scw[64 * wn];
                    float san = sca[asl((BM / 2) * wm + frow)];
#pragma unroll
                    for (int mi = 0; mi < MS; ++mi) {
                        if constexpr (ROLE == kCopyMid) {
                            if (mi == MID) issue_next(kb);
                        }
                        const v8i af = afn;
                        const float sa = san;
                        if (mi < MS - 1) {
                            afn = frag(sta + (mi + 1) * 2048);
                            san = sca[asl((BM / 2) * wm + 16 * (mi + 1) + frow)];
                        }
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) {
                            const v4f qv = mfma_fp8(bfr[ni], af, v4f{0.f, 0.f, 0.f, 0.f});
                            fold(mi == 0 ? MS - 1 : mi - 1, ni);
                            pend[ni] = qv;
                        }
                        ps = sa * sws;
                    }
                }
            };
#pragma clang loop unroll(disable)
            for (int64_t kb = 0; kb < p.KB; ++kb) kblock(kb);
            if constexpr (!MX) {
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) fold(MS - 1, ni);
            }
            // this wave's results to z, subtile by subtile
            KGParams& pr = params_reloaded();
            const int64_t r0 = q.m0 + (BM / 2) * wm, c0 = q.n0 + 64 * wn, zrs = pr.G * pr.R;
            uint16_t* zb = pr.z + r0 * zrs + q.g * pr.R + c0;
#pragma unroll
            for (int mi = 0; mi < MS; ++mi) store_sub(mi, zb, zrs, pr.T - r0, pr.R - c0);
        }
    };
    if (wave < 2) run(std::integral_constant<int, kCopyTop>{});
    else if (copier) run(std::integral_constant<int, kCopyMid>{});
    else run(std::integral_constant<int, kComputeOnly>{});
    wait_vmcnt<0>();  // no copy may still be writing LDS when the workgroup exits
}

// ---------------------------------------------------------------------------
// Decode kernel (few tokens): the weight stream is the cost.
// Workgroup tile: one group, 64 tokens (128 above 64 tokens) x 64 columns,
// the whole K.  Each K-block is one pipeline stage in LDS: the 64x128-byte
// (128x128-byte) activation slab, the 64x128-byte weight slab and the
// block's scales, all copied by the DMA form
// of the global loads (global_load_lds: no staging registers).  The eight
// waves form DKS K-groups of four; each K-group walks its share of the
// K-blocks through its own ring of DNS stages (DNS2 with 128-token tiles),
// all but one of them in flight, with
// one s_waitcnt + barrier per K-block.  Every wave of a K-group issues a
// quarter of the copies (the one-launch path: waves 0-1 half each).  Rows
// are 128 bytes with the 16-byte pieces XOR-swizzled, which makes the
// fragment reads conflict-free.  For the MFMAs
// the waves of a K-group split M: wave w owns token rows 16w..16w+15 (32w..
// 32w+31 with 128-token tiles) against all 64 columns (one or two activation
// fragments and four weight fragments per K-block, a
// third less LDS reading than splitting N); the K-groups' partial tiles are
// summed through LDS and written as whole 128-byte rows of z.
#ifndef OPROJ_DEC_DNS
#define OPROJ_DEC_DNS 4
#endif
#ifndef OPROJ_DEC_DKS
#define OPROJ_DEC_DKS 2
#endif
constexpr int DBM = 64, DBN = 64, DNS = OPROJ_DEC_DNS, DKS = OPROJ_DEC_DKS;
constexpr int DSTAGE = 64 * 128 * 2 + 512;  // activations + weights + scales
// Token rows of a workgroup's tile: 64 * MM.  With MM = 2 (65-256 tokens)
// the 128-token activation slab and the 64-row weight slab of a stage, with
// their scales, take 24.75 KiB, so each K-group's ring holds 3 stages.
template <int MM>
constexpr int dstage() { return (64 * MM + DBN) * (128 + 4); }
static_assert(dstage<1>() == DSTAGE, "one stage layout for 64-token tiles");
constexpr int DNS2 = 3;  // ring stages with 128-token tiles
constexpr int DVM = 9;  // one-launch path: copy instructions per copying wave per stage
constexpr int DPROW = DBN + 4;  // fp32 per row of an epilogue partial tile (pad against bank conflicts)
static_assert(DKS * DBM * DPROW * 4 <= DKS * DNS * DSTAGE, "the epilogue fits in the ring");

// Barrier state of the one-launch decode path: one 64-bit word per group, on
// a cache line of its own, in the caller's workspace (zero before the first
// call with that workspace).  Fields, low bit first: arrivals at the current
// barrier (9 bits), the sum of the arrivals' XCD numbers (12 bits) and of
// their squares (16 bits), whether the previous barrier's arrivals ran on
// more than one XCD (1 bit), and the count of barriers the group has completed
// (its epoch, the top 26 bits).  One returning atomic add per arrival; the
// last arrival replaces the word with the next epoch and its XCD flag in a
// second add, so every launch leaves the word ready for the next one whatever
// its group size.  Launches with distinct workspaces never meet.
constexpr int kMaxFusedGroups = 256;
constexpr int kSyncStride = 16;  // 128-byte cache line
constexpr int kGroupSpinLimit = 4096;  // bounded wait: a missing workgroup is covered by a fallback
constexpr int kSyncSum = 9, kSyncSq = 21, kSyncMixed = 37, kSyncEpoch = 38;

// XCD (XCC) this wave runs on.
__device__ __forceinline__ uint64_t xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xFu; }

// Arrive at group g's barrier of n (at most 256) workgroups and wait for the
// others.  Returns 0 when every workgroup of the group arrived and all ran on
// one XCD, 1 when they arrived from several XCDs, 2 when the wait gave up
// (the caller then does the missing work itself).  Called by one thread.
__device__ int group_barrier(uint64_t* sync, int64_t g, int64_t n, int spin) {
    uint64_t* word = sync + kSyncStride * g;
    const uint64_t x = xcc_id();
    const uint64_t inc = 1ull + (x << kSyncSum) + ((x * x) << kSyncSq);
    const uint64_t old = __hip_atomic_fetch_add(word, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t epoch = old >> kSyncEpoch;
    if ((old & ((1ull << kSyncSum) - 1)) == (uint64_t)(n - 1)) {
        const uint64_t fin = old + inc;
        const uint64_t s1 = (fin >> kSyncSum) & ((1ull << (kSyncSq - kSyncSum)) - 1);
        const uint64_t s2 = (fin >> kSyncSq) & ((1ull << (kSyncMixed - kSyncSq)) - 1);
        const uint64_t mixed = (uint64_t)n * s2 != s1 * s1;  // equal only when every x is the same
        const uint64_t next = ((epoch + 1) << kSyncEpoch) | (mixed << kSyncMixed);
        __hip_atomic_fetch_add(word, next - fin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return (int)mixed;
    }
    for (int it = 0; it < spin; ++it) {
        const uint64_t w = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((w >> kSyncEpoch) != epoch) return (int)((w >> kSyncMixed) & 1);
        __builtin_amdgcn_s_sleep(2);
    }
    return 2;
}

// One workgroup's output tile (the whole decode pipeline); ring is the
// workgroup's LDS.  QCH > 0 is the one-launch path: the workgroup also
// quantises its share of the group's activations (items of QCH heads, with
// the rq::Params q) before the GEMM reads them.
template <bool MX, bool W1, int QCH, int MM = 1, int NS = DNS>
__device__ __forceinline__ void decode_tile(const GParams& p, uint8_t (&ring)[DKS][NS][dstage<MM>()],
                                            const rq::Params& q) {
    static_assert(QCH == 0 || (MM == 1 && NS == DNS), "the one-launch path runs 64-token tiles");
    constexpr int BM = 64 * MM;             // token rows of the tile
    constexpr int STG = dstage<MM>();       // bytes per stage
    constexpr int SWO = BM * 128;           // weight slab offset in a stage
    constexpr int SCO = (BM + DBN) * 128;   // scale offset in a stage
    static_assert(DKS * BM * DPROW * 4 <= DKS * NS * STG, "the epilogue fits in the ring");
    const int tid = threadIdx.x, lane = tid & 63;
    const int kq = __builtin_amdgcn_readfirstlane(tid >> 8);           // K-group
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);  // column group within the tile
    // Copying waves of the K-group: all four on the plain path (one wave
    // issues a DMA copy only about every hundred cycles, so two waves' nine
    // copies per K-block took about half of each step), waves 0-1 on the
    // one-launch path, whose prologue waits count that plan.
    constexpr int CW = QCH == 0 ? 4 : 2;
    constexpr int CR = DBN / CW;  // weight rows per copying wave
    constexpr int CI = CR / 8;    // weight copy instructions per copying wave
    constexpr int CRA = BM / CW;  // activation rows per copying wave
    constexpr int CIA = CRA / 8;  // activation copy instructions per copying wave
    const bool copier = wave < CW;
    // scale gathers: waves 0-1 (64-token tiles), waves 0..MM (larger tiles)
    const bool scaler = wave < (MM == 1 ? 2 : MM + 1);
    static_assert(QCH == 0 || 2 * CI + 1 == DVM, "the one-launch waits count DVM copies per step");
    const TileCoord tc = tile_coord(p);
    const int64_t g = tc.g, mt = tc.mt, nt = tc.nt;
    const int64_t m0 = mt * BM, n0 = nt * DBN;
    // this K-group's K-blocks: [kb0, kb0 + nkb)
    const int64_t kb0 = p.KB * kq / DKS;
    const int64_t nkb = p.KB * (kq + 1) / DKS - kb0;

    // ---- copy plan.  Copying wave c: activation rows CR*c..CR*c+CR-1 and the
    // same weight rows (8 rows of 128 bytes per instruction); waves c = 0-1
    // also make one scale gather (lanes 0-31: activation scales of tokens
    // 32c+l; lanes 32-63: weight scales of columns 32c+l-32).  Sources are
    // uniform bases plus 32-bit lane offsets.
    const uint8_t* abase = p.a + g * p.sg;
    const uint8_t* wbase = p.w + g * p.R * p.D;
    uint32_t off[CIA + CI];
    if (copier) {
#pragma unroll
        for (int j = 0; j < CIA; ++j) {
            const int row = CRA * wave + 8 * j + (lane >> 3);
            const int piece = (lane & 7) ^ swz(row);
            int64_t m = m0 + row;
            m = m < p.T ? m : p.T - 1;  // rows past T are computed but never stored
            off[j] = (uint32_t)(m * p.st + piece * 16);
        }
#pragma unroll
        for (int j = 0; j < CI; ++j) {
            const int row = CR * wave + 8 * j + (lane >> 3);
            const int piece = (lane & 7) ^ swz(row);
            int64_t n = n0 + row;
            n = n < p.R ? n : p.R - 1;
            off[CIA + j] = (uint32_t)(n * p.D + piece * 16);
        }
    }
    // the scale gather mixes two sources across lanes: 64-bit lane addresses
    // (larger tiles: wave c < MM gathers the activation scales of tokens
    // 64c + l, wave MM the weight scales of the 64 columns)
    const float* ssrc;
    int64_t sstep;
    int kshl;  // K-blocks per scale word: activation words may pack four
    if (MM > 1 ? wave < MM : lane < 32) {
        int64_t m = m0 + (MM > 1 ? 64 * wave + lane : 32 * (wave & 1) + lane);
        m = m < p.T ? m : p.T - 1;
        ssrc = p.sa + m * p.sst + g * p.ssg;
        sstep = p.sskb;
        kshl = p.kshift;
    } else {
        int64_t n = n0 + (MM > 1 ? lane : 32 * (wave & 1) + (lane - 32));
        n = n < p.R ? n : p.R - 1;
        ssrc = p.sw + wscale_index(p, g * p.R + n, 0);
        sstep = 1;
        kshl = p.wkshift;
    }
    const uint32_t ring0 = lds_offset(&ring[kq][0][0]);
    // step i's copies: the activation slab and the scales (CI + 1
    // instructions on waves 0-1, CI on the others), the weight slab (CI)
    auto issue_a = [&](int64_t i, int slot) __attribute__((always_inline)) {
        const int64_t kb = kb0 + i;
        const uint32_t st = ring0 + (uint32_t)(slot * STG);
#pragma unroll
        for (int j = 0; j < CIA; ++j) dma16s(abase + kb * 128, off[j], st + (CRA * wave + 8 * j) * 128);
        if (scaler) dma4(ssrc + (kb >> kshl) * sstep, st + SCO + 256 * wave);
    };
    auto issue_w = [&](int64_t i, int slot) __attribute__((always_inline)) {
        const int64_t kb = kb0 + i;
        const uint32_t st = ring0 + (uint32_t)(slot * STG);
#pragma unroll
        for (int j = 0; j < CI; ++j) {
            if (OPROJ_DEC_W_NT)
                dma16s_nt(wbase + kb * 128, off[CIA + j], st + SWO + (CR * wave + 8 * j) * 128);
            else
                dma16s(wbase + kb * 128, off[CIA + j], st + SWO + (CR * wave + 8 * j) * 128);
        }
    };
    auto issue = [&](int64_t i, int slot) __attribute__((always_inline)) {
        issue_a(i, slot);
        issue_w(i, slot);
    };

    if constexpr (QCH == 0) {
        if (copier) {
#pragma unroll
            for (int s = 0; s < NS - 1; ++s)
                if (s < nkb) issue(s, s);
        }
    } else {
        static_assert(QCH == 0 || DNS == 4, "the one-launch waits below assume a 4-stage ring");
        // One-launch path (the launcher guarantees nkb >= DNS and one M-tile).
        // The weights of the first DNS-1 steps do not depend on the
        // quantisation: the copying waves request them first.
        if (copier) {
#pragma unroll
            for (int s = 0; s < DNS - 1; ++s) issue_w(s, s);
        }
        // All eight waves then quantise this workgroup's share of the group's
        // items (token, head chunk) into the workspace; a copying wave's
        // first wait also covers its weight copies, which were issued first.
        const rq::Wave<QCH> qwv(q, lane);
        auto quantise = [&](int64_t first, int64_t step) __attribute__((always_inline)) {
            const int64_t items = q.T * q.nchunk;
            for (int64_t it = first; it < items; it += step) {
                const int64_t t = it / q.nchunk, chunk = it % q.nchunk;
                typename rq::Wave<QCH>::RowsT raw;
                qwv.load_rows(t, g, chunk, raw);
                const int64_t ps = q.pos[t];
                float4 cs, sn;
                qwv.load_table(ps, cs, sn);
                // system-coherent stores: visible to the group's readers on
                // this XCD through L2 and on any other XCD through memory
                qwv.template process<true>(t, g, chunk, ps, raw, cs, sn);
            }
            wait_vmcnt<0>();  // the stores have completed before the arrival
        };
        quantise(nt * 8 + (tid >> 6), p.ntiles * 8);
        __shared__ int sync_state;
        __syncthreads();
        if (tid == 0) sync_state = group_barrier(p.sync, g, p.ntiles, p.spin);
        __syncthreads();
        if (sync_state == 2) {
            // a workgroup of the group did not arrive in time: quantise the
            // whole group here (the same bytes the others write)
            quantise(tid >> 6, 8);
            __syncthreads();
        }
        // A reader's L2 on an XCD other than a writer's may hold stale lines
        // of the workspace from an earlier launch: drop them.  Only then: the
        // invalidation also drops the lines that the XCD's other workgroups
        // are sharing, which costs far more than the instruction.
        if (sync_state != 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (copier) {
#pragma unroll
            for (int s = 0; s < DNS - 1; ++s) issue_a(s, s);
        }
    }

    v4f acc[MM][4];
#pragma unroll
    for (int mi = 0; mi < MM; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;
    const int p0 = 2 * (lane >> 4);
    const int64_t nstages = (p.KB + DKS - 1) / DKS;  // the largest share: same barrier count in every group
    for (int64_t i = 0; i < nstages; ++i) {
        // this wave's copies of stage i have landed; the copies of the stages
        // after it that were issued (at most DNS-2, none past the group's
        // last block) may still be in flight
        if (copier) {
            if (QCH > 0 && i < DNS - 1) {
                // the prologue issued the weights of steps 0..DNS-2 before their
                // activations: after step i's activations come those of steps
                // i+1..DNS-2 (5 instructions each) and the i whole steps issued
                // by the loop so far
                if (i == 0) wait_vmcnt<5 * (DNS - 2)>();
                else if (i == 1) wait_vmcnt<5 * (DNS - 3) + DVM>();
                else wait_vmcnt<5 * (DNS - 4 > 0 ? DNS - 4 : 0) + 2 * DVM>();
            } else if (scaler) {
                wait_ahead<NS - 2, CIA + CI + 1>(nkb - 1 - i);
            } else {
                wait_ahead<NS - 2, CIA + CI>(nkb - 1 - i);
            }
        }
        __builtin_amdgcn_s_barrier();  // ... and every other wave's (no fence)
        if (copier && i + NS - 1 < nkb) issue(i + NS - 1, (int)((i + NS - 1) % NS));
        if (i >= nkb) continue;        // uniform per wave group
        const uint8_t* st = ring[kq][i % NS];
        // wave w: the 16*MM token rows 16*MM*w.. against all 64 columns (MM
        // activation fragments, four weight fragments per K-block)
        const float* sc = reinterpret_cast<const float*>(st + SCO);
        // scales, 64-token tiles: [64 * c + t] activation scale of token
        // 32c + t, [64 * c + 32 + j] weight scale of column 32c + j (c =
        // copying wave); larger tiles: [t] token t, [BM + j] column j
        auto asc = [&](int r) __attribute__((always_inline)) { return MM > 1 ? r : 64 * (r >> 5) + (r & 31); };
        auto wsc = [&](int n) __attribute__((always_inline)) { return MM > 1 ? BM + n : 64 * (n >> 5) + 32 + (n & 31); };
        v8i af[MM];
        float4 t4[MM];
        int ea[MM];
#pragma unroll
        for (int mi = 0; mi < MM; ++mi) {
            const int r = 16 * (MM * wave + mi) + frow;
            const uint4 lo = *reinterpret_cast<const uint4*>(st + r * 128 + 16 * (p0 ^ swz(r)));
            const uint4 hi = *reinterpret_cast<const uint4*>(st + r * 128 + 16 * ((p0 + 1) ^ swz(r)));
            af[mi] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const int r0 = 16 * (MM * wave + mi);  // this fragment's 16 token scales
            if constexpr (MX) ea[mi] = act_e8m0(p, __float_as_uint(sc[asc(r0 + frow)]), kb0 + i);
            else t4[mi] = *reinterpret_cast<const float4*>(sc + asc(r0 + 4 * (lane >> 4)));
        }
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int r = 16 * ni + frow;
            const uint4 lo = *reinterpret_cast<const uint4*>(st + SWO + r * 128 + 16 * (p0 ^ swz(r)));
            const uint4 hi = *reinterpret_cast<const uint4*>(st + SWO + r * 128 + 16 * ((p0 + 1) ^ swz(r)));
            const v8i bfr = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const float swv = sc[wsc(16 * ni + (W1 || MX ? frow : 0))];
#pragma unroll
            for (int mi = 0; mi < MM; ++mi) {
                if constexpr (MX) {
                    acc[mi][ni] = mfma_fp8_mx(af[mi], bfr, acc[mi][ni], ea[mi], w_e8m0(p, __float_as_uint(swv), kb0 + i));
                } else {
                    const float cmb[4] = {t4[mi].x * swv, t4[mi].y * swv, t4[mi].z * swv, t4[mi].w * swv};
                    const v4f pp = mfma_fp8(af[mi], bfr, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                    for (int i2 = 0; i2 < 4; ++i2) acc[mi][ni][i2] = __builtin_fmaf(pp[i2], cmb[i2], acc[mi][ni][i2]);
                }
            }
        }
    }
    wait_vmcnt<0>();  // (already true: the last stage was waited for in full)
    __syncthreads();

    // ---- each K-group's fp32 partial tile into LDS (the ring is free now),
    // then every thread sums one 8-column chunk of one row over the K-groups
    // and writes it to z as bf16: whole 128-byte tile rows, 16-byte stores
    float* part = reinterpret_cast<float*>(&ring[0][0][0]);  // [DKS][BM][DPROW]
#pragma unroll
    for (int mi = 0; mi < MM; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part[(kq * BM + 16 * (MM * wave + mi) + 4 * (lane >> 4) + i) * DPROW + 16 * ni + frow] = acc[mi][ni][i];
    __syncthreads();
    for (int idx = tid; idx < BM * (DBN / 8); idx += DKS * 256) {
        const int r = idx / (DBN / 8), ch = idx % (DBN / 8);
        float4 s0 = *reinterpret_cast<const float4*>(part + r * DPROW + 8 * ch);
        float4 s1 = *reinterpret_cast<const float4*>(part + r * DPROW + 8 * ch + 4);
#pragma unroll
        for (int q = 1; q < DKS; ++q) {
            const float4 u0 = *reinterpret_cast<const float4*>(part + (q * BM + r) * DPROW + 8 * ch);
            const float4 u1 = *reinterpret_cast<const float4*>(part + (q * BM + r) * DPROW + 8 * ch + 4);
            s0.x += u0.x; s0.y += u0.y; s0.z += u0.z; s0.w += u0.w;
            s1.x += u1.x; s1.y += u1.y; s1.z += u1.z; s1.w += u1.w;
        }
        const uint4 v = {f32_to_bf16_bits(s0.x) | (f32_to_bf16_bits(s0.y) << 16),
                         f32_to_bf16_bits(s0.z) | (f32_to_bf16_bits(s0.w) << 16),
                         f32_to_bf16_bits(s1.x) | (f32_to_bf16_bits(s1.y) << 16),
                         f32_to_bf16_bits(s1.z) | (f32_to_bf16_bits(s1.w) << 16)};
        const int64_t row = m0 + r, col = n0 + 8 * ch;
        if (row < p.T && col < p.R) *reinterpret_cast<uint4*>(p.z + (row * p.G + g) * p.R + col) = v;
    }
}

template <bool MX, bool W1, int MM>
__global__ __launch_bounds__(DKS * 256) void gemm_fp8_decode_kernel(GParams p) {
    constexpr int NS = MM == 1 ? DNS : DNS2;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[DKS][NS][dstage<MM>()];
    const rq::Params none{};
    decode_tile<MX, W1, 0, MM, NS>(p, ring, none);
}

// One launch for a decode step: quantisation (spread over the GEMM's own
// workgroups, a barrier per group) and the grouped GEMM.
template <bool MX, bool W1, int QCH>
__global__ __launch_bounds__(DKS * 256) void fused_decode_kernel(GParams p, rq::Params q) {
    __shared__ __attribute__((aligned(1024))) uint8_t ring[DKS][DNS][DSTAGE];
    decode_tile<MX, W1, QCH>(p, ring, q);
}

// Fills p's tile map for a grid of G x mtiles x ntiles workgroups of `threads`
// work-items; false when the grid is beyond one launch (more than 2^32 - 1
// work-items in all).
bool set_tile_map(GParams& p, int threads) {
    const int64_t nblocks = p.G * p.mtiles * p.ntiles;
    if (nblocks < 1 || nblocks > (int64_t)UINT32_MAX / threads) return false;
    p.tpg = (uint32_t)(p.mtiles * p.ntiles);
    p.nt32 = (uint32_t)p.ntiles;
    p.xcd_per = 0;
    p.xcd_shift = 0;
    const int nx = current_device_info().xcds;
    if (nx > 1 && (nx & (nx - 1)) == 0 && nblocks % nx == 0) {
        p.xcd_shift = __builtin_ctz((unsigned)nx);
        p.xcd_per = (uint32_t)(nblocks / nx);
    }
    return true;
}

template <int MM>
void launch_decode(const GParams& p, bool mx, bool w1, hipStream_t stream) {
    const dim3 grid(p.tpg * (uint32_t)p.G), block(DKS * 256);
    if (mx) {
        if (w1)
            hipLaunchKernelGGL((gemm_fp8_decode_kernel<true, true, MM>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_fp8_decode_kernel<true, false, MM>), grid, block, 0, stream, p);
    } else {
        if (w1)
            hipLaunchKernelGGL((gemm_fp8_decode_kernel<false, true, MM>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((gemm_fp8_decode_kernel<false, false, MM>), grid, block, 0, stream, p);
    }
}

}  // namespace


const char* fused_decode_unfit(int64_t T, int64_t G, int64_t hpg, int64_t R) {
    // eligible: one M-tile, every K-group long enough for the prologue, a
    // two- or four-head quantisation item, and every workgroup resident at
    // once (one per CU) so that the per-group barriers complete without the
    // fallback
    if (T > DBM) return "more than 64 tokens";
    if (G > kMaxFusedGroups) return "more than 256 groups";
    const int ch = rq::heads_per_item(hpg);
    if (ch != 2 && ch != 4) return "heads_per_group is neither 2 nor a multiple of 4";
    if (hpg * 512 / 128 / DKS < DNS) return "head dimension too short for the copy pipeline";
    if (G * ((R + DBN - 1) / DBN) > current_device_info().cus)
        return "more workgroups (n_groups x o_lora_rank / 64) than compute units";
    return nullptr;
}

hipError_t launch_fused_decode(const RopeQuantArgs& qa, const GroupedGemmArgs& a, uint64_t* sync,
                               hipStream_t stream, bool* launched) {
    *launched = false;
    if (fused_decode_unfit(a.T, a.G, qa.hpg, a.R)) return hipSuccess;
    const int64_t KB = a.D / 128;
    const int64_t ntiles = (a.R + DBN - 1) / DBN;
    const int ch = rq::heads_per_item(qa.hpg);
    GParams p;
    p.a = a.a;
    p.sa = static_cast<const float*>(a.sa);
    p.w = a.w;
    p.sw = static_cast<const float*>(a.sw);
    p.z = a.z;
    p.T = a.T;
    p.G = a.G;
    p.D = a.D;
    p.R = a.R;
    p.KB = KB;
    p.st = a.lay.stride_t;
    p.sg = a.lay.stride_g;
    p.sst = a.lay.s_stride_t;
    p.ssg = a.lay.s_stride_g;
    p.sskb = a.lay.s_stride_kb;
    p.w_shift = a.w_1x128 ? 0 : 7;
    p.e8 = a.a_e8m0;
    p.kshift = a.a_e8m0 ? 2 : 0;
    p.we8 = a.w_e8m0;
    p.wkshift = a.w_e8m0 ? 2 : 0;
    p.kbw = a.w_e8m0 ? KB / 4 : KB;
    p.mtiles = 1;
    p.ntiles = ntiles;
    if (!set_tile_map(p, DKS * 256)) return hipErrorInvalidConfiguration;
    p.sync = sync;
    // OPROJ_FUSED_DECODE_SPIN_LIMIT (diagnostics and tests) lowers the polls a
    // workgroup makes before it quantises its whole group itself; 0 sends every
    // workgroup but the last arrival of each group down that fallback
    p.spin = kGroupSpinLimit;
    if (const char* e = getenv("OPROJ_FUSED_DECODE_SPIN_LIMIT")) {
        const long v = strtol(e, nullptr, 10);
        p.spin = v < 0 ? 0 : (v < kGroupSpinLimit ? (int)v : kGroupSpinLimit);
    }
    const rq::Params q = rq::make_params(qa, ch);
    const dim3 grid((unsigned)(a.G * ntiles)), block(DKS * 256);
#define OPROJ_FUSED_LAUNCH(MXV, W1V, CHV) \
    hipLaunchKernelGGL((fused_decode_kernel<MXV, W1V, CHV>), grid, block, 0, stream, p, q)
#define OPROJ_FUSED_CH(MXV, W1V) \
    if (ch == 2) OPROJ_FUSED_LAUNCH(MXV, W1V, 2); else OPROJ_FUSED_LAUNCH(MXV, W1V, 4)
    if (a.mx) {
        if (a.w_1x128) { OPROJ_FUSED_CH(true, true); } else { OPROJ_FUSED_CH(true, false); }
    } else {
        if (a.w_1x128) { OPROJ_FUSED_CH(false, true); } else { OPROJ_FUSED_CH(false, false); }
    }
#undef OPROJ_FUSED_CH
#undef OPROJ_FUSED_LAUNCH
    *launched = true;
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, hipStream_t stream) {
    GParams p;
    p.a = a.a;
    p.sa = static_cast<const float*>(a.sa);  // fp32 scales or UE8M0 words: copied as 4-byte words
    p.w = a.w;
    p.sw = static_cast<const float*>(a.sw);  // fp32 scales or UE8M0 words: copied as 4-byte words
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
    p.we8 = a.w_e8m0;
    p.wkshift = a.w_e8m0 ? 2 : 0;
    p.kbw = a.w_e8m0 ? p.KB / 4 : p.KB;
    p.e8 = a.a_e8m0;
    p.kshift = a.a_e8m0 ? 2 : 0;
    // decode kernel for few tokens (the weight stream dominates), tile kernel
    // otherwise.  Up to 256 tokens the tile kernel has a single M-tile per
    // group, so at G=16, R=1024 it keeps 64 of 256 CUs busy (52-59 us for any
    // T <= 256), while the decode kernel's tiles fill the chip (17-18 us at
    // 64 tokens, 22 at 96-128, 40-43 at 160-256); from 320 tokens on the
    // tile kernel is ahead (55 vs 63 us).
    const bool decode = a.T <= 256;
    if (decode) {
        // 64-token tiles up to 64 tokens, 128-token tiles above (one weight
        // stream per 128 tokens instead of two)
        const int bm = a.T <= DBM ? DBM : 2 * DBM;
        p.mtiles = (a.T + bm - 1) / bm;
        p.ntiles = (a.R + DBN - 1) / DBN;
        if (!set_tile_map(p, DKS * 256)) return hipErrorInvalidConfiguration;
        if (bm == DBM)
            launch_decode<1>(p, a.mx != 0, a.w_1x128 != 0, stream);
        else
            launch_decode<2>(p, a.mx != 0, a.w_1x128 != 0, stream);
    } else {
        // 256-row tiles, or 128-row tiles when 256-row tiles would leave at
        // least half the CUs idle and 128-row tiles still fit in one round.
        // A 128-row tile costs 62-64% of a 256-row one (its copies per MFMA
        // are 1.5x), so only then do they pay: G=16, R=1024, 288-512 tokens
        // 46.8-49.8 against 55.8-60.3 us; at 640-1024 tokens (a second round
        // of 128-row tiles) 80-90 against 60-72 us.
        const DeviceInfo dev = current_device_info();
        const int64_t nt = (a.R + TBN - 1) / TBN;
        const int64_t t256 = a.G * ((a.T + 255) / 256) * nt, t128 = a.G * ((a.T + 127) / 128) * nt;
        const int bm = 2 * t256 <= dev.cus && t128 <= dev.cus ? 128 : 256;
        p.mtiles = (a.T + bm - 1) / bm;
        p.ntiles = nt;
        if (!set_tile_map(p, TNW * 64)) return hipErrorInvalidConfiguration;
        p.pfd = kTilePrefetch;
        // persistent grid: at most one workgroup per CU, the same number on every XCD
        const uint32_t nblocks = p.tpg * (uint32_t)p.G;
        uint32_t wgs;
        if (p.xcd_per) {
            const uint32_t per = (uint32_t)(dev.cus >> p.xcd_shift);
            wgs = (per < p.xcd_per ? (per > 0 ? per : 1u) : p.xcd_per) << p.xcd_shift;
        } else {
            wgs = nblocks < (uint32_t)dev.cus ? nblocks : (uint32_t)dev.cus;
        }
        p.ntot = nblocks;
        p.xnext = a.R % TBN == 0;
        const dim3 grid(wgs), block(TNW * 64);
#define OPROJ_PTILE(MXV, W1V)                                                                      \
    if (bm == 256) hipLaunchKernelGGL((gemm_fp8_ptile_kernel<MXV, W1V, 8>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((gemm_fp8_ptile_kernel<MXV, W1V, 4>), grid, block, 0, stream, p)
        if (a.mx) {
            if (a.w_1x128) { OPROJ_PTILE(true, true); } else { OPROJ_PTILE(true, false); }
        } else {
            if (a.w_1x128) { OPROJ_PTILE(false, true); } else { OPROJ_PTILE(false, false); }
        }
#undef OPROJ_PTILE
    }
    return hipGetLastError();
}

}  // namespace oproj
