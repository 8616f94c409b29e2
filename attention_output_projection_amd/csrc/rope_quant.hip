// rope_quant.hip -- step a1 + a2 on gfx950: inverse RoPE on the last 64 dims
// of each 512-dim head, then 1x128 block FP8 e4m3fn quantisation, in one pass
// over the bf16 attention output (vLLM API page
// "vllm.models.deepseek_v4.common.ops.fused_inv_rope_fp8_quant",
// fused_inv_rope_fp8_quant; sglang source page
// "python/sglang/srt/models/deepseek_v4.py", MQALayer.forward).
//
// Work unit: one wave takes one (token, group, head-chunk) item of CH heads.
// Lane l holds elements 8l..8l+7 of every head of the chunk (one 16-byte load
// per head: each head row is read as one coalesced 1 KiB transaction), so the
// 16-lane row c of the wave covers quantisation block c (dims 128c..128c+127)
// and lanes 56..63 hold the 64 RoPE dims.  Per item:
//   * lanes 56..63 fetch cos[4(l-56)..+3] and sin[..] of the token's position
//     and rotate their 4 pairs: e' = fma(d, s, e*c), d' = fma(-e, s, d*c);
//   * per head, |v| max over 8 values, then a 16-lane DPP max gives the amax
//     of each block;
//   * the CH x 4 block scales are computed once each (lane 16c+j, j < CH,
//     computes block (j, c): s = max(amax,1e-10)/448, optional pow2 ceiling,
//     r = 1/s, both IEEE), then broadcast back over the row;
//   * codes: q = v/s via r and one correction step (exact quotient), clamp to
//     +-448, hardware e4m3fn conversion; 8 bytes per lane per head.
// Items are numbered in address order (chunk fastest, then group, then
// token) and dealt round-robin over all waves of the grid, so at any moment
// the grid reads one compact window of the input (DRAM pages stay open).
// Each wave loads the next item (head rows, position, table row) while it
// works on the current one.  The input rows and the codes are streamed with
// non-temporal loads and stores (each byte is touched once here).  The
// kernel is HBM-bound: read 1 KiB + write 512 B per head row; a moderate
// population of waves (12 per CU) keeps enough in flight without crowding
// the memory controllers.  Small batches (a few thousand head rows) are
// latency-bound instead: items of two heads, one wave each.
#include "device_common.hpp"
#include "kernels.hpp"
#include "rq_item.hpp"

#pragma clang fp contract(off)

namespace oproj {

namespace {

constexpr int kWaves = 4;  // waves per workgroup

typedef rq::Params RQParams;

template <int CH, bool PIPE, bool F32>
__global__ __launch_bounds__(kWaves * 64) void inv_rope_quant_kernel(RQParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int64_t first = (int64_t)blockIdx.x * kWaves + wave;  // this wave's item k is first + k*nwaves
    if (first >= p.nitems) return;
    const rq::Wave<CH, F32> w(p, lane);

    int64_t tn, gn, cn;
    w.split(first, tn, gn, cn);
    typename rq::Wave<CH, F32>::RowsT rawn;
    w.load_rows(tn, gn, cn, rawn);
    int64_t psn = p.pos[tn];
    float4 csn, snn;
    w.load_table(psn, csn, snn);
    if constexpr (!PIPE) {  // one item per wave (small batches): no pipeline
        w.process(tn, gn, cn, psn, rawn, csn, snn);
        return;
    }

    // pipeline: rows and table row of item k+1 and the position of item k+2
    // are in flight while item k is processed
    int64_t t2, g2, c2;
    w.split(first + nwaves, t2, g2, c2);
    int64_t ps2 = p.pos[t2];

    for (int64_t item = first; item < p.nitems; item += nwaves) {
        const int64_t t = tn, g = gn, chunk = cn, ps = psn;
        const typename rq::Wave<CH, F32>::RowsT raw = rawn;
        const float4 cs = csn, sn = snn;
        // prefetch item + nwaves (its position is already here) and the
        // position of item + 2*nwaves
        tn = t2, gn = g2, cn = c2, psn = ps2;
        w.load_rows(tn, gn, cn, rawn);
        w.load_table(psn, csn, snn);
        w.split(item + 2 * nwaves, t2, g2, c2);
        ps2 = p.pos[t2];
        w.process(t, g, chunk, ps, raw, cs, sn);
    }
}

// ---------------------------------------------------------------------------
// Offline weight quantisation: one workgroup per (row block, 128-column block).
constexpr int kWqThreads = 256;

__global__ __launch_bounds__(kWqThreads) void quantize_weight_kernel(const float* __restrict__ w,
                                                                    uint8_t* __restrict__ codes,
                                                                    void* __restrict__ scales,
                                                                    int64_t rows, int64_t K,
                                                                    int64_t brows, int pow2, int e8m0) {
    __shared__ float red[kWqThreads / 64];
    const int64_t rb = blockIdx.x;
    const int64_t kb = blockIdx.y;
    const int64_t r0 = rb * brows;
    const int64_t r1 = (r0 + brows < rows) ? r0 + brows : rows;
    const int64_t n = (r1 - r0) * 128;
    float a = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += kWqThreads) {
        const int64_t r = r0 + i / 128, k = kb * 128 + (i % 128);
        a = fmaxf(a, fabsf(w[r * K + k]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = red[0];
#pragma unroll
    for (int i = 1; i < kWqThreads / 64; ++i) a = fmaxf(a, red[i]);
    float s = fmaxf(a, kAmaxFloor) / kFp8Max;
    if (pow2) s = pow2_ceil(s);
    const float r = 1.0f / s;
    if (threadIdx.x == 0) {
        if (e8m0)  // byte kb of the row: byte kb % 4 of word kb / 4, words in memory order
            static_cast<uint8_t*>(scales)[rb * (K / 128) + kb] = (uint8_t)((__float_as_uint(s) >> 23) & 0xFFu);
        else
            static_cast<float*>(scales)[rb * (K / 128) + kb] = s;
    }
    for (int64_t i = threadIdx.x; i < n; i += kWqThreads) {
        const int64_t rr = r0 + i / 128, k = kb * 128 + (i % 128);
        const float q = div_by_scale(w[rr * K + k], s, r);
        codes[rr * K + k] = (uint8_t)(cvt2_fp8<false>(q, 0.f, 0u) & 0xFFu);
    }
}

}  // namespace

#ifndef OPROJ_Q_WAVES_PER_CU
#define OPROJ_Q_WAVES_PER_CU 12
#endif

hipError_t launch_inv_rope_quant(const RopeQuantArgs& a, hipStream_t stream) {
    const int cus = current_device_info().cus;
    int ch = rq::heads_per_item(a.hpg);  // 1, 2 or 4
    // small batches: two-head items when that still gives every item its own
    // wave within the occupancy limit (32 waves per CU) -- the kernel is then
    // latency-bound and more, smaller items finish sooner (measured)
    const bool small = ch == 4 && a.T * a.G * (a.hpg / 2) <= (int64_t)cus * 32;
    if (small) ch = 2;
    const RQParams p = rq::make_params(a, ch);
    // otherwise a fixed population of waves (OPROJ_Q_WAVES_PER_CU per CU of
    // the device) walks the items
    int64_t waves = (int64_t)cus * OPROJ_Q_WAVES_PER_CU;
    if (small || p.nitems < waves) waves = p.nitems;
    const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
    const dim3 block(kWaves * 64);
    const bool pipe = p.nitems > waves;  // else every wave takes exactly one item
    const bool f32 = a.o_f32 != nullptr;
#define OPROJ_RQ_LAUNCH(C)                                                                          \
    if (f32) {                                                                                      \
        if (pipe)                                                                                   \
            hipLaunchKernelGGL((inv_rope_quant_kernel<C, true, true>), grid, block, 0, stream, p);  \
        else                                                                                        \
            hipLaunchKernelGGL((inv_rope_quant_kernel<C, false, true>), grid, block, 0, stream, p); \
    } else {                                                                                        \
        if (pipe)                                                                                   \
            hipLaunchKernelGGL((inv_rope_quant_kernel<C, true, false>), grid, block, 0, stream, p); \
        else                                                                                        \
            hipLaunchKernelGGL((inv_rope_quant_kernel<C, false, false>), grid, block, 0, stream, p);\
    }
    switch (ch) {
        case 1: OPROJ_RQ_LAUNCH(1) break;
        case 2: OPROJ_RQ_LAUNCH(2) break;
        default: OPROJ_RQ_LAUNCH(4) break;
    }
#undef OPROJ_RQ_LAUNCH
    return hipGetLastError();
}

hipError_t launch_quantize_weight(const WeightQuantArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.rows + a.brows - 1) / a.brows), (unsigned)(a.K / 128));
    hipLaunchKernelGGL(quantize_weight_kernel, grid, dim3(kWqThreads), 0, stream, a.w, a.codes,
                       a.scales, a.rows, a.K, a.brows, a.pow2 | a.e8m0, a.e8m0);
    return hipGetLastError();
}

}  // namespace oproj
