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
// The kernel is HBM-bound: read 1 KiB + write 512 B per head row.
#include "device_common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace oproj {

namespace {

constexpr int kWaves = 4;  // waves per workgroup

struct RQParams {
    const uint16_t* o;
    const int64_t* pos;
    const float* table;
    uint8_t* codes;
    float* scales;
    int64_t T, H, hpg, max_pos, nitems;
    int64_t st, sg, sst, ssg, sskb;
    int nchunk, ipw, pow2;
};

template <int CH>
__global__ __launch_bounds__(kWaves * 64) void inv_rope_quant_kernel(RQParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane >> 4;  // quantisation block within the head
    const int li = lane & 15;
    const int64_t base = (int64_t)blockIdx.x * (kWaves * p.ipw);

    for (int k = 0; k < p.ipw; ++k) {
        const int64_t item = base + (int64_t)k * kWaves + wave;
        if (item >= p.nitems) break;  // wave-uniform
        const int64_t t = item % p.T;
        const int64_t rest = item / p.T;
        const int64_t chunk = rest % p.nchunk;
        const int64_t g = rest / p.nchunk;
        const int64_t head0 = g * p.hpg + chunk * CH;

        // ---- loads: CH head rows of 1 KiB, 16 bytes per lane each
        const uint16_t* src = p.o + (t * p.H + head0) * 512 + 8 * lane;
        uint4 raw[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) raw[j] = *reinterpret_cast<const uint4*>(src + (int64_t)j * 512);

        const int64_t ps = p.pos[t];
        const bool bad = (ps < 0) | (ps >= p.max_pos);
        float4 cs = make_float4(1.f, 1.f, 1.f, 1.f), sn = make_float4(0.f, 0.f, 0.f, 0.f);
        if (lane >= 56 && !bad) {
            const float* row = p.table + ps * 64 + 4 * (lane - 56);
            cs = *reinterpret_cast<const float4*>(row);
            sn = *reinterpret_cast<const float4*>(row + 32);
        }

        // ---- unpack, rotate the RoPE lanes, per-lane |v| max
        float v[CH][8];
        float am[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const uint32_t w4[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                v[j][2 * m] = bf16_lo(w4[m]);
                v[j][2 * m + 1] = bf16_hi(w4[m]);
            }
        }
        if (lane >= 56) {
            const float cc[4] = {cs.x, cs.y, cs.z, cs.w};
            const float ss[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
            for (int j = 0; j < CH; ++j) {
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float e = v[j][2 * m], d = v[j][2 * m + 1];
                    v[j][2 * m] = __builtin_fmaf(d, ss[m], e * cc[m]);
                    v[j][2 * m + 1] = __builtin_fmaf(-e, ss[m], d * cc[m]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            float a = fabsf(v[j][0]);
#pragma unroll
            for (int m = 1; m < 8; ++m) a = fmaxf(a, fabsf(v[j][m]));
            am[j] = row16_max(a);
        }

        // ---- one scale per (head j, block c), computed by lane 16c + j
        float asel = am[0];
#pragma unroll
        for (int j = 1; j < CH; ++j) asel = ((li % CH) == j) ? am[j] : asel;
        float s = fmaxf(asel, kAmaxFloor) / kFp8Max;
        if (p.pow2) s = pow2_ceil(s);
        if (bad) s = __builtin_nanf("");
        const float r = 1.0f / s;

        if (li < CH) {
            const int64_t kb = (chunk * CH + li) * 4 + c;
            p.scales[t * p.sst + g * p.ssg + kb * p.sskb] = s;
        }

        uint8_t* dst = p.codes + t * p.st + g * p.sg + chunk * CH * 512 + 8 * lane;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const float sj = __shfl(s, (lane & ~15) + j);
            const float rj = __shfl(r, (lane & ~15) + j);
            float q[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) q[m] = div_by_scale(v[j][m], sj, rj);
            uint32_t w0 = cvt2_fp8<false>(q[0], q[1], 0u);
            w0 = cvt2_fp8<true>(q[2], q[3], w0);
            uint32_t w1 = cvt2_fp8<false>(q[4], q[5], 0u);
            w1 = cvt2_fp8<true>(q[6], q[7], w1);
            *reinterpret_cast<uint2*>(dst + (int64_t)j * 512) = make_uint2(w0, w1);
        }
    }
}

// ---------------------------------------------------------------------------
// Offline weight quantisation: one workgroup per (row block, 128-column block).
constexpr int kWqThreads = 256;

__global__ __launch_bounds__(kWqThreads) void quantize_weight_kernel(const float* __restrict__ w,
                                                                    uint8_t* __restrict__ codes,
                                                                    float* __restrict__ scales,
                                                                    int64_t rows, int64_t K,
                                                                    int64_t brows, int pow2) {
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
    if (threadIdx.x == 0) scales[rb * (K / 128) + kb] = s;
    for (int64_t i = threadIdx.x; i < n; i += kWqThreads) {
        const int64_t rr = r0 + i / 128, k = kb * 128 + (i % 128);
        const float q = div_by_scale(w[rr * K + k], s, r);
        codes[rr * K + k] = (uint8_t)(cvt2_fp8<false>(q, 0.f, 0u) & 0xFFu);
    }
}

}  // namespace

hipError_t launch_inv_rope_quant(const RopeQuantArgs& a, hipStream_t stream) {
    const int ch = (a.hpg % 8 == 0) ? 8 : (int)a.hpg;  // 1, 2, 4 or 8
    RQParams p;
    p.o = a.o;
    p.pos = a.positions;
    p.table = a.cos_sin;
    p.codes = a.codes;
    p.scales = a.scales;
    p.T = a.T;
    p.H = a.G * a.hpg;
    p.hpg = a.hpg;
    p.max_pos = a.max_pos;
    p.nchunk = (int)(a.hpg / ch);
    p.nitems = a.T * a.G * p.nchunk;
    p.st = a.lay.stride_t;
    p.sg = a.lay.stride_g;
    p.sst = a.lay.s_stride_t;
    p.ssg = a.lay.s_stride_g;
    p.sskb = a.lay.s_stride_kb;
    p.pow2 = a.pow2;
    // items per wave: enough workgroups to fill 256 CUs several times over
    int64_t ipw = p.nitems / (256 * 8 * kWaves);
    ipw = ipw < 1 ? 1 : (ipw > 16 ? 16 : ipw);
    p.ipw = (int)ipw;
    const int64_t per_block = kWaves * ipw;
    const dim3 grid((unsigned)((p.nitems + per_block - 1) / per_block));
    const dim3 block(kWaves * 64);
    switch (ch) {
        case 1: hipLaunchKernelGGL(inv_rope_quant_kernel<1>, grid, block, 0, stream, p); break;
        case 2: hipLaunchKernelGGL(inv_rope_quant_kernel<2>, grid, block, 0, stream, p); break;
        case 4: hipLaunchKernelGGL(inv_rope_quant_kernel<4>, grid, block, 0, stream, p); break;
        default: hipLaunchKernelGGL(inv_rope_quant_kernel<8>, grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_weight(const WeightQuantArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((a.rows + a.brows - 1) / a.brows), (unsigned)(a.K / 128));
    hipLaunchKernelGGL(quantize_weight_kernel, grid, dim3(kWqThreads), 0, stream, a.w, a.codes,
                       a.scales, a.rows, a.K, a.brows, a.pow2);
    return hipGetLastError();
}

}  // namespace oproj
