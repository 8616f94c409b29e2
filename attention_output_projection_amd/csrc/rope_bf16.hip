// rope_bf16.hip -- step a1 without quantisation on gfx950: the bf16
// inverse-rotated groups (vLLM API page
// "vllm.models.deepseek_v4.common.grouped_wo_a", grouped_input: the fused
// kernel called with quantize=False returns bf16 [num_tokens, n_groups,
// group_dim]; vLLM API page "vllm.models.deepseek_v4.nvidia.ops.o_proj",
// deep_gemm_fp8_o_proj: without FP8 the grouped product is a bf16 batched
// matmul over that tensor).
//
// x(t, g, (h % hpg)*512 + k) = o(t, h, k) for k < 448; the 64 RoPE dims of
// each head are rotated by -theta with the same fp32 operation order as the
// quantising kernel (e' = fma(d, s, e*c), d' = fma(-e, s, d*c)) and rounded
// to bf16, nearest even.  Work unit: one wave per two consecutive head rows;
// lane l moves elements 8l..8l+7 of each (16-byte non-temporal loads and
// stores), lanes 56..63 hold the RoPE dims and fetch cos[4(l-56)..+3],
// sin[..] of each row's token position.  Items are numbered in address order
// and dealt round-robin over a fixed population of waves (32 per CU, the
// occupancy limit: measured best), each of which loads its next item while
// it stores the current one.  HBM-bound: 1 KiB read + 1 KiB
// written per head row.  A position outside [0, max_pos) writes NaN into the
// token's RoPE dims.
#include "device_common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace oproj {

namespace {

typedef unsigned int rb_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRbWaves = 4;  // waves per workgroup

struct RBParams {
    const uint16_t* o;
    const int64_t* pos;
    const float* table;
    uint16_t* x;
    int64_t H, hpg, max_pos, nrows, nitems, st, sg;
};

#ifndef OPROJ_RB_ROWS
#define OPROJ_RB_ROWS 2
#endif
constexpr int kRbRows = OPROJ_RB_ROWS;  // head rows per work item

struct RbItem {
    rb_u32x4 raw[kRbRows];
    float4 cs[kRbRows], sn[kRbRows];
    bool bad[kRbRows];
};

// rows past the end load the last row (kept in bounds) and are never stored
__device__ __forceinline__ RbItem rb_load(const RBParams& p, int64_t item, int lane) {
    RbItem r;
#pragma unroll
    for (int j = 0; j < kRbRows; ++j) {
        int64_t row = item * kRbRows + j;
        row = row < p.nrows ? row : p.nrows - 1;
        r.raw[j] = __builtin_nontemporal_load(reinterpret_cast<const rb_u32x4*>(p.o + row * 512 + 8 * lane));
    }
#pragma unroll
    for (int j = 0; j < kRbRows; ++j) {
        int64_t row = item * kRbRows + j;
        row = row < p.nrows ? row : p.nrows - 1;
        const int64_t ps = p.pos[row / p.H];
        r.bad[j] = (ps < 0) | (ps >= p.max_pos);
        r.cs[j] = make_float4(1.f, 1.f, 1.f, 1.f);
        r.sn[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (lane >= 56 && !r.bad[j]) {
            const float* trow = p.table + ps * 64 + 4 * (lane - 56);
            r.cs[j] = *reinterpret_cast<const float4*>(trow);
            r.sn[j] = *reinterpret_cast<const float4*>(trow + 32);
        }
    }
    return r;
}

__device__ __forceinline__ void rb_store(const RBParams& p, int64_t item, int lane, const RbItem& r) {
#pragma unroll
    for (int j = 0; j < kRbRows; ++j) {
        const int64_t row = item * kRbRows + j;
        if (row >= p.nrows) break;
        rb_u32x4 out = r.raw[j];
        if (lane >= 56) {
            const uint32_t w4[4] = {r.raw[j].x, r.raw[j].y, r.raw[j].z, r.raw[j].w};
            const float cc[4] = {r.cs[j].x, r.cs[j].y, r.cs[j].z, r.cs[j].w};
            const float ss[4] = {r.sn[j].x, r.sn[j].y, r.sn[j].z, r.sn[j].w};
            uint32_t o4[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float e = bf16_lo(w4[m]), d = bf16_hi(w4[m]);
                const float e2 = __builtin_fmaf(d, ss[m], e * cc[m]);
                const float d2 = __builtin_fmaf(-e, ss[m], d * cc[m]);
                o4[m] = r.bad[j] ? 0x7FC07FC0u : (f32_to_bf16_bits(e2) | (f32_to_bf16_bits(d2) << 16));
            }
            out = rb_u32x4{o4[0], o4[1], o4[2], o4[3]};
        }
        const int64_t t = row / p.H, h = row % p.H, g = h / p.hpg;
        uint16_t* dst = p.x + t * p.st + g * p.sg + (h % p.hpg) * 512 + 8 * lane;
        __builtin_nontemporal_store(out, reinterpret_cast<rb_u32x4*>(dst));
    }
}

__global__ __launch_bounds__(kRbWaves * 64) void inv_rope_bf16_kernel(RBParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kRbWaves;
    const int64_t first = (int64_t)blockIdx.x * kRbWaves + wave;
    if (first >= p.nitems) return;
    RbItem next = rb_load(p, first, lane);
    for (int64_t item = first; item < p.nitems; item += nwaves) {
        const RbItem cur = next;
        if (item + nwaves < p.nitems) next = rb_load(p, item + nwaves, lane);
        rb_store(p, item, lane, cur);
    }
}

}  // namespace

#ifndef OPROJ_RB_WAVES_PER_CU
#define OPROJ_RB_WAVES_PER_CU 32
#endif

hipError_t launch_inv_rope_bf16(const RopeBf16Args& a, hipStream_t stream) {
    RBParams p;
    p.o = a.o;
    p.pos = a.positions;
    p.table = a.cos_sin;
    p.x = a.x;
    p.H = a.G * a.hpg;
    p.hpg = a.hpg;
    p.max_pos = a.max_pos;
    p.nrows = a.T * p.H;
    p.nitems = (p.nrows + kRbRows - 1) / kRbRows;
    p.st = a.stride_t;
    p.sg = a.stride_g;
    int64_t waves = (int64_t)current_device_info().cus * OPROJ_RB_WAVES_PER_CU;
    if (p.nitems < waves) waves = p.nitems;
    const dim3 grid((unsigned)((waves + kRbWaves - 1) / kRbWaves)), block(kRbWaves * 64);
    hipLaunchKernelGGL(inv_rope_bf16_kernel, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace oproj
