// rq_item.hpp -- one work item of the fused inverse-RoPE + 1x128 FP8
// quantisation on gfx950 (vLLM API page
// "vllm.models.deepseek_v4.common.ops.fused_inv_rope_fp8_quant"): a wave
// loads CH head rows of one token and group, rotates the RoPE dims, forms the
// block scales and writes the FP8 codes and scales.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace oproj {
namespace rq {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct Params {
    const uint16_t* o;   // bf16 input rows
    const float* of;     // or fp32 input rows (the attention-epilogue producer)
    const int64_t* pos;
    const float* table;
    uint8_t* codes;
    void* scales;  // fp32 per block, or packed UE8M0 words (one per head)
    int64_t T, H, hpg, max_pos, nitems;
    int64_t st, sg, sst, ssg, sskb;
    int nchunk, pow2, e8m0;
};

// Heads per item for a group of hpg heads: 4 (4 KiB of input per wave) when
// the group size allows, else the whole group (1 or 2 heads).
inline int heads_per_item(int64_t hpg) { return (hpg % 4 == 0) ? 4 : (int)hpg; }

inline Params make_params(const RopeQuantArgs& a, int ch) {
    Params p;
    p.o = a.o;
    p.of = a.o_f32;
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
    p.pow2 = a.pow2 | a.e8m0;
    p.e8m0 = a.e8m0;
    return p;
}

// The CH head rows of one item as loaded: one 16-byte piece per head and
// lane for bf16 input, two for fp32 input (lane l: elements 8l..8l+7).
template <int CH, bool F32>
struct Rows;
template <int CH>
struct Rows<CH, false> {
    uint4 r[CH];
    __device__ __forceinline__ void unpack(float (&v)[CH][8]) const {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const uint32_t w4[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                v[j][2 * m] = bf16_lo(w4[m]);
                v[j][2 * m + 1] = bf16_hi(w4[m]);
            }
        }
    }
};
template <int CH>
struct Rows<CH, true> {
    u32x4 r[CH][2];
    // Loaded contiguously (half the memory requests of two 16-byte pieces per
    // lane 32 bytes apart): r[j][0] holds floats 4l..4l+3 of head j, r[j][1]
    // floats 256+4l..256+4l+3; lane l's elements 8l..8l+7 sit in lanes 2l and
    // 2l+1 (mod 64), in the first load for l < 32 and the second above
    __device__ __forceinline__ void unpack(float (&v)[CH][8]) const {
        const int l = __lane_id();
        const int sa = (2 * l) & 63, sb = (2 * l + 1) & 63;
        const bool up = l >= 32;
#pragma unroll
        for (int j = 0; j < CH; ++j)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t a0 = __shfl(r[j][0][k], sa), a1 = __shfl(r[j][1][k], sa);
                const uint32_t b0 = __shfl(r[j][0][k], sb), b1 = __shfl(r[j][1][k], sb);
                v[j][k] = __uint_as_float(up ? a1 : a0);
                v[j][4 + k] = __uint_as_float(up ? b1 : b0);
            }
    }
};

// Items are numbered in address order: head chunk fastest, then group, then
// token.  Lane l holds elements 8l..8l+7 of every head of the chunk, so the
// 16-lane row c covers quantisation block c and lanes 56..63 the RoPE dims.
template <int CH, bool F32 = false>
struct Wave {
    using RowsT = Rows<CH, F32>;
    const Params& p;
    const int lane, c, li;
    const int64_t G;

    __device__ __forceinline__ Wave(const Params& p_, int lane_)
        : p(p_), lane(lane_), c(lane_ >> 4), li(lane_ & 15), G(p_.H / p_.hpg) {}

    // item -> (token, group, chunk); items past the end load the last item
    // (kept in bounds) and are never stored
    __device__ __forceinline__ void split(int64_t item, int64_t& t, int64_t& g, int64_t& chunk) const {
        item = item < p.nitems ? item : p.nitems - 1;
        chunk = item % p.nchunk;
        const int64_t rest = item / p.nchunk;
        g = rest % G;
        t = rest / G;
    }
    // the CH head rows, non-temporal 16-byte loads (bf16: one per head and
    // lane, elements 8l..8l+7; fp32: two per head and lane, each instruction
    // reading 1 KiB of the row contiguously, rearranged by unpack())
    __device__ __forceinline__ void load_rows(int64_t t, int64_t g, int64_t chunk, RowsT& raw) const {
        const int64_t row0 = (t * p.H + g * p.hpg + chunk * CH) * 512;
        if constexpr (F32) {
            const float* src = p.of + row0 + 4 * lane;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                raw.r[j][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)j * 512));
                raw.r[j][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)j * 512 + 256));
            }
        } else {
            const uint16_t* src = p.o + row0 + 8 * lane;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (int64_t)j * 512));
                raw.r[j] = make_uint4(x.x, x.y, x.z, x.w);
            }
        }
    }
    // cos/sin of the lane's 4 pairs (identity for other lanes and bad positions)
    __device__ __forceinline__ void load_table(int64_t ps, float4& cs, float4& sn) const {
        const bool bad = (ps < 0) | (ps >= p.max_pos);
        cs = make_float4(1.f, 1.f, 1.f, 1.f);
        sn = make_float4(0.f, 0.f, 0.f, 0.f);
        if (lane >= 56 && !bad) {
            const float* row = p.table + ps * 64 + 4 * (lane - 56);
            cs = *reinterpret_cast<const float4*>(row);
            sn = *reinterpret_cast<const float4*>(row + 32);
        }
    }
    // rotate, reduce, scale, convert and store one item; SYS stores with
    // system-scope coherence (written through to memory, for readers in other
    // workgroups of the same launch), else non-temporal codes
    template <bool SYS = false>
    __device__ __forceinline__ void process(int64_t t, int64_t g, int64_t chunk, int64_t ps, const RowsT& raw,
                                            float4 cs, float4 sn) const {
        const bool bad = (ps < 0) | (ps >= p.max_pos);

        // ---- unpack, rotate the RoPE lanes, per-lane |v| max
        float v[CH][8];
        float am[CH];
        raw.unpack(v);
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

        if (p.e8m0) {
            // UE8M0 byte of block (head li, block c) is the exponent field of
            // the power-of-two scale (0xFF for NaN); lane li of row 0 packs
            // the head's four bytes into one word, block c in byte c
            const uint32_t e = bad ? 0xFFu : ((__float_as_uint(s) >> 23) & 0xFFu);
            const uint32_t e1 = __shfl(e, (lane + 16) & 63), e2 = __shfl(e, (lane + 32) & 63),
                           e3 = __shfl(e, (lane + 48) & 63);
            if (c == 0 && li < CH) {
                const int64_t hw = chunk * CH + li;  // head within the group = word index
                uint32_t* dst = static_cast<uint32_t*>(p.scales) + t * p.sst + g * p.ssg + hw * p.sskb;
                const uint32_t word = e | (e1 << 8) | (e2 << 16) | (e3 << 24);
                if constexpr (SYS)
                    __hip_atomic_store(dst, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                else
                    *dst = word;
            }
        } else if (li < CH) {
            const int64_t kb = (chunk * CH + li) * 4 + c;
            float* dst = static_cast<float*>(p.scales) + t * p.sst + g * p.ssg + kb * p.sskb;
            if constexpr (SYS)
                __hip_atomic_store(dst, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            else
                *dst = s;
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
            u32x2 x;
            x.x = w0;
            x.y = w1;
            if constexpr (SYS)
                __hip_atomic_store(reinterpret_cast<uint64_t*>(dst + (int64_t)j * 512),
                                   (uint64_t)w0 | ((uint64_t)w1 << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            else
                __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(dst + (int64_t)j * 512));
        }
    }
};

}  // namespace rq
}  // namespace oproj
