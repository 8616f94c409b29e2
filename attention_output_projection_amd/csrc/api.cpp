// api.cpp -- the C ABI declared in include/oproj.h: host-side validation and
// dispatch to the gfx950 kernels.  Nothing here allocates or synchronises.
#include "oproj.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "kernels.hpp"

namespace oproj {

DeviceInfo current_device_info() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];  // (cus << 8) | xcds, 0 until queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < kMaxDevices ? dev : kMaxDevices - 1;
    int v = dev < kMaxDevices ? cached[slot].load(std::memory_order_relaxed) : 0;
    if (v == 0) {
        int cus = 0, xcds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1 ||
            xcds > 255)
            xcds = 1;
        v = (cus << 8) | xcds;
        if (dev < kMaxDevices) cached[slot].store(v, std::memory_order_relaxed);
    }
    return DeviceInfo{v >> 8, v & 0xFF};
}

}  // namespace oproj

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Size checks of non-negative values that cannot overflow: products and sums
// saturate at INT64_MAX, which every limit below rejects.
int64_t mul_sat(int64_t a, int64_t b) {
    if (a <= 0 || b <= 0) return 0;
    return a > INT64_MAX / b ? INT64_MAX : a * b;
}
int64_t add_sat(int64_t a, int64_t b) { return a > INT64_MAX - b ? INT64_MAX : a + b; }

constexpr int64_t kLim32 = int64_t(1) << 32;  // the kernels' 32-bit lane offsets
constexpr int64_t kLimMem = int64_t(1) << 47;  // larger than any device allocation

// Head geometry and shape checks shared by every entry point.  Mirrors the
// preconditions fused_inv_rope_fp8_quant asserts (vLLM API page
// "vllm.models.deepseek_v4.common.ops.fused_inv_rope_fp8_quant"): H = G*hpg,
// head_dim = nope + rope, head_dim % block == 0, nope % block == block - rope,
// rope even; the fixed geometry of this library is 448 + 64 with blocks of 128.
oproj_status check_shape(const oproj_shape* s, bool need_rank) {
    if (!s) return OPROJ_E_NULL;
    if (s->T < 0 || s->n_groups < 1 || s->heads_per_group < 1 || s->max_pos < 1)
        return OPROJ_E_SHAPE;
    if (s->nope_dim < 0 || s->rope_dim < 0 || s->quant_block < 1) return OPROJ_E_SHAPE;
    const int64_t hd = s->nope_dim + s->rope_dim;
    if (hd % s->quant_block != 0) return OPROJ_E_SHAPE;
    if (s->nope_dim % s->quant_block != s->quant_block - s->rope_dim) return OPROJ_E_SHAPE;
    if (s->rope_dim % 2 != 0) return OPROJ_E_SHAPE;
    if (s->nope_dim != 448 || s->rope_dim != 64 || s->quant_block != 128) return OPROJ_E_MODE;
    const int64_t hpg = s->heads_per_group;
    if (!(hpg == 1 || hpg == 2 || hpg == 4 || hpg % 8 == 0)) return OPROJ_E_MODE;
    if (s->T > (int64_t(1) << 31) || s->n_groups > 65536 || hpg > 65536 || s->n_groups * hpg > 65536)
        return OPROJ_E_SHAPE;
    if (need_rank) {
        if (s->o_lora_rank < 64 || s->o_lora_rank % 64 != 0 || s->o_lora_rank > 65536) return OPROJ_E_SHAPE;
        // z [T][G][R] in bf16 must be addressable
        if (mul_sat(mul_sat(mul_sat(s->T, s->n_groups), s->o_lora_rank), 2) > kLimMem) return OPROJ_E_SHAPE;
    }
    return OPROJ_OK;
}

bool valid_mode(int32_t m) {
    return m == OPROJ_SCALE_FP32 || m == OPROJ_SCALE_POW2 || m == OPROJ_SCALE_E8M0;
}

// weight block mode valid with this scale mode (UE8M0 words need power-of-two scales)
bool valid_wblock(int32_t b, int32_t mode) {
    if (b == OPROJ_WBLOCK_128x128 || b == OPROJ_WBLOCK_1x128) return true;
    return b == OPROJ_WBLOCK_1x128_UE8M0 && mode != OPROJ_SCALE_FP32;
}

// default layout; in UE8M0 mode a scale word covers four K-blocks
oproj::ActLayout default_layout(const oproj_shape* s, int32_t mode) {
    const int64_t D = s->heads_per_group * 512, KB = D / 128 / (mode == OPROJ_SCALE_E8M0 ? 4 : 1);
    oproj::ActLayout l;
    l.stride_t = D;
    l.stride_g = s->T * D;
    l.s_stride_t = 1;
    l.s_stride_kb = s->T;
    l.s_stride_g = KB * s->T;
    return l;
}

oproj_status check_layout(const oproj_act_layout* l) {
    if (!l) return OPROJ_OK;
    if (l->stride_t < 0 || l->stride_g < 0 || l->s_stride_t < 0 || l->s_stride_g < 0 ||
        l->s_stride_kb < 0)
        return OPROJ_E_SHAPE;
    if (l->stride_t > kLimMem || l->stride_g > kLimMem || l->s_stride_t > kLimMem || l->s_stride_g > kLimMem ||
        l->s_stride_kb > kLimMem)
        return OPROJ_E_SHAPE;
    if (l->stride_t % 16 != 0 || l->stride_g % 16 != 0) return OPROJ_E_ALIGN;
    return OPROJ_OK;
}

oproj::ActLayout to_layout(const oproj_act_layout* l, const oproj_shape* s, int32_t mode) {
    if (!l) return default_layout(s, mode);
    oproj::ActLayout o;
    o.stride_t = l->stride_t;
    o.stride_g = l->stride_g;
    o.s_stride_t = l->s_stride_t;
    o.s_stride_g = l->s_stride_g;
    o.s_stride_kb = l->s_stride_kb;
    return o;
}

oproj_status from_hip(hipError_t e) { return e == hipSuccess ? OPROJ_OK : OPROJ_E_HIP; }

size_t round_up(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

extern "C" {

const char* oproj_status_string(oproj_status s) {
    switch (s) {
        case OPROJ_OK: return "ok";
        case OPROJ_E_NULL: return "null pointer";
        case OPROJ_E_SHAPE: return "invalid shape";
        case OPROJ_E_ALIGN: return "misaligned pointer or stride";
        case OPROJ_E_MODE: return "unsupported mode or head geometry";
        case OPROJ_E_HIP: return "HIP launch error";
        case OPROJ_E_SCRATCH: return "larger than the no-allocation scratch array";
    }
    return "unknown status";
}

const char* oproj_version(void) { return "0.1.0"; }

namespace {

// Validation + argument set-up of step a1+a2 (shared by the entry points).
oproj_status prep_quant(const oproj_shape* shape, int32_t scale_mode, const void* o, const int64_t* positions,
                        const float* cos_sin, void* a_codes, void* a_scales, const oproj_act_layout* out_layout,
                        oproj::RopeQuantArgs* a) {
    oproj_status st = check_shape(shape, false);
    if (st != OPROJ_OK) return st;
    if (!valid_mode(scale_mode)) return OPROJ_E_MODE;
    if ((st = check_layout(out_layout)) != OPROJ_OK) return st;
    if (shape->T == 0) return OPROJ_OK;
    if (!o || !positions || !cos_sin || !a_codes || !a_scales) return OPROJ_E_NULL;
    if (!aligned16(o) || !aligned16(cos_sin) || !aligned16(a_codes) ||
        (reinterpret_cast<uintptr_t>(positions) & 7u) || (reinterpret_cast<uintptr_t>(a_scales) & 3u))
        return OPROJ_E_ALIGN;
    a->T = shape->T;
    a->G = shape->n_groups;
    a->hpg = shape->heads_per_group;
    a->max_pos = shape->max_pos;
    a->pow2 = scale_mode != OPROJ_SCALE_FP32;
    a->e8m0 = scale_mode == OPROJ_SCALE_E8M0;
    a->o = static_cast<const uint16_t*>(o);
    a->o_f32 = nullptr;
    a->positions = positions;
    a->cos_sin = cos_sin;
    a->codes = static_cast<uint8_t*>(a_codes);
    a->scales = a_scales;
    a->lay = to_layout(out_layout, shape, scale_mode);
    return OPROJ_OK;
}

// Validation + argument set-up of step a3 (shared by the entry points).
oproj_status prep_gemm(const oproj_shape* shape, int32_t scale_mode, const void* a_codes, const void* a_scales,
                       const oproj_act_layout* a_layout, const void* w_codes, const void* w_scales,
                       int32_t w_block, void* z, oproj::GroupedGemmArgs* a) {
    oproj_status st = check_shape(shape, true);
    if (st != OPROJ_OK) return st;
    if (!valid_mode(scale_mode)) return OPROJ_E_MODE;
    if (!valid_wblock(w_block, scale_mode)) return OPROJ_E_MODE;
    if ((st = check_layout(a_layout)) != OPROJ_OK) return st;
    if (shape->T == 0) return OPROJ_OK;
    if (!a_codes || !a_scales || !w_codes || !w_scales || !z) return OPROJ_E_NULL;
    if (!aligned16(a_codes) || !aligned16(w_codes) || !aligned16(z) ||
        (reinterpret_cast<uintptr_t>(a_scales) & 3u) || (reinterpret_cast<uintptr_t>(w_scales) & 3u))
        return OPROJ_E_ALIGN;
    {
        // the kernels address operands as a uniform base plus 32-bit lane offsets
        const oproj::ActLayout l = to_layout(a_layout, shape, scale_mode);
        const int64_t D = shape->heads_per_group * 512, KB = D / 128, lim = kLim32;
        const int64_t rows = shape->n_groups * shape->o_lora_rank, T1 = shape->T - 1, G1 = shape->n_groups - 1;
        if (add_sat(mul_sat(T1, l.stride_t), D) >= lim || add_sat(mul_sat(mul_sat(T1, l.s_stride_t), 4), 4) >= lim ||
            rows * D >= lim || rows * KB * 4 >= lim)
            return OPROJ_E_SHAPE;
        // each group's operand base (64-bit) stays inside an addressable range
        if (mul_sat(G1, l.stride_g) >= kLimMem || add_sat(mul_sat(G1, l.s_stride_g), mul_sat(KB, l.s_stride_kb)) >=
                                                        kLimMem)
            return OPROJ_E_SHAPE;
    }
    a->T = shape->T;
    a->G = shape->n_groups;
    a->D = shape->heads_per_group * 512;
    a->R = shape->o_lora_rank;
    a->mx = scale_mode != OPROJ_SCALE_FP32;
    a->a_e8m0 = scale_mode == OPROJ_SCALE_E8M0;
    a->w_1x128 = w_block != OPROJ_WBLOCK_128x128;
    a->w_e8m0 = w_block == OPROJ_WBLOCK_1x128_UE8M0;
    a->a = static_cast<const uint8_t*>(a_codes);
    a->sa = a_scales;
    a->lay = to_layout(a_layout, shape, scale_mode);
    a->w = static_cast<const uint8_t*>(w_codes);
    a->sw = w_scales;
    a->z = static_cast<uint16_t*>(z);
    return OPROJ_OK;
}

// Validation and workspace layout shared by the FP8 whole-path entry points:
// the codes, then the scales, then (when hidden > 0) z, each region 256-byte
// aligned; a3 writes z there or, without wo_b, straight to out.
oproj_status prep_fused(const oproj_shape* shape, int32_t scale_mode, const void* o, const int64_t* positions,
                        const float* cos_sin, const void* w_codes, const void* w_scales, int32_t w_block,
                        int64_t hidden, void* workspace, size_t workspace_bytes, void* out,
                        oproj::RopeQuantArgs* qa, oproj::GroupedGemmArgs* ga, void** zbuf) {
    if (!o || !positions || !cos_sin || !w_codes || !w_scales || !workspace || !out) return OPROJ_E_NULL;
    if (workspace_bytes < oproj_fused_workspace_bytes(shape, hidden)) return OPROJ_E_SHAPE;
    if (!aligned16(workspace)) return OPROJ_E_ALIGN;
    const size_t T = (size_t)shape->T, G = (size_t)shape->n_groups;
    const size_t D = (size_t)shape->heads_per_group * 512, KB = D / 128;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    void* codes = ws;
    float* scales = reinterpret_cast<float*>(ws + round_up(T * G * D));
    *zbuf = hidden > 0 ? (void*)(ws + round_up(T * G * D) + round_up(T * G * KB * sizeof(float))) : out;
    oproj_status st = prep_quant(shape, scale_mode, o, positions, cos_sin, codes, scales, nullptr, qa);
    if (st != OPROJ_OK) return st;
    return prep_gemm(shape, scale_mode, codes, scales, nullptr, w_codes, w_scales, w_block, *zbuf, ga);
}

}  // namespace

oproj_status oproj_inv_rope_quant(const oproj_shape* shape, int32_t scale_mode, const void* o,
                                  const int64_t* positions, const float* cos_sin, void* a_codes,
                                  void* a_scales, const oproj_act_layout* out_layout,
                                  void* stream) {
    oproj::RopeQuantArgs a;
    const oproj_status st = prep_quant(shape, scale_mode, o, positions, cos_sin, a_codes, a_scales, out_layout, &a);
    if (st != OPROJ_OK || shape->T == 0) return st;
    return from_hip(oproj::launch_inv_rope_quant(a, static_cast<hipStream_t>(stream)));
}

oproj_status oproj_inv_rope_quant_f32(const oproj_shape* shape, int32_t scale_mode, const float* o,
                                     const int64_t* positions, const float* cos_sin, void* a_codes,
                                     void* a_scales, const oproj_act_layout* out_layout, void* stream) {
    oproj::RopeQuantArgs a;
    const oproj_status st = prep_quant(shape, scale_mode, o, positions, cos_sin, a_codes, a_scales, out_layout, &a);
    if (st != OPROJ_OK || shape->T == 0) return st;
    a.o = nullptr;
    a.o_f32 = o;
    return from_hip(oproj::launch_inv_rope_quant(a, static_cast<hipStream_t>(stream)));
}

oproj_status oproj_grouped_wo_a(const oproj_shape* shape, int32_t scale_mode, const void* a_codes,
                                const void* a_scales, const oproj_act_layout* a_layout,
                                const void* w_codes, const void* w_scales, int32_t w_block,
                                void* z, void* stream) {
    oproj::GroupedGemmArgs a;
    const oproj_status st =
        prep_gemm(shape, scale_mode, a_codes, a_scales, a_layout, w_codes, w_scales, w_block, z, &a);
    if (st != OPROJ_OK || shape->T == 0) return st;
    return from_hip(oproj::launch_grouped_gemm(a, static_cast<hipStream_t>(stream)));
}

oproj_status oproj_dense_bf16_gemm(int64_t M, int64_t N, int64_t K, const void* x, const void* w,
                                   void* y, void* stream) {
    if (M < 0 || N < 1 || K < 64 || K % 64 != 0 || N % 16 != 0) return OPROJ_E_SHAPE;
    // the kernel addresses each operand as a uniform base plus 32-bit lane offsets
    if (mul_sat(mul_sat(M, K), 2) > kLim32 || mul_sat(mul_sat(N, K), 2) > kLim32) return OPROJ_E_SHAPE;
    if (mul_sat(mul_sat(M, N), 2) > kLimMem) return OPROJ_E_SHAPE;
    if (M == 0) return OPROJ_OK;
    if (!x || !w || !y) return OPROJ_E_NULL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return OPROJ_E_ALIGN;
    oproj::DenseGemmArgs a;
    a.M = M;
    a.N = N;
    a.K = K;
    a.x = static_cast<const uint16_t*>(x);
    a.w = static_cast<const uint16_t*>(w);
    a.y = static_cast<uint16_t*>(y);
    return from_hip(oproj::launch_dense_bf16_gemm(a, static_cast<hipStream_t>(stream)));
}

namespace {

// default and validated layout of a bf16 activation operand
oproj_status bf16_layout(const oproj_shape* s, const oproj_bf16_layout* l, int64_t* st, int64_t* sg) {
    const int64_t D = s->heads_per_group * 512;
    if (!l) {
        *st = s->n_groups * D;
        *sg = D;
        return OPROJ_OK;
    }
    if (l->stride_t < 0 || l->stride_g < 0 || l->stride_t > kLimMem || l->stride_g > kLimMem) return OPROJ_E_SHAPE;
    if (mul_sat(s->n_groups - 1, l->stride_g) >= kLimMem) return OPROJ_E_SHAPE;
    if (l->stride_t % 8 != 0 || l->stride_g % 8 != 0) return OPROJ_E_ALIGN;
    *st = l->stride_t;
    *sg = l->stride_g;
    return OPROJ_OK;
}

}  // namespace

oproj_status oproj_inv_rope_bf16(const oproj_shape* shape, const void* o, const int64_t* positions,
                                 const float* cos_sin, void* x, const oproj_bf16_layout* x_layout,
                                 void* stream) {
    oproj_status st = check_shape(shape, false);
    if (st != OPROJ_OK) return st;
    int64_t xst, xsg;
    if ((st = bf16_layout(shape, x_layout, &xst, &xsg)) != OPROJ_OK) return st;
    if (shape->T == 0) return OPROJ_OK;
    if (!o || !positions || !cos_sin || !x) return OPROJ_E_NULL;
    if (!aligned16(o) || !aligned16(cos_sin) || !aligned16(x) || (reinterpret_cast<uintptr_t>(positions) & 7u))
        return OPROJ_E_ALIGN;
    oproj::RopeBf16Args a;
    a.T = shape->T;
    a.G = shape->n_groups;
    a.hpg = shape->heads_per_group;
    a.max_pos = shape->max_pos;
    a.o = static_cast<const uint16_t*>(o);
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.x = static_cast<uint16_t*>(x);
    a.stride_t = xst;
    a.stride_g = xsg;
    return from_hip(oproj::launch_inv_rope_bf16(a, static_cast<hipStream_t>(stream)));
}

oproj_status oproj_grouped_wo_a_bf16(const oproj_shape* shape, const void* x,
                                     const oproj_bf16_layout* x_layout, const void* w, void* z,
                                     void* stream) {
    oproj_status st = check_shape(shape, true);
    if (st != OPROJ_OK) return st;
    int64_t xst, xsg;
    if ((st = bf16_layout(shape, x_layout, &xst, &xsg)) != OPROJ_OK) return st;
    if (shape->T == 0) return OPROJ_OK;
    if (!x || !w || !z) return OPROJ_E_NULL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(z)) return OPROJ_E_ALIGN;
    const int64_t D = shape->heads_per_group * 512, R = shape->o_lora_rank, G = shape->n_groups;
    // the kernel addresses a group's operands as a uniform base plus 32-bit lane offsets
    if (add_sat(mul_sat(mul_sat(shape->T - 1, xst), 2), D * 2) > kLim32 || R * D * 2 > kLim32) return OPROJ_E_SHAPE;
    oproj::Bf16GemmArgs a;
    a.G = G;
    a.M = shape->T;
    a.N = R;
    a.K = D;
    a.x = static_cast<const uint16_t*>(x);
    a.w = static_cast<const uint16_t*>(w);
    a.y = static_cast<uint16_t*>(z);
    a.sx = xst;
    a.gx = xsg;
    a.gw = R * D;
    a.sy = G * R;
    a.gy = R;
    return from_hip(oproj::launch_bf16_gemm(a, static_cast<hipStream_t>(stream)));
}

size_t oproj_fused_bf16_workspace_bytes(const oproj_shape* shape, int64_t hidden) {
    if (check_shape(shape, true) != OPROJ_OK) return 0;
    const size_t T = (size_t)shape->T, G = (size_t)shape->n_groups;
    const size_t D = (size_t)shape->heads_per_group * 512;
    size_t b = round_up(T * G * D * 2);
    if (hidden > 0) b += round_up(T * G * (size_t)shape->o_lora_rank * 2);
    return b;
}

oproj_status oproj_fused_bf16(const oproj_shape* shape, const void* o, const int64_t* positions,
                              const float* cos_sin, const void* w, const void* wo_b, int64_t hidden,
                              void* workspace, size_t workspace_bytes, void* out, void* stream) {
    oproj_status st = check_shape(shape, true);
    if (st != OPROJ_OK) return st;
    if (wo_b && (hidden < 16 || hidden % 16 != 0)) return OPROJ_E_SHAPE;
    if (shape->T == 0) return OPROJ_OK;
    if (!o || !positions || !cos_sin || !w || !workspace || !out) return OPROJ_E_NULL;
    if (workspace_bytes < oproj_fused_bf16_workspace_bytes(shape, wo_b ? hidden : 0)) return OPROJ_E_SHAPE;
    if (!aligned16(workspace) || !aligned16(o) || !aligned16(cos_sin) || !aligned16(w) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(positions) & 7u))
        return OPROJ_E_ALIGN;
    const int64_t T = shape->T, G = shape->n_groups, R = shape->o_lora_rank;
    const int64_t D = shape->heads_per_group * 512, lim = int64_t(1) << 32;
    // the GEMM kernels address each group's operands as a base plus 32-bit lane offsets
    if ((T - 1) * G * D * 2 + D * 2 > lim || R * D * 2 > lim) return OPROJ_E_SHAPE;
    if (wo_b) {
        const int64_t K = G * R;
        if (K % 64 != 0 || mul_sat(mul_sat(T, K), 2) > lim || mul_sat(mul_sat(hidden, K), 2) > lim ||
            mul_sat(mul_sat(T, hidden), 2) > kLimMem)
            return OPROJ_E_SHAPE;
        if (!aligned16(wo_b)) return OPROJ_E_ALIGN;
    }
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    void* x = ws;
    void* zbuf = wo_b ? (void*)(ws + round_up((size_t)(T * G * D * 2))) : out;
    if ((st = oproj_inv_rope_bf16(shape, o, positions, cos_sin, x, nullptr, stream)) != OPROJ_OK) return st;
    if ((st = oproj_grouped_wo_a_bf16(shape, x, nullptr, w, zbuf, stream)) != OPROJ_OK) return st;
    if (!wo_b) return OPROJ_OK;
    return oproj_dense_bf16_gemm(T, hidden, G * R, zbuf, wo_b, out, stream);
}

size_t oproj_fused_workspace_bytes(const oproj_shape* shape, int64_t hidden) {
    if (check_shape(shape, true) != OPROJ_OK) return 0;
    const size_t T = (size_t)shape->T, G = (size_t)shape->n_groups;
    const size_t D = (size_t)shape->heads_per_group * 512, KB = D / 128;
    size_t b = round_up(T * G * D) + round_up(T * G * KB * sizeof(float));
    if (hidden > 0) b += round_up(T * G * (size_t)shape->o_lora_rank * 2);
    return b;
}

oproj_status oproj_fused(const oproj_shape* shape, int32_t scale_mode, const void* o,
                         const int64_t* positions, const float* cos_sin, const void* w_codes,
                         const void* w_scales, int32_t w_block, const void* wo_b, int64_t hidden,
                         void* workspace, size_t workspace_bytes, void* out, void* stream) {
    oproj_status st = check_shape(shape, true);
    if (st != OPROJ_OK) return st;
    if (!valid_mode(scale_mode)) return OPROJ_E_MODE;
    if (!valid_wblock(w_block, scale_mode)) return OPROJ_E_MODE;
    if (wo_b && (hidden < 16 || hidden % 16 != 0)) return OPROJ_E_SHAPE;
    if (shape->T == 0) return OPROJ_OK;
    oproj::RopeQuantArgs qa;
    oproj::GroupedGemmArgs ga;
    void* zbuf = nullptr;
    if ((st = prep_fused(shape, scale_mode, o, positions, cos_sin, w_codes, w_scales, w_block, wo_b ? hidden : 0,
                         workspace, workspace_bytes, out, &qa, &ga, &zbuf)) != OPROJ_OK)
        return st;
    if (wo_b) {  // validate a4 before anything is enqueued
        const int64_t K = shape->n_groups * shape->o_lora_rank, lim = kLim32;
        if (K % 64 != 0 || mul_sat(mul_sat(shape->T, K), 2) > lim || mul_sat(mul_sat(hidden, K), 2) > lim ||
            mul_sat(mul_sat(shape->T, hidden), 2) > kLimMem)
            return OPROJ_E_SHAPE;
        if (!aligned16(wo_b)) return OPROJ_E_ALIGN;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = from_hip(oproj::launch_inv_rope_quant(qa, s))) != OPROJ_OK) return st;
    if ((st = from_hip(oproj::launch_grouped_gemm(ga, s))) != OPROJ_OK) return st;
    if (!wo_b) return OPROJ_OK;
    return oproj_dense_bf16_gemm(shape->T, hidden, shape->n_groups * shape->o_lora_rank, zbuf, wo_b,
                                 out, stream);
}

size_t oproj_fused_decode_workspace_bytes(const oproj_shape* shape) {
    const size_t b = oproj_fused_workspace_bytes(shape, 0);
    if (b == 0) return 0;
    return b + round_up((size_t)shape->n_groups * oproj::kFusedDecodeSyncBytesPerGroup);
}

oproj_status oproj_fused_decode(const oproj_shape* shape, int32_t scale_mode, const void* o,
                                const int64_t* positions, const float* cos_sin, const void* w_codes,
                                const void* w_scales, int32_t w_block, void* workspace,
                                size_t workspace_bytes, void* z, void* stream) {
    oproj_status st = check_shape(shape, true);
    if (st != OPROJ_OK) return st;
    if (!valid_mode(scale_mode)) return OPROJ_E_MODE;
    if (!valid_wblock(w_block, scale_mode)) return OPROJ_E_MODE;
    if (shape->T > 64 || shape->n_groups > 256) return OPROJ_E_SHAPE;
    if (shape->heads_per_group != 2 && shape->heads_per_group % 4 != 0) return OPROJ_E_MODE;
    if (shape->T == 0) return OPROJ_OK;
    if (workspace && workspace_bytes < oproj_fused_decode_workspace_bytes(shape)) return OPROJ_E_SHAPE;
    oproj::RopeQuantArgs qa;
    oproj::GroupedGemmArgs ga;
    void* zbuf = nullptr;
    if ((st = prep_fused(shape, scale_mode, o, positions, cos_sin, w_codes, w_scales, w_block, 0, workspace,
                         workspace_bytes, z, &qa, &ga, &zbuf)) != OPROJ_OK)
        return st;
    // the groups' barrier words follow the codes and scales
    uint64_t* sync = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) +
                                                 oproj_fused_workspace_bytes(shape, 0));
    bool launched = false;
    if ((st = from_hip(oproj::launch_fused_decode(qa, ga, sync, static_cast<hipStream_t>(stream), &launched))) !=
        OPROJ_OK)
        return st;
    return launched ? OPROJ_OK : OPROJ_E_SHAPE;
}

const char* oproj_fused_decode_unsupported(const oproj_shape* shape, int32_t scale_mode, int32_t w_block) {
    if (check_shape(shape, true) != OPROJ_OK) return "invalid shape";
    if (!valid_mode(scale_mode) || !valid_wblock(w_block, scale_mode))
        return "unsupported scale mode or weight block mode";
    if (shape->T == 0) return nullptr;  // the entry point returns at once
    return oproj::fused_decode_unfit(shape->T, shape->n_groups, shape->heads_per_group, shape->o_lora_rank);
}

oproj_status oproj_quantize_weight(int64_t rows, int64_t K, int32_t w_block, int32_t scale_mode,
                                   const float* w, void* codes, void* scales, void* stream) {
    if (rows < 0 || K < 128 || K % 128 != 0) return OPROJ_E_SHAPE;
    // grid: one workgroup per block (rows / block rows, K / 128 <= 65535)
    if (rows >= (int64_t(1) << 31) || K / 128 > 65535 || mul_sat(rows, K) > kLimMem) return OPROJ_E_SHAPE;
    if (!valid_mode(scale_mode) || !valid_wblock(w_block, scale_mode)) return OPROJ_E_MODE;
    if (w_block == OPROJ_WBLOCK_1x128_UE8M0 && K % 512 != 0) return OPROJ_E_SHAPE;
    if (rows == 0) return OPROJ_OK;
    if (!w || !codes || !scales) return OPROJ_E_NULL;
    if ((reinterpret_cast<uintptr_t>(w) & 3u) || (reinterpret_cast<uintptr_t>(scales) & 3u))
        return OPROJ_E_ALIGN;
    oproj::WeightQuantArgs a;
    a.rows = rows;
    a.K = K;
    a.brows = w_block == OPROJ_WBLOCK_128x128 ? 128 : 1;
    a.e8m0 = w_block == OPROJ_WBLOCK_1x128_UE8M0;
    a.pow2 = scale_mode != OPROJ_SCALE_FP32;  // weight scales stay fp32 powers of two in UE8M0 mode
    a.w = w;
    a.codes = static_cast<uint8_t*>(codes);
    a.scales = scales;
    return from_hip(oproj::launch_quantize_weight(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
