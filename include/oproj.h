/*
 * oproj.h -- C ABI of the MI355X (gfx950) O-projection front half:
 *   inverse RoPE -> 1x128 block FP8 e4m3fn quantisation -> grouped wo_a GEMM
 *   [-> dense wo_b GEMM] (as separate calls, in two launches, or in one launch
 *   for decode-sized batches), the same rotation and quantisation from fp32
 *   attention output (the attention-epilogue producer), and the unquantised
 *   variant (bf16 inverse RoPE -> grouped bf16 wo_a GEMM).
 *
 * Sources (web pages; cited by page title and section):
 *  [FUSED] vLLM API page "vllm.models.deepseek_v4.common.ops.fused_inv_rope_fp8_quant",
 *          fused_inv_rope_fp8_quant: parameters, returns and preconditions.
 *  [OPROJ] vLLM API page "vllm.models.deepseek_v4.nvidia.ops.o_proj":
 *          compute_fp8_einsum_recipe (scale recipes), deep_gemm_fp8_o_proj
 *          (the path; caller-allocated z; pre-quantised input with padding groups).
 *  [GWA]   vLLM API page "vllm.models.deepseek_v4.common.grouped_wo_a",
 *          DeepseekV4GroupedWoA (group g meets only rows g*R .. g*R+R-1).
 *  [SGL]   sglang source page "python/sglang/srt/models/deepseek_v4.py":
 *          MQALayer.forward (inverse RoPE, group view, FP8 einsum, wo_b),
 *          _dequant_fp8 (weight scales multiply), _setup_fp8_wo_a_scales.
 *
 * Conventions for every entry point
 *  - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *    never allocates device memory, never synchronises the host and never
 *    throws; all work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream) and completes asynchronously.
 *  - The return value reports argument validation and launch errors only.
 *    Validation runs on the host before anything is enqueued, so an error
 *    return means nothing was launched.
 *  - T == 0 is a valid no-op that returns OPROJ_OK (pointers are not checked).
 *  - Device pointers must be 16-byte aligned; strides are in elements.
 *  - Fixed in this library: head_dim 512 = nope_dim 448 + rope_dim 64,
 *    quantisation blocks of 128 ([FUSED] asserts head_dim % block == 0 and
 *    nope_dim % block == block - rope_dim; 448 % 128 == 64 satisfies it).
 *    Other values return OPROJ_E_MODE.
 *  - The FP8 format is OCP e4m3fn (max 448, no infinities).
 *  - Inputs must be finite.  A position outside [0, max_pos) does not fault:
 *    the affected token's scales are written as NaN (its codes are then
 *    meaningless) so the error is visible downstream.
 */
#ifndef OPROJ_H
#define OPROJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum oproj_status {
    OPROJ_OK = 0,
    OPROJ_E_NULL = 1,  /* a required pointer is NULL */
    OPROJ_E_SHAPE = 2, /* sizes inconsistent or outside the supported range */
    OPROJ_E_ALIGN = 3, /* a pointer or stride breaks the 16-byte rule */
    OPROJ_E_MODE = 4,  /* unsupported scale mode / head geometry */
    OPROJ_E_HIP = 5,   /* a HIP launch or device query failed */
    OPROJ_E_SCRATCH = 6 /* the call needs more than the library's scratch array holds */
} oproj_status;

/* Scale recipe ([OPROJ] compute_fp8_einsum_recipe names two):
 *  OPROJ_SCALE_FP32: activation scale = amax / 448 as fp32 (1x128 blocks).
 *  OPROJ_SCALE_POW2: that value rounded up to a power of two (E8M0-style),
 *                    still stored as fp32.
 *  OPROJ_SCALE_E8M0: the POW2 scales stored packed ([OPROJ]
 *                    rope_quant_attn_out: one int32 per head over its four
 *                    128-wide blocks): byte b of activation scale word j
 *                    (bits 8b..8b+7) is the UE8M0 byte of block 4j+b, i.e. the
 *                    biased exponent k+127 of the scale 2^k (0xFF = NaN).
 *                    Weight scales stay fp32 powers of two. */
typedef enum oproj_scale_mode {
    OPROJ_SCALE_FP32 = 0,
    OPROJ_SCALE_POW2 = 1,
    OPROJ_SCALE_E8M0 = 2
} oproj_scale_mode;

/* Weight scale blocks:
 *  OPROJ_WBLOCK_128x128: scale (i, kb) covers rows 128i..128i+127 of the flat
 *                        [G*R, D] weight and columns 128kb..128kb+127;
 *                        scales are fp32 [ceil(G*R/128), D/128] row-major.
 *  OPROJ_WBLOCK_1x128:   scale (r, kb) per row r; fp32 [G*R, D/128] row-major.
 *  OPROJ_WBLOCK_1x128_UE8M0: per-row power-of-two scales stored as packed
 *                        UE8M0 words [G*R][D/512] (row r's block kb is byte
 *                        kb % 4 of word kb / 4; [SGL] format_ue8m0 weight
 *                        scales); only with OPROJ_SCALE_POW2 / OPROJ_SCALE_E8M0.
 * The stored scale multiplies the decoded code ([SGL] _dequant_fp8). */
typedef enum oproj_wblock {
    OPROJ_WBLOCK_128x128 = 0,
    OPROJ_WBLOCK_1x128 = 1,
    OPROJ_WBLOCK_1x128_UE8M0 = 2
} oproj_wblock;

/* Shape of one call ([FUSED] parameter table; [OPROJ] deep_gemm_fp8_o_proj). */
typedef struct oproj_shape {
    int64_t T;               /* tokens (>= 0) */
    int64_t n_groups;        /* G: live wo_a groups (>= 1) */
    int64_t heads_per_group; /* hpg: 1, 2, 4 or a multiple of 8; H = G * hpg */
    int64_t nope_dim;        /* 448 */
    int64_t rope_dim;        /* 64 */
    int64_t quant_block;     /* 128 */
    int64_t o_lora_rank;     /* R: wo_a rows per group; multiple of 64 */
    int64_t max_pos;         /* rows of the cos||sin table (> 0) */
} oproj_shape;
/* Derived: head_dim = nope_dim + rope_dim (512), D = hpg * head_dim,
 * KB = D / quant_block. */

/* Layout of an FP8 activation operand (codes + scales), element strides.
 *  code  (t, g, k)  at codes [t*stride_t   + g*stride_g   + k]
 *  scale (t, g, kb) at scales[t*s_stride_t + g*s_stride_g + kb*s_stride_kb]
 * Passing NULL for a layout selects the default group-major layout
 *  codes  [G][T][D]   (stride_t = D, stride_g = T*D) -- the physical layout
 *                     [FUSED] returns ([T,G,D] viewed with strides (D, T*D, 1))
 *  scales [G][KB][T]  (s_stride_t = 1, s_stride_kb = T, s_stride_g = KB*T),
 *                     i.e. MN-major, tokens contiguous.
 * In OPROJ_SCALE_E8M0 mode a scale is a 4-byte word holding four blocks and
 * kb above counts words (kb < KB/4); the default is then [G][KB/4][T]
 * (s_stride_t = 1, s_stride_kb = T, s_stride_g = (KB/4)*T).
 * stride_t and stride_g must be multiples of 16. */
typedef struct oproj_act_layout {
    int64_t stride_t, stride_g;
    int64_t s_stride_t, s_stride_g, s_stride_kb;
} oproj_act_layout;

/* Steps a1 + a2 ([FUSED] fused_inv_rope_fp8_quant; [SGL] MQALayer.forward):
 * for every token t and head h, rotate the pairs (o[t,h,448+2i], o[t,h,449+2i])
 * by -theta(positions[t]) using c = cos_sin[p][i], s = cos_sin[p][32+i]:
 *     e' = fma(d, s, e*c),  d' = fma(-e, s, d*c)      (fp32)
 * keep dims 0..447, view head h as group h / hpg at offset (h % hpg)*512, and
 * quantise each 128-wide block of each (t, g) row from the fp32 values:
 *     amax = max(max|v|, 1e-10); s = amax / 448 (IEEE fp32; pow2: rounded up
 *     to a power of two); code = e4m3fn(v / s), nearest even.
 *  o          bf16 [T][H][512], contiguous
 *  positions  int64 [T]
 *  cos_sin    fp32 [max_pos][64]: cos[0..31] then sin[0..31]
 *  a_codes    FP8 codes, layout `out_layout` (NULL: default group-major)
 *  a_scales   fp32 scales (uint32 UE8M0 words in OPROJ_SCALE_E8M0 mode),
 *             layout `out_layout`
 * Codes and scales of groups the layout does not name are untouched. */
oproj_status oproj_inv_rope_quant(const oproj_shape* shape, int32_t scale_mode, const void* o,
                                  const int64_t* positions, const float* cos_sin, void* a_codes,
                                  void* a_scales, const oproj_act_layout* out_layout,
                                  void* stream);

/* The attention-epilogue producer: steps a1 + a2 from the attention output as
 * fp32 values, the form an attention kernel holds before rounding it to bf16
 * ([OPROJ] rope_quant_attn_out: the FP8 codes and packed UE8M0 scales a fused
 * attention epilogue writes instead of a bf16 output; [FUSED] for the steps).
 * The rotation and quantisation are those of oproj_inv_rope_quant, applied to
 * the fp32 values with no rounding to bf16 anywhere; for inputs that are bf16
 * values the results are bit-identical to oproj_inv_rope_quant's.  The same
 * per-wave work item is what an attention kernel's epilogue would run on its
 * accumulators; here it reads o from memory so that it can be used and
 * checked on its own.
 *  o          fp32 [T][H][512], contiguous, 16-byte aligned
 * Every other argument, layout, mode and error as for oproj_inv_rope_quant. */
oproj_status oproj_inv_rope_quant_f32(const oproj_shape* shape, int32_t scale_mode, const float* o,
                                      const int64_t* positions, const float* cos_sin, void* a_codes,
                                      void* a_scales, const oproj_act_layout* out_layout, void* stream);

/* Step a3 ([OPROJ] deep_gemm_fp8_o_proj's einsum "bhr,hdr->bhd"; [GWA]):
 *   z[t][g][n] = sum_k (decode(a[t,g,k]) * sa[t,g,k/128])
 *                      * (decode(w[g*R+n][k]) * sw(g*R+n, k/128))
 * with fp32 accumulation and one bf16 rounding (nearest even) at the end.
 *  a_codes/a_scales  activation operand in layout `a_layout` (NULL: default).
 *                    Only groups 0..G-1 are read, so a pre-quantised input
 *                    [T][Gp][D] with Gp > G padding groups is passed with
 *                    stride_t = Gp*D, stride_g = D ([OPROJ]: live groups first,
 *                    padding sliced off).
 *  w_codes   FP8 [G*R][D] row-major (K contiguous)
 *  w_scales  fp32 (or UE8M0 words), blocks per `w_block`
 *  scale_mode  OPROJ_SCALE_POW2 declares that BOTH activation and weight
 *              scales are powers of two (they are then applied by the matrix
 *              cores' block scaling); OPROJ_SCALE_E8M0 is the same with the
 *              activation scales as packed UE8M0 words; OPROJ_SCALE_FP32
 *              accepts any positive fp32 scales.
 *  z         bf16 [T][G][R] contiguous */
oproj_status oproj_grouped_wo_a(const oproj_shape* shape, int32_t scale_mode, const void* a_codes,
                                const void* a_scales, const oproj_act_layout* a_layout,
                                const void* w_codes, const void* w_scales, int32_t w_block,
                                void* z, void* stream);

/* Step a4 ([SGL] MQALayer.forward applies wo_b to z.flatten(1)):
 *   y[m][j] = sum_c x[m][c] * w[j][c], bf16 inputs, fp32 accumulation, bf16 out.
 *  x  bf16 [M][K] row-major;  w  bf16 [N][K] row-major;  y  bf16 [M][N].
 *  K must be a multiple of 64 and N a multiple of 16; each operand must span
 *  at most 4 GiB (M*K*2 and N*K*2 bytes), else OPROJ_E_SHAPE. */
oproj_status oproj_dense_bf16_gemm(int64_t M, int64_t N, int64_t K, const void* x, const void* w,
                                   void* y, void* stream);

/* Layout of a bf16 activation operand of the unquantised path, element strides:
 *  x(t, g, k) at x[t*stride_t + g*stride_g + k],  k < D.
 * Passing NULL selects token-major [T][G][D] (stride_t = G*D, stride_g = D),
 * the [num_tokens, n_groups, group_dim] tensor [GWA] grouped_input returns
 * (the same memory order as o).  Both strides must be multiples of 8
 * (16 bytes) and non-negative. */
typedef struct oproj_bf16_layout {
    int64_t stride_t, stride_g;
} oproj_bf16_layout;

/* Step a1 without quantisation ([GWA] grouped_input: the fused kernel with
 * quantize=False): the bf16 inverse-rotated groups.  For every token t and
 * head h (group g = h / hpg, offset j = (h % hpg)*512):
 *     x(t, g, j + k) = o[t][h][k]                      for k < 448 (copied)
 *     rotated pair i of the last 64 dims as in oproj_inv_rope_quant
 *     (e' = fma(d, s, e*c), d' = fma(-e, s, d*c) in fp32), rounded to bf16,
 *     nearest even.
 *  o          bf16 [T][H][512], contiguous;  positions int64 [T]
 *  cos_sin    fp32 [max_pos][64]
 *  x          bf16, layout `x_layout` (NULL: token-major [T][G][D])
 * o_lora_rank is not used.  A position outside [0, max_pos) writes NaN into
 * that token's 64 rotated dims of every head. */
oproj_status oproj_inv_rope_bf16(const oproj_shape* shape, const void* o, const int64_t* positions,
                                 const float* cos_sin, void* x, const oproj_bf16_layout* x_layout,
                                 void* stream);

/* Step a3 without quantisation ([OPROJ] deep_gemm_fp8_o_proj without FP8: a
 * batched matmul of the bf16 groups with wo_a viewed [G, R, D]; [GWA]):
 *   z[t][g][n] = sum_k x(t, g, k) * w[g*R + n][k],
 * bf16 inputs, fp32 accumulation, one bf16 rounding (nearest even).
 *  x   bf16 in layout `x_layout` (NULL: token-major [T][G][D])
 *  w   bf16 [G*R][D] row-major;  z bf16 [T][G][R]
 * Per group the activation rows must span at most 4 GiB ((T-1)*stride_t*2 +
 * D*2 bytes), and so must the group's R weight rows; else OPROJ_E_SHAPE. */
oproj_status oproj_grouped_wo_a_bf16(const oproj_shape* shape, const void* x,
                                     const oproj_bf16_layout* x_layout, const void* w, void* z,
                                     void* stream);

/* Bytes of caller-provided workspace oproj_fused_bf16 needs: the bf16 x and,
 * when hidden > 0, the bf16 z; each region 256-byte aligned. */
size_t oproj_fused_bf16_workspace_bytes(const oproj_shape* shape, int64_t hidden);

/* The unquantised path in one call ([OPROJ] deep_gemm_fp8_o_proj without
 * FP8): the bf16 rotation into the workspace (token-major x), the grouped
 * bf16 GEMM, and when wo_b != NULL the dense GEMM over z.flatten(1).
 *  w    bf16 [G*R][D];  wo_b bf16 [hidden][G*R] or NULL
 *  out  z bf16 [T][G][R] when wo_b == NULL, else y bf16 [T][hidden]
 * Every argument is validated before the first launch. */
oproj_status oproj_fused_bf16(const oproj_shape* shape, const void* o, const int64_t* positions,
                              const float* cos_sin, const void* w, const void* wo_b, int64_t hidden,
                              void* workspace, size_t workspace_bytes, void* out, void* stream);

/* Bytes of caller-provided workspace oproj_fused needs: the FP8 codes, the
 * scales and, when hidden > 0, the bf16 z; each region 256-byte aligned. */
size_t oproj_fused_workspace_bytes(const oproj_shape* shape, int64_t hidden);

/* The whole path in one call: a1 + a2 into the workspace, a3, and when
 * wo_b != NULL, a4 over z.flatten(1) ([OPROJ] deep_gemm_fp8_o_proj).
 *  out  z bf16 [T][G][R] when wo_b == NULL, else y bf16 [T][hidden]
 *  wo_b bf16 [hidden][G*R] row-major or NULL (hidden ignored when NULL)
 * The activation scales follow scale_mode; the weight scales must match it.
 * Enqueues the quantisation kernel, the grouped GEMM and, with wo_b, the dense
 * GEMM; every argument (wo_b included) is validated before the first launch. */
oproj_status oproj_fused(const oproj_shape* shape, int32_t scale_mode, const void* o,
                         const int64_t* positions, const float* cos_sin, const void* w_codes,
                         const void* w_scales, int32_t w_block, const void* wo_b, int64_t hidden,
                         void* workspace, size_t workspace_bytes, void* out, void* stream);

/* Size of the device array oproj_fused_noalloc uses as its workspace, one per
 * GPU, held until the process ends. */
#define OPROJ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* oproj_fused without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, kernels and result as oproj_fused
 * (out: z bf16 [T][G][R], or y bf16 [T][hidden] when wo_b != NULL); the
 * workspace is a device array the library holds per GPU, of
 * OPROJ_NOALLOC_SCRATCH_BYTES.  Allocates nothing: no hipMalloc, no hipFree.
 * A call whose oproj_fused_workspace_bytes(shape, wo_b ? hidden : 0) exceeds
 * that size returns OPROJ_E_SCRATCH and enqueues nothing.  Every call on one
 * GPU shares that GPU's array (whose contents persist between calls): calls
 * that overlap in time on one GPU, on any streams, race and give wrong
 * results.  The first call on each GPU looks up its array's device address
 * (hipGetSymbolAddress; OPROJ_E_HIP if that fails). */
oproj_status oproj_fused_noalloc(const oproj_shape* shape, int32_t scale_mode, const void* o,
                                 const int64_t* positions, const float* cos_sin, const void* w_codes,
                                 const void* w_scales, int32_t w_block, const void* wo_b, int64_t hidden,
                                 void* out, void* stream);

/* EXPERIMENTAL, opt-in: on MI355X this one-launch form has measured slower
 * than oproj_fused's two launches (about 24 us against 22 us per step at
 * T = 64, 16 groups x 8 heads, o_lora_rank 1024), so oproj_fused does not
 * use it.
 * Steps a1 + a2 + a3 of oproj_fused (wo_b == NULL) in ONE kernel launch, for
 * decode-sized batches, where the launch and the quantisation round trip sit
 * on the per-token critical path ([SGL] the wo_a decode path; [FUSED] feeds
 * the grouped GEMM directly).  Each workgroup first quantises its share of
 * its group's activations into the workspace, meets the group's other
 * workgroups at a barrier, then runs its output tile of the grouped GEMM.
 * Arguments and result are those of oproj_fused with wo_b == NULL; z is
 * bit-identical to it.  The workspace (oproj_fused_decode_workspace_bytes)
 * holds the codes and scales of oproj_fused followed by the groups' barrier
 * words: that last region (n_groups * 128 bytes, 256-byte rounded) must be
 * zero before the first call with a workspace, and each call leaves it ready
 * for the next one.
 * Supported: T <= 64, n_groups <= 256, heads_per_group 2 or a multiple of 4,
 * D / 128 >= 8, and n_groups * ceil(o_lora_rank / 64) workgroups no more than
 * the device's compute units (every workgroup resident at once); otherwise
 * OPROJ_E_SHAPE (or OPROJ_E_MODE for the head geometry) and nothing is
 * enqueued.
 * Concurrency: calls with distinct workspaces are independent and may
 * overlap; calls that share a workspace must not overlap in time.  A
 * workgroup that waits too long at its barrier quantises its whole group
 * itself, so a slow neighbour costs time, never correctness.  The environment
 * variable OPROJ_FUSED_DECODE_SPIN_LIMIT (read at each call; diagnostics and
 * tests) lowers the number of polls before that fallback, down to 0. */
size_t oproj_fused_decode_workspace_bytes(const oproj_shape* shape);
oproj_status oproj_fused_decode(const oproj_shape* shape, int32_t scale_mode, const void* o,
                                const int64_t* positions, const float* cos_sin, const void* w_codes,
                                const void* w_scales, int32_t w_block, void* workspace,
                                size_t workspace_bytes, void* z, void* stream);

/* Whether oproj_fused_decode can take a call of this shape and these modes on
 * the current device: NULL when it can, else a short reason (static storage),
 * like the eligibility check that reports why a layer cannot take the fused
 * inverse RoPE + FP8 output, or None ([OPROJ] rope_quant_unsupported_reason).
 * Pointers are not examined; T == 0 is reported as supported.  Queries the
 * current device's compute-unit count. */
const char* oproj_fused_decode_unsupported(const oproj_shape* shape, int32_t scale_mode, int32_t w_block);

/* Offline weight preparation ([OPROJ] compute_fp8_einsum_recipe; [SGL]
 * _setup_fp8_wo_a_scales): quantise fp32 w[rows][K] to FP8 codes with one
 * scale per block (128x128 or 1x128 per `w_block`), scale = amax/448
 * (pow2: rounded up to a power of two; OPROJ_SCALE_E8M0 gives the same fp32
 * powers of two), code = e4m3fn(w / scale).
 *  w        fp32 [rows][K];  codes FP8 [rows][K];  scales per oproj_wblock
 *  K must be a multiple of 128 (of 512 for OPROJ_WBLOCK_1x128_UE8M0, which
 *  also needs a power-of-two scale_mode). */
oproj_status oproj_quantize_weight(int64_t rows, int64_t K, int32_t w_block, int32_t scale_mode,
                                   const float* w, void* codes, void* scales, void* stream);

/* Human-readable name of a status code (static storage). */
const char* oproj_status_string(oproj_status status);

/* Library version, "MAJOR.MINOR.PATCH" (static storage). */
const char* oproj_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OPROJ_H */
