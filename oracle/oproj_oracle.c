/*
 * oproj_oracle.c -- plain, slow CPU reference of the DeepSeek-V4 attention
 * O-projection front half: inverse RoPE -> 1x128 block FP8 (e4m3fn)
 * quantisation -> grouped wo_a contraction -> optional dense wo_b.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle the HIP library is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it; the product path never does.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 *        (no contraction: every fused multiply-add below is written as fmaf()).
 *
 * Sources (web pages; cited by page title and section):
 *  [FUSED] vLLM API page "vllm.models.deepseek_v4.common.ops.fused_inv_rope_fp8_quant",
 *          function fused_inv_rope_fp8_quant (parameter table, returns, preconditions).
 *  [OPROJ] vLLM API page "vllm.models.deepseek_v4.nvidia.ops.o_proj",
 *          functions compute_fp8_einsum_recipe and deep_gemm_fp8_o_proj.
 *  [GWA]   vLLM API page "vllm.models.deepseek_v4.common.grouped_wo_a",
 *          class DeepseekV4GroupedWoA.
 *  [SGL]   sglang source page "python/sglang/srt/models/deepseek_v4.py":
 *          MQALayer.forward (O-projection half), _freqs_cis_to_cos_sin,
 *          _dequant_fp8, _setup_fp8_wo_a_scales, _apply_gguf_grouped_wo_a.
 *  [OCP]   OCP 8-bit Floating Point Specification (OFP8), E4M3 format.
 *
 * Readings taken where the pages leave a step open (each restated where used):
 *  R1  "inverse" RoPE is rotation by -theta: the pair (e, d) is multiplied by
 *      conj(cos + i sin).  Pairs are interleaved (2i, 2i+1) and use cos[i] and
 *      sin[i] from the cos||sin table row of the token's position.
 *  R2  rotation op order in fp32: e' = fmaf(d, s, e*c), d' = fmaf(-e, s, d*c).
 *  R3  quantisation reads the fp32 rotated values (no bf16 re-rounding).
 *  R4  all-zero block: amax is floored at 1e-10 before the scale is formed.
 *  R5  scale = amax / 448 by IEEE fp32 division; pow2 mode rounds that fp32
 *      value up to the next power of two (kept as-is when already one).
 *  R6  codes: q = encode(v / scale), IEEE fp32 division, then round to the
 *      nearest e4m3fn value with ties to even, saturating to +-448.
 *  R7  weight scales are multipliers: W ~= decode(q) * scale ([SGL] _dequant_fp8),
 *      over 128x128 tiles of the flat [G*R, D] matrix or 1x128 per-row blocks.
 *  R8  grouped GEMM accumulates in fp64; z rounds once fp64 -> bf16 (nearest
 *      even) when it feeds wo_b; wo_b accumulates in fp64.
 *  R9  unquantised path ([GWA] grouped_input calls the fused kernel with
 *      quantize=False and returns bf16 groups): the rotated dims are rounded
 *      fp32 -> bf16 to nearest even; dims 0..nope-1 are copied unchanged.  The
 *      grouped bf16 contraction ([OPROJ] deep_gemm_fp8_o_proj without FP8:
 *      one matmul per group) accumulates in fp64.
 *  R10 packed UE8M0 scales ([OPROJ] rope_quant_attn_out and
 *      compute_fp8_einsum_recipe: one int32 per head over its four 128-wide
 *      blocks, MN-major): the byte of a power-of-two scale 2^k is k + 127 (an
 *      unsigned biased exponent, no mantissa); NaN is 0xFF; block 4j+b of the
 *      row sits in bits 8b..8b+7 of word j (the four bytes in memory order).
 *  R2, R3 and R4 are conventions the pages leave open: parity unpinned for
 *  those choices (both sides follow them; the tests pin everything else).
 *  R11 attention-epilogue producer ([OPROJ] rope_quant_attn_out: the output
 *      pair a fused attention epilogue writes, FP8 codes plus packed UE8M0
 *      scales, with no bf16 attention output in between): its input is the
 *      attention output as fp32 values, which go through the same rotation
 *      (R1, R2) and quantisation (R3-R6) with no rounding to bf16 anywhere.
 *      For fp32 inputs that are bf16 values it is step a1 + a2 exactly.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FP8_MAX 448.0f /* largest finite e4m3fn magnitude [OCP]; [FUSED] uses finfo(e4m3fn).max */
#define ORC_AMAX_FLOOR 1e-10f /* R4 */

/* ------------------------------------------------------------------ */
/* scalar codecs                                                       */
/* ------------------------------------------------------------------ */

/* bf16 -> fp32 is exact: bf16 is the top half of an fp32 bit pattern. */
float orc_bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Decode one e4m3fn code from its definition [OCP]: sign bit, 4 exponent bits
 * (bias 7), 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9);
 * S.1111.111 is NaN; there is no infinity. */
float orc_e4m3_decode(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return sign ? -NAN : NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(sign ? -v : v);
}

/* Round a non-negative double to the nearest integer, ties to even. */
static double orc_round_half_even(double x) {
    double f = floor(x);
    double r = x - f;
    if (r > 0.5) return f + 1.0;
    if (r < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* Encode fp32 -> e4m3fn, round to nearest (ties to even), saturating finite
 * values to +-448 (R6).  NaN gives the NaN code with the input's sign. */
uint8_t orc_e4m3_encode(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (isnan(x)) return (uint8_t)(sign | 0x7F);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E); /* 448 = 1.75 * 2^8 */
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: value = n * 2^-9, n in 0..8 (8 becomes the min normal) */
        double n = orc_round_half_even(a * 512.0);
        /* a*512 is exact; n == 8 encodes as exponent field 1, mantissa 0 */
        return (uint8_t)(sign | (uint8_t)n);
    }
    {
        int e;
        double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
        int ue = e - 1;          /* a = (2f) * 2^ue, 2f in [1, 2) */
        double frac = (2.0 * f - 1.0) * 8.0; /* exact: mantissa in units of 2^-3 */
        /* frac is a multiple of 2^-20 at most, not necessarily of 0.5: round properly */
        double k = floor(frac);
        double rem = frac - k;
        if (rem > 0.5 || (rem == 0.5 && fmod(k, 2.0) != 0.0)) k += 1.0;
        if (k == 8.0) {
            k = 0.0;
            ue += 1;
        }
        /* a < 448 guarantees ue <= 8 and (ue == 8 -> k <= 6) */
        return (uint8_t)(sign | (uint8_t)(((ue + 7) << 3) | (int)k));
    }
}

/* fp64 -> bf16, round to nearest even, from the 8-bit significand definition
 * (R8).  Finite, non-overflowing inputs are assumed (z and y are O(1)). */
uint16_t orc_f64_to_bf16(double x) {
    float f;
    uint32_t u;
    if (x == 0.0 || isnan(x)) {
        f = (float)x;
    } else {
        int e;
        double m = frexp(fabs(x), &e);        /* |x| = m * 2^e, m in [0.5, 1) */
        double sig = m * 256.0;                /* 8 significant bits before the point */
        double k = floor(sig);
        double rem = sig - k;
        if (rem > 0.5 || (rem == 0.5 && fmod(k, 2.0) != 0.0)) k += 1.0;
        double v = ldexp(k, e - 8);
        f = (float)(x < 0 ? -v : v);
    }
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* R5: round a positive normal fp32 scale up to a power of two, exactly. */
float orc_pow2_ceil(float s) {
    int e;
    double f = frexp((double)s, &e); /* s = f * 2^e, f in [0.5, 1) */
    if (f == 0.5) return s;         /* already a power of two */
    return (float)ldexp(1.0, e);
}

/* ------------------------------------------------------------------ */
/* step a1: inverse RoPE                                               */
/* ------------------------------------------------------------------ */

/* Inverse RoPE of one head row, fp32 in and out (R1, R2).  The last rope_dim
 * dims of the head are the rotated slice ([SGL] MQALayer.forward rotates
 * o[..., -rope_dim:] with inverse=True; [FUSED] requires
 * head_dim == nope_dim + rope_dim).  The table row is cos[0..rope/2) followed
 * by sin[0..rope/2) ([FUSED] parameter table: cos||sin; [SGL]
 * _freqs_cis_to_cos_sin: cos is the real and sin the imaginary part). */
static void orc_inv_rope_row(float* x, int64_t nope, int64_t rope, const float* row) {
    int64_t half = rope / 2;
    for (int64_t i = 0; i < half; ++i) {
        float e = x[nope + 2 * i];
        float d = x[nope + 2 * i + 1];
        float c = row[i];
        float s = row[half + i];
        x[nope + 2 * i] = fmaf(d, s, e * c);
        x[nope + 2 * i + 1] = fmaf(-e, s, d * c);
    }
}

/* Forward RoPE (rotation by +theta), used only to pin the inverse. */
static void orc_fwd_rope_row(float* x, int64_t nope, int64_t rope, const float* row) {
    int64_t half = rope / 2;
    for (int64_t i = 0; i < half; ++i) {
        float e = x[nope + 2 * i];
        float d = x[nope + 2 * i + 1];
        float c = row[i];
        float s = row[half + i];
        x[nope + 2 * i] = fmaf(-d, s, e * c);
        x[nope + 2 * i + 1] = fmaf(e, s, d * c);
    }
}

/* Apply inverse (dir=-1) or forward (dir=+1) RoPE to fp32 rows
 * x[T][H][head_dim] in place, with positions[T] and table[max_pos][rope]. */
void orc_rope_f32(int64_t T, int64_t H, int64_t nope, int64_t rope, float* x,
                  const int64_t* positions, const float* table, int dir) {
    int64_t hd = nope + rope;
    for (int64_t t = 0; t < T; ++t) {
        const float* row = table + positions[t] * rope;
        for (int64_t h = 0; h < H; ++h) {
            float* xr = x + (t * H + h) * hd;
            if (dir < 0)
                orc_inv_rope_row(xr, nope, rope, row);
            else
                orc_fwd_rope_row(xr, nope, rope, row);
        }
    }
}

/* ------------------------------------------------------------------ */
/* step a2: 1 x block FP8 quantisation                                 */
/* ------------------------------------------------------------------ */

/* Quantise one block of n fp32 values (R4, R5, R6).  Returns the scale. */
static float orc_quant_block(const float* v, int64_t n, int64_t stride, int pow2, uint8_t* q,
                             int64_t qstride) {
    float amax = 0.0f;
    for (int64_t j = 0; j < n; ++j) {
        float a = fabsf(v[j * stride]);
        if (a > amax) amax = a;
    }
    if (amax < ORC_AMAX_FLOOR) amax = ORC_AMAX_FLOOR;
    float s = amax / ORC_FP8_MAX;
    if (pow2) s = orc_pow2_ceil(s);
    for (int64_t j = 0; j < n; ++j) q[j * qstride] = orc_e4m3_encode(v[j * stride] / s);
    return s;
}

/* Quantise rows v[rows][D] in contiguous 1 x blk blocks:
 * q[rows][D] codes, s[rows][D/blk] scales. */
void orc_block_quant_rows(int64_t rows, int64_t D, int64_t blk, int pow2, const float* v,
                          uint8_t* q, float* s) {
    int64_t nb = D / blk;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b)
            s[r * nb + b] = orc_quant_block(v + r * D + b * blk, blk, 1, pow2, q + r * D + b * blk, 1);
}

/* a1 + a2 for the whole batch, the way [FUSED] fused_inv_rope_fp8_quant
 * describes its result: codes logically [T][G][D] with D = hpg*head_dim,
 * one scale per (token, group, blk-wide block).  Here both outputs are written
 * token-major and contiguous: q[T][G][D], s[T][G][D/blk].  The grouping of heads
 * follows [SGL] MQALayer.forward (o.view(T, n_groups, -1): head h belongs to
 * group h / hpg at offset (h % hpg) * head_dim).
 * Positions must lie in [0, max_pos).  Threads split the tokens. */
struct orc_irq_job {
    int64_t t0, t1, G, hpg, nope, rope, blk;
    int pow2;
    const uint16_t* o; /* bf16 input, or NULL when of is given */
    const float* of;   /* fp32 input (R11) */
    const int64_t* pos;
    const float* table;
    uint8_t* q;
    float* s;
};

static void* orc_irq_worker(void* arg) {
    struct orc_irq_job* j = (struct orc_irq_job*)arg;
    int64_t hd = j->nope + j->rope;
    int64_t H = j->G * j->hpg;
    int64_t D = j->hpg * hd;
    int64_t nb = D / j->blk;
    float* row = (float*)malloc((size_t)D * sizeof(float));
    for (int64_t t = j->t0; t < j->t1; ++t) {
        const float* trow = j->table + j->pos[t] * j->rope;
        for (int64_t g = 0; g < j->G; ++g) {
            /* gather the group's heads as fp32, rotating each head's tail */
            for (int64_t hh = 0; hh < j->hpg; ++hh) {
                const int64_t at = (t * H + g * j->hpg + hh) * hd;
                float* dst = row + hh * hd;
                for (int64_t k = 0; k < hd; ++k) dst[k] = j->of ? j->of[at + k] : orc_bf16_to_f32(j->o[at + k]);
                orc_inv_rope_row(dst, j->nope, j->rope, trow);
            }
            uint8_t* qd = j->q + (t * j->G + g) * D;
            float* sd = j->s + (t * j->G + g) * nb;
            for (int64_t b = 0; b < nb; ++b)
                sd[b] = orc_quant_block(row + b * j->blk, j->blk, 1, j->pow2, qd + b * j->blk, 1);
        }
    }
    free(row);
    return NULL;
}

static int orc_clamp_threads(int64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n < nthreads) nthreads = (int)(n > 0 ? n : 1);
    return nthreads;
}

static void orc_irq_run(int64_t T, int64_t G, int64_t hpg, int64_t nope, int64_t rope, int64_t blk,
                        int pow2, const uint16_t* o, const float* of, const int64_t* pos,
                        const float* table, uint8_t* q, float* s, int nthreads) {
    nthreads = orc_clamp_threads(T, nthreads);
    pthread_t th[256];
    struct orc_irq_job jobs[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (struct orc_irq_job){T * i / nthreads, T * (i + 1) / nthreads, G, hpg, nope, rope,
                                       blk, pow2, o, of, pos, table, q, s};
        pthread_create(&th[i], NULL, orc_irq_worker, &jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

void orc_inv_rope_quant(int64_t T, int64_t G, int64_t hpg, int64_t nope, int64_t rope,
                        int64_t blk, int pow2, const uint16_t* o, const int64_t* pos,
                        const float* table, uint8_t* q, float* s, int nthreads) {
    orc_irq_run(T, G, hpg, nope, rope, blk, pow2, o, NULL, pos, table, q, s, nthreads);
}

/* The attention-epilogue producer (R11): the same steps from fp32 o[T][H][head_dim]. */
void orc_inv_rope_quant_f32(int64_t T, int64_t G, int64_t hpg, int64_t nope, int64_t rope,
                            int64_t blk, int pow2, const float* o, const int64_t* pos,
                            const float* table, uint8_t* q, float* s, int nthreads) {
    orc_irq_run(T, G, hpg, nope, rope, blk, pow2, NULL, o, pos, table, q, s, nthreads);
}

/* Unquantised step a1 (R1, R2, R9): o[T][H][head_dim] bf16 -> x bf16 in the
 * same token-major layout, i.e. [T][G][hpg*head_dim] ([GWA] grouped_input's
 * [num_tokens, n_groups, group_dim] view of the heads). */
void orc_inv_rope_bf16(int64_t T, int64_t H, int64_t nope, int64_t rope, const uint16_t* o,
                       const int64_t* pos, const float* table, uint16_t* x) {
    int64_t hd = nope + rope;
    float* row = (float*)malloc((size_t)hd * sizeof(float));
    for (int64_t t = 0; t < T; ++t) {
        const float* trow = table + pos[t] * rope;
        for (int64_t h = 0; h < H; ++h) {
            const uint16_t* src = o + (t * H + h) * hd;
            uint16_t* dst = x + (t * H + h) * hd;
            for (int64_t k = 0; k < hd; ++k) row[k] = orc_bf16_to_f32(src[k]);
            orc_inv_rope_row(row, nope, rope, trow);
            for (int64_t k = 0; k < nope; ++k) dst[k] = src[k];
            /* fp32 -> fp64 is exact, so this is the nearest-even bf16 of the fp32 value */
            for (int64_t k = nope; k < hd; ++k) dst[k] = orc_f64_to_bf16((double)row[k]);
        }
    }
    free(row);
}

/* ------------------------------------------------------------------ */
/* offline weight quantisation (R7)                                    */
/* ------------------------------------------------------------------ */

/* w[rows][K] fp32 -> q[rows][K] codes and s[ceil(rows/brows)][K/128] scales.
 * brows = 128 gives 128x128 tiles of the flat matrix; brows = 1 gives 1x128
 * per-row blocks ([OPROJ] compute_fp8_einsum_recipe names the two recipes
 * (1,128,128) and (1,1,128)). */
void orc_quant_weight(int64_t rows, int64_t K, int64_t brows, int pow2, const float* w,
                      uint8_t* q, float* s) {
    int64_t kb = K / 128;
    int64_t rb = (rows + brows - 1) / brows;
    for (int64_t i = 0; i < rb; ++i) {
        int64_t r0 = i * brows;
        int64_t r1 = r0 + brows < rows ? r0 + brows : rows;
        for (int64_t b = 0; b < kb; ++b) {
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t k = b * 128; k < b * 128 + 128; ++k) {
                    float a = fabsf(w[r * K + k]);
                    if (a > amax) amax = a;
                }
            if (amax < ORC_AMAX_FLOOR) amax = ORC_AMAX_FLOOR;
            float sc = amax / ORC_FP8_MAX;
            if (pow2) sc = orc_pow2_ceil(sc);
            s[i * kb + b] = sc;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t k = b * 128; k < b * 128 + 128; ++k)
                    q[r * K + k] = orc_e4m3_encode(w[r * K + k] / sc);
        }
    }
}

/* Dequantised weight element (R7): decode(q) * scale. */
static double orc_wdq(const uint8_t* qw, const float* sw, int64_t K, int64_t brows, int64_t r,
                      int64_t k) {
    return (double)orc_e4m3_decode(qw[r * K + k]) * (double)sw[(r / brows) * (K / 128) + k / 128];
}

/* ------------------------------------------------------------------ */
/* step a3: grouped wo_a contraction (R8)                              */
/* ------------------------------------------------------------------ */

/* Activation operand descriptor: code (t, g, k) at qa[t*st + g*sg + k],
 * scale (t, g, b) at sa[t*sst + g*ssg + b*ssb].  Only groups < G are read
 * ([OPROJ] deep_gemm_fp8_o_proj keeps the live groups of a pre-quantised
 * input and drops the padding groups after them). */
struct orc_act {
    const uint8_t* qa;
    const float* sa;
    int64_t st, sg, sst, ssg, ssb;
};

/* z[t][g][n] = sum_k (decode(qa[t,g,k]) * sa[t,g,k/128]) * Wd[g*R + n][k]:
 * group g meets only weight rows g*R .. g*R+R-1 ([GWA] class docstring;
 * [OPROJ] einsum "bhr,hdr->bhd" on wo_a viewed [G, R, D]). */
static double orc_gemm_one(const struct orc_act* a, const uint8_t* qw, const float* sw,
                           int64_t D, int64_t R, int64_t brows, int64_t t, int64_t g, int64_t n) {
    double acc = 0.0;
    int64_t wr = g * R + n;
    for (int64_t k = 0; k < D; ++k) {
        double av = (double)orc_e4m3_decode(a->qa[t * a->st + g * a->sg + k]) *
                    (double)a->sa[t * a->sst + g * a->ssg + (k / 128) * a->ssb];
        acc += av * orc_wdq(qw, sw, D, brows, wr, k);
    }
    return acc;
}

struct orc_gemm_job {
    int64_t i0, i1, T, G, D, R, brows;
    struct orc_act a;
    const uint8_t* qw;
    const float* sw;
    const int64_t* idx; /* NULL: dense [T][G][R]; else triples (t, g, n) */
    double* z;
};

static void* orc_gemm_worker(void* arg) {
    struct orc_gemm_job* j = (struct orc_gemm_job*)arg;
    for (int64_t i = j->i0; i < j->i1; ++i) {
        int64_t t, g, n;
        if (j->idx) {
            t = j->idx[3 * i];
            g = j->idx[3 * i + 1];
            n = j->idx[3 * i + 2];
        } else {
            t = i / (j->G * j->R);
            g = (i / j->R) % j->G;
            n = i % j->R;
        }
        j->z[i] = orc_gemm_one(&j->a, j->qw, j->sw, j->D, j->R, j->brows, t, g, n);
    }
    return NULL;
}

/* Dense (idx == NULL, count ignored, z[T][G][R]) or sampled (idx = count
 * triples (t, g, n), z[count]) grouped contraction in fp64. */
void orc_grouped_gemm(int64_t T, int64_t G, int64_t D, int64_t R, const uint8_t* qa,
                      const float* sa, int64_t st, int64_t sg, int64_t sst, int64_t ssg,
                      int64_t ssb, const uint8_t* qw, const float* sw, int64_t brows,
                      const int64_t* idx, int64_t count, double* z, int nthreads) {
    int64_t total = idx ? count : T * G * R;
    nthreads = orc_clamp_threads(total, nthreads);
    pthread_t th[256];
    struct orc_gemm_job jobs[256];
    struct orc_act a = {qa, sa, st, sg, sst, ssg, ssb};
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (struct orc_gemm_job){total * i / nthreads, total * (i + 1) / nthreads, T, G, D, R,
                                        brows, a, qw, sw, idx, z};
        pthread_create(&th[i], NULL, orc_gemm_worker, &jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* ------------------------------------------------------------------ */
/* step a4: dense wo_b over the flattened z (R8)                       */
/* ------------------------------------------------------------------ */

/* y[m][j] = sum_c x[m][c] * w[j][c] with bf16 x[M][K], bf16 w[N][K] (linear
 * layer convention: wo_b maps G*R -> hidden, [SGL] MQALayer.forward applies
 * wo_b to z.flatten(1)). */
struct orc_dense_job {
    int64_t i0, i1, N, K;
    const uint16_t* x;
    const uint16_t* w;
    const int64_t* idx; /* NULL: dense [M][N]; else pairs (m, j) */
    double* y;
};

static void* orc_dense_worker(void* arg) {
    struct orc_dense_job* j = (struct orc_dense_job*)arg;
    for (int64_t i = j->i0; i < j->i1; ++i) {
        int64_t m = j->idx ? j->idx[2 * i] : i / j->N;
        int64_t c = j->idx ? j->idx[2 * i + 1] : i % j->N;
        double acc = 0.0;
        for (int64_t k = 0; k < j->K; ++k)
            acc += (double)orc_bf16_to_f32(j->x[m * j->K + k]) *
                   (double)orc_bf16_to_f32(j->w[c * j->K + k]);
        j->y[i] = acc;
    }
    return NULL;
}

void orc_dense_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t* x, const uint16_t* w,
                         const int64_t* idx, int64_t count, double* y, int nthreads) {
    int64_t total = idx ? count : M * N;
    nthreads = orc_clamp_threads(total, nthreads);
    pthread_t th[256];
    struct orc_dense_job jobs[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (struct orc_dense_job){total * i / nthreads, total * (i + 1) / nthreads, N, K, x, w,
                                         idx, y};
        pthread_create(&th[i], NULL, orc_dense_worker, &jobs[i]);
    }
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
}

/* UE8M0 byte of one scale (R10): the biased exponent of a power of two,
 * found by halving/doubling in exact fp64 arithmetic (no bit tricks); 0xFF
 * for NaN; -1 if the value is not a positive power of two in [2^-127, 2^127]. */
int orc_e8m0_byte(float s) {
    if (isnan(s)) return 0xFF;
    double v = (double)s;
    if (!(v > 0.0)) return -1;
    int k = 0;
    while (v >= 2.0) { v /= 2.0; ++k; }
    while (v < 1.0) { v *= 2.0; --k; }
    if (v != 1.0 || k < -127 || k > 127) return -1;
    return k + 127;
}

/* Pack rows of n scales (n % 4 == 0) into n/4 words per row (R10).
 * Returns 0, or -1 when some scale has no UE8M0 byte. */
int orc_e8m0_pack(int64_t rows, int64_t n, const float* s, uint32_t* w) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < n / 4; ++j) {
            uint32_t word = 0;
            for (int b = 0; b < 4; ++b) {
                int e = orc_e8m0_byte(s[r * n + 4 * j + b]);
                if (e < 0) return -1;
                word |= (uint32_t)e << (8 * b);
            }
            w[r * (n / 4) + j] = word;
        }
    return 0;
}

/* Array helpers for the Python side (vectorised codecs). */
void orc_e4m3_encode_array(int64_t n, const float* x, uint8_t* q) {
    for (int64_t i = 0; i < n; ++i) q[i] = orc_e4m3_encode(x[i]);
}
void orc_e4m3_decode_array(int64_t n, const uint8_t* q, float* x) {
    for (int64_t i = 0; i < n; ++i) x[i] = orc_e4m3_decode(q[i]);
}
void orc_f64_to_bf16_array(int64_t n, const double* x, uint16_t* h) {
    for (int64_t i = 0; i < n; ++i) h[i] = orc_f64_to_bf16(x[i]);
}
void orc_pow2_ceil_array(int64_t n, const float* x, float* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = orc_pow2_ceil(x[i]);
}
