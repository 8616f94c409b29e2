/* Host AddressSanitizer / UndefinedBehaviorSanitizer run of the CPU oracle
 * (test infrastructure): every oracle routine on small ragged inputs, dense
 * and sampled, several threads, with odd sizes that end buffers exactly where
 * the routines must stop reading or writing.  Built with -fsanitize=address,
 * undefined and -fno-sanitize-recover=all by tests/test_sanitizers_cpu.py,
 * so any out-of-bounds access, leak or undefined operation fails the run.
 * The arithmetic is checked elsewhere; here only memory and UB are. */
#include "../../oracle/oproj_oracle.c"

#include <stdio.h>

static uint64_t rng = 0x243F6A8885A308D3ull;
static double urand(void) { /* xorshift64*: inputs only */
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (double)((rng * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static float nrand(void) { return (float)(2.0 * urand() - 1.0); }

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

int main(void) {
    /* codecs over every code and a spread of floats */
    for (int c = 0; c < 256; ++c) (void)orc_e4m3_encode(orc_e4m3_decode((uint8_t)c));
    float xs[7] = {0.f, -0.f, 1e-30f, 448.f, 449.f, -1e30f, 3.5f};
    for (int i = 0; i < 7; ++i) { (void)orc_e4m3_encode(xs[i]); (void)orc_pow2_ceil(xs[i] > 0 ? xs[i] : 1.f); }
    for (int i = 0; i < 7; ++i) (void)orc_f64_to_bf16((double)xs[i]);

    const int64_t T = 5, G = 3, hpg = 2, nope = 448, rope = 64, blk = 128, hd = 512, max_pos = 17;
    const int64_t H = G * hpg, D = hpg * hd, KB = D / blk, R = 192;
    uint16_t* o = xmalloc(sizeof(uint16_t) * T * H * hd);
    float* of = xmalloc(sizeof(float) * T * H * hd);
    for (int64_t i = 0; i < T * H * hd; ++i) { of[i] = nrand(); o[i] = orc_f64_to_bf16(of[i]); }
    int64_t* pos = xmalloc(sizeof(int64_t) * T);
    for (int64_t t = 0; t < T; ++t) pos[t] = (t * 7) % max_pos;
    pos[T - 1] = max_pos - 1;
    float* tab = xmalloc(sizeof(float) * max_pos * rope);
    for (int64_t i = 0; i < max_pos * rope; ++i) tab[i] = nrand();

    /* a1 + a2, both producers, both scale modes, 1..4 threads */
    uint8_t* qa = xmalloc((size_t)T * G * D);
    float* sa = xmalloc(sizeof(float) * T * G * KB);
    for (int pow2 = 0; pow2 < 2; ++pow2)
        for (int nt = 1; nt <= 4; nt += 3) {
            orc_inv_rope_quant(T, G, hpg, nope, rope, blk, pow2, o, pos, tab, qa, sa, nt);
            orc_inv_rope_quant_f32(T, G, hpg, nope, rope, blk, pow2, of, pos, tab, qa, sa, nt);
        }
    float* x = xmalloc(sizeof(float) * T * H * hd);
    memcpy(x, of, sizeof(float) * T * H * hd);
    orc_rope_f32(T, H, nope, rope, x, pos, tab, -1);
    orc_rope_f32(T, H, nope, rope, x, pos, tab, 1);
    uint16_t* xb = xmalloc(sizeof(uint16_t) * T * H * hd);
    orc_inv_rope_bf16(T, H, nope, rope, o, pos, tab, xb);
    uint8_t* qr = xmalloc((size_t)3 * 384);
    float* sr = xmalloc(sizeof(float) * 3 * 3);
    orc_block_quant_rows(3, 384, 128, 1, of, qr, sr);

    /* weights: 128x128 blocks over rows that end mid-block, and 1x128 */
    float* w = xmalloc(sizeof(float) * G * R * D);
    for (int64_t i = 0; i < G * R * D; ++i) w[i] = 0.02f * nrand();
    uint8_t* qw = xmalloc((size_t)G * R * D);
    const int64_t rb = (G * R + 127) / 128;
    float* sw = xmalloc(sizeof(float) * G * R * KB);
    orc_quant_weight(G * R, D, 128, 0, w, qw, sw);

    /* grouped contraction: dense and sampled, with a padding group */
    const int64_t Gp = G + 1;
    uint8_t* qp = xmalloc((size_t)T * Gp * D);
    float* sp = xmalloc(sizeof(float) * T * Gp * KB);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t g = 0; g < Gp; ++g) {
            for (int64_t k = 0; k < D; ++k) qp[(t * Gp + g) * D + k] = g < G ? qa[(t * G + g) * D + k] : 0x7F;
            for (int64_t b = 0; b < KB; ++b) sp[(t * Gp + g) * KB + b] = g < G ? sa[(t * G + g) * KB + b] : 1.f;
        }
    double* z = xmalloc(sizeof(double) * T * G * R);
    for (int nt = 1; nt <= 5; nt += 4)
        orc_grouped_gemm(T, G, D, R, qp, sp, Gp * D, D, Gp * KB, KB, 1, qw, sw, 128, NULL, 0, z, nt);
    int64_t idx[6] = {0, 0, 0, T - 1, G - 1, R - 1};
    double zs[2];
    orc_grouped_gemm(T, G, D, R, qp, sp, Gp * D, D, Gp * KB, KB, 1, qw, sw, 128, idx, 2, zs, 2);
    orc_quant_weight(G * R, D, 1, 1, w, qw, sw);
    orc_grouped_gemm(T, G, D, R, qp, sp, Gp * D, D, Gp * KB, KB, 1, qw, sw, 1, NULL, 0, z, 3);
    (void)rb;

    /* wo_b over the flattened z */
    const int64_t M = T, K = G * R, N = 40;
    uint16_t* zb = xmalloc(sizeof(uint16_t) * M * K);
    orc_f64_to_bf16_array(M * K, z, zb);
    uint16_t* wb = xmalloc(sizeof(uint16_t) * N * K);
    for (int64_t i = 0; i < N * K; ++i) wb[i] = orc_f64_to_bf16(0.02 * nrand());
    double* y = xmalloc(sizeof(double) * M * N);
    orc_dense_gemm_bf16(M, N, K, zb, wb, NULL, 0, y, 3);
    int64_t yidx[4] = {0, 0, M - 1, N - 1};
    double ys[2];
    orc_dense_gemm_bf16(M, N, K, zb, wb, yidx, 2, ys, 1);

    /* packed UE8M0 and array codecs */
    float ps[8] = {1.f, 0.5f, 0.25f, 2.f, 4.f, 8.f, 0.125f, 1.f};
    uint32_t pw[2];
    if (orc_e8m0_pack(1, 8, ps, pw) != 0) return 3;
    float bad[4] = {1.f, 3.f, 1.f, 1.f};
    if (orc_e8m0_pack(1, 4, bad, pw) == 0) return 4;
    uint8_t cq[7];
    float cf[7];
    orc_e4m3_encode_array(7, xs, cq);
    orc_e4m3_decode_array(7, cq, cf);
    float pc[7];
    float pin[7] = {1.f, 3.f, 1e-20f, 5.f, 448.f, 0.001f, 7.f};
    orc_pow2_ceil_array(7, pin, pc);

    free(o); free(of); free(pos); free(tab); free(qa); free(sa); free(x); free(xb); free(qr); free(sr);
    free(w); free(qw); free(sw); free(qp); free(sp); free(z); free(zb); free(wb); free(y);
    printf("oracle sanitizer run: ok\n");
    return 0;
}
