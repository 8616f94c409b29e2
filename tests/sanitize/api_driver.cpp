// Host AddressSanitizer / UndefinedBehaviorSanitizer run of the C-ABI
// validation (test infrastructure).  api.cpp is compiled for the host with
// the kernel launchers replaced by stubs that only count calls, so every
// entry point's argument checks and size arithmetic run without a GPU: bad
// and extreme shapes (sizes near the documented limits, where an unchecked
// product would overflow), null and misaligned pointers, every mode value.
// Each refused call must launch nothing; accepted calls launch the stubs.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "kernels.hpp"
#include "oproj.h"

static int g_launches = 0;

namespace oproj {
hipError_t launch_inv_rope_quant(const RopeQuantArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_quantize_weight(const WeightQuantArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_grouped_gemm(const GroupedGemmArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fused_decode(const RopeQuantArgs&, const GroupedGemmArgs&, uint64_t*, hipStream_t, bool* l) {
    ++g_launches;
    *l = true;
    return hipSuccess;
}
const char* fused_decode_unfit(int64_t T, int64_t, int64_t, int64_t) { return T > 64 ? "more than 64 tokens" : nullptr; }
hipError_t launch_inv_rope_bf16(const RopeBf16Args&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bf16_gemm(const Bf16GemmArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_dense_bf16_gemm(const DenseGemmArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace oproj

static int g_fail = 0;
#define EXPECT(cond)                                                       \
    do {                                                                   \
        if (!(cond)) {                                                     \
            std::fprintf(stderr, "line %d: %s failed\n", __LINE__, #cond); \
            ++g_fail;                                                      \
        }                                                                  \
    } while (0)

static oproj_shape shape(int64_t T, int64_t G, int64_t hpg, int64_t R, int64_t max_pos = 4096) {
    oproj_shape s{};
    s.T = T;
    s.n_groups = G;
    s.heads_per_group = hpg;
    s.nope_dim = 448;
    s.rope_dim = 64;
    s.quant_block = 128;
    s.o_lora_rank = R;
    s.max_pos = max_pos;
    return s;
}

int main() {
    void* P = reinterpret_cast<void*>(0x10000);  // aligned, never dereferenced (the stubs do not launch)
    void* BAD = reinterpret_cast<void*>(0x10004);
    const int64_t* pos = static_cast<const int64_t*>(P);
    const float* tab = static_cast<const float*>(P);
    const int64_t Ts[] = {0, 1, 63, 64, 65, 8192, (int64_t)1 << 20, ((int64_t)1 << 31) - 1, (int64_t)1 << 31,
                          ((int64_t)1 << 31) + 1, (int64_t)1 << 40, INT64_MAX / 2, INT64_MAX, -1, INT64_MIN};
    const int64_t Gs[] = {1, 16, 8192, (int64_t)1 << 20, -1};
    const int64_t hpgs[] = {1, 2, 3, 4, 8, 16, 1024, 65536, -4};
    const int64_t Rs[] = {0, 64, 1024, 65536, (int64_t)1 << 40};
    for (int64_t T : Ts)
        for (int64_t G : Gs)
            for (int64_t hpg : hpgs)
                for (int64_t R : Rs) {
                    const oproj_shape s = shape(T, G, hpg, R);
                    for (int mode = -1; mode <= 3; ++mode) {
                        const int before = g_launches;
                        const oproj_status a = oproj_inv_rope_quant(&s, mode, P, pos, tab, P, P, nullptr, nullptr);
                        const oproj_status b =
                            oproj_grouped_wo_a(&s, mode, P, P, nullptr, P, P, (mode + 3) % 3, P, nullptr);
                        const size_t ws = oproj_fused_workspace_bytes(&s, 7168);
                        const size_t wd = oproj_fused_decode_workspace_bytes(&s);
                        const oproj_status c = oproj_fused(&s, mode, P, pos, tab, P, P, 0, P, 7168, P, ws, P, nullptr);
                        const oproj_status d = oproj_fused_decode(&s, mode, P, pos, tab, P, P, 0, P, wd, P, nullptr);
                        const oproj_status e = oproj_inv_rope_bf16(&s, P, pos, tab, P, nullptr, nullptr);
                        const oproj_status f = oproj_grouped_wo_a_bf16(&s, P, nullptr, P, P, nullptr);
                        (void)oproj_fused_decode_unsupported(&s, mode, 0);
                        (void)oproj_fused_bf16_workspace_bytes(&s, 7168);
                        const oproj_status h = oproj_fused(&s, mode, P, pos, tab, P, P, 0, nullptr, 0, P,
                                                           oproj_fused_workspace_bytes(&s, 0) - 1, P, nullptr);
                        // a refused call launches nothing (an accepted one at most three kernels)
                        const int launched = g_launches - before;
                        int ok = 0;
                        for (oproj_status st : {a, b, c, d, e, f, h}) ok += st == OPROJ_OK;
                        EXPECT(launched <= 3 * ok);
                        if (T > 0 && (mode < 0 || mode > 2))
                            EXPECT(a != OPROJ_OK && b != OPROJ_OK && c != OPROJ_OK && d != OPROJ_OK);
                        if (T < 0 || G < 1 || hpg < 1) EXPECT(a != OPROJ_OK && e != OPROJ_OK && f != OPROJ_OK);
                    }
                }
    // null and misaligned pointers on a valid decode shape launch nothing
    const oproj_shape s = shape(64, 16, 8, 1024, 32768);
    const int before = g_launches;
    EXPECT(oproj_inv_rope_quant(&s, 0, nullptr, pos, tab, P, P, nullptr, nullptr) == OPROJ_E_NULL);
    EXPECT(oproj_inv_rope_quant(&s, 0, BAD, pos, tab, P, P, nullptr, nullptr) == OPROJ_E_ALIGN);
    EXPECT(oproj_grouped_wo_a(&s, 0, P, P, nullptr, P, P, 0, BAD, nullptr) == OPROJ_E_ALIGN);
    oproj_act_layout lay{4096, 64 * 4096 + 8, 1, 32 * 64, 64};
    EXPECT(oproj_grouped_wo_a(&s, 0, P, P, &lay, P, P, 0, P, nullptr) == OPROJ_E_ALIGN);
    EXPECT(oproj_dense_bf16_gemm(64, 7168, 16384, P, P, BAD, nullptr) == OPROJ_E_ALIGN);
    EXPECT(oproj_dense_bf16_gemm(INT64_MAX, 16, 64, P, P, P, nullptr) == OPROJ_E_SHAPE);
    EXPECT(oproj_dense_bf16_gemm(64, INT64_MAX - 15, 64, P, P, P, nullptr) == OPROJ_E_SHAPE);
    EXPECT(oproj_quantize_weight(INT64_MAX, 128, 0, 0, tab, P, P, nullptr) != OPROJ_OK);
    EXPECT(oproj_quantize_weight(128, INT64_MAX - 127, 0, 0, tab, P, P, nullptr) != OPROJ_OK);
    EXPECT(g_launches == before);
    // accepted calls reach the launchers
    EXPECT(oproj_inv_rope_quant(&s, 0, P, pos, tab, P, P, nullptr, nullptr) == OPROJ_OK);
    EXPECT(oproj_fused(&s, 0, P, pos, tab, P, P, 0, P, 7168, P, oproj_fused_workspace_bytes(&s, 7168), P,
                       nullptr) == OPROJ_OK);
    EXPECT(g_launches == before + 4);
    for (int st = -1; st <= 7; ++st) EXPECT(oproj_status_string(static_cast<oproj_status>(st)) != nullptr);
    EXPECT(oproj_version() != nullptr);
    if (g_fail) return 1;
    std::printf("api sanitizer run: ok (%d stub launches)\n", g_launches);
    return 0;
}
