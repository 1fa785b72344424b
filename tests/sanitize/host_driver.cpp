// Host-side exercise of libmdlstm's C ABI for a build with AddressSanitizer and UndefinedBehaviorSanitizer on
// the host code (no GPU: only entry points that run on the host, and the argument checks of the device entry
// points, which return before any launch). Exits 0 when every call returned what its declaration promises.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "mdlstm.h"

static int g_bad = 0;
#define EXPECT(cond)                                                                   \
    do {                                                                               \
        if (!(cond)) {                                                                 \
            std::fprintf(stderr, "%s:%d: failed: %s (%s)\n", __FILE__, __LINE__, #cond, \
                         mdl_last_error());                                            \
            ++g_bad;                                                                   \
        }                                                                              \
    } while (0)

// every host accessor of a layout, with buffers of exactly the documented sizes
static void inspect(const mdl_layout* L) {
    int64_t info[MDL_INFO_COUNT];
    EXPECT(mdl_layout_info(L, info) == MDL_OK);
    const int64_t n = info[MDL_INFO_N], P = info[MDL_INFO_CANVAS_H] * info[MDL_INFO_CANVAS_W];
    std::vector<int32_t> rects(4 * n), real(4 * n), row_start(info[MDL_INFO_ROWS] + 1), row_ex(n), eid(P);
    std::vector<uint8_t> border(P);
    EXPECT(mdl_layout_rects(L, rects.data(), real.data()) == MDL_OK);
    EXPECT(mdl_layout_rows(L, row_start.data(), row_ex.data()) == MDL_OK);
    EXPECT(mdl_layout_maps(L, eid.data(), border.data()) == MDL_OK);
    size_t bytes = 0, eo = 0, bo = 0;
    EXPECT(mdl_layout_device_size(L, &bytes, &eo, &bo) == MDL_OK);
    EXPECT(eo + 4 * (size_t)P <= bytes && bo + (size_t)P <= bytes);
    size_t ws = 0;
    EXPECT(mdl_workspace_size(L, 4, 16, &ws) == MDL_OK && ws > 0);
    EXPECT(mdl_ctc_workspace_size(L, 16, 80, 64, &ws) == MDL_OK);
    int64_t pixels = 0;
    for (int64_t e = 0; e < n; ++e) pixels += (int64_t)real[4 * e + 2] * real[4 * e + 3];
    int64_t inside = 0;
    for (int64_t p = 0; p < P; ++p) inside += eid[p] >= 0;
    EXPECT(pixels == info[MDL_INFO_REAL_PIXELS]);
    if (info[MDL_INFO_MODE] != MDL_PACK_PADDED) EXPECT(inside == pixels);
}

int main() {
    std::mt19937 rng(12345);
    const int modes[3] = {MDL_PACK_ALG1, MDL_PACK_PADDED, MDL_PACK_EXACT};
    for (int it = 0; it < 300; ++it) {
        const int n = 1 + (int)(rng() % 40);
        std::vector<int32_t> h(n), w(n);
        const int hmax = 1 + (int)(rng() % 50), wmax = 1 + (int)(rng() % 300);
        for (int e = 0; e < n; ++e) {
            h[e] = 1 + (int)(rng() % hmax);
            w[e] = 1 + (int)(rng() % wmax);
        }
        const int cw = 1 + (int)(rng() % 400), sep = (int)(rng() % 3), mode = modes[it % 3];
        mdl_layout* L = nullptr;
        EXPECT(mdl_pack(h.data(), w.data(), n, cw, sep, mode, &L) == MDL_OK);
        if (!L) continue;
        inspect(L);
        mdl_layout* L2 = nullptr;
        EXPECT(mdl_pack_level(L, 2, 4, 1 + cw / 4, sep, MDL_PACK_ALG1, &L2) == MDL_OK);
        if (L2) inspect(L2);
        size_t cb = 0;
        if (L2) EXPECT(mdl_blockconv_workspace_size(L2, 10, 2, 4, 20, &cb) == MDL_OK);
        mdl_layout_free(L2);
        mdl_layout_free(L);
    }
    // argument errors, each with a message and nothing written
    int32_t h1 = 3, w1 = 5, h0 = 0, wneg = -2;
    mdl_layout* L = nullptr;
    EXPECT(mdl_pack(&h1, &w1, 0, 8, 1, MDL_PACK_ALG1, &L) == MDL_EINVAL && L == nullptr);
    EXPECT(mdl_pack(&h0, &w1, 1, 8, 1, MDL_PACK_ALG1, &L) == MDL_EINVAL);
    EXPECT(mdl_pack(&h1, &wneg, 1, 8, 1, MDL_PACK_ALG1, &L) == MDL_EINVAL);
    EXPECT(mdl_pack(&h1, &w1, 1, 8, -1, MDL_PACK_ALG1, &L) == MDL_EINVAL);
    EXPECT(mdl_pack(&h1, &w1, 1, 8, 1, 99, &L) == MDL_EINVAL);
    EXPECT(mdl_pack(nullptr, &w1, 1, 8, 1, MDL_PACK_ALG1, &L) == MDL_EINVAL);
    EXPECT(mdl_pack(&h1, &w1, 1, 8, 1, MDL_PACK_ALG1, nullptr) == MDL_EINVAL);
    int32_t hb = 1 << 16, wb = 1 << 16;
    EXPECT(mdl_pack(&hb, &wb, 1, 8, 1, MDL_PACK_ALG1, &L) == MDL_EOVERFLOW);
    EXPECT(mdl_layout_info(nullptr, nullptr) == MDL_EINVAL);
    EXPECT(mdl_pack(&h1, &w1, 1, 8, 1, MDL_PACK_ALG1, &L) == MDL_OK);
    mdl_layout* L2 = nullptr;
    EXPECT(mdl_pack_level(L, 0, 4, 8, 1, MDL_PACK_ALG1, &L2) == MDL_EINVAL && L2 == nullptr);
    EXPECT(mdl_pack_level(nullptr, 2, 4, 8, 1, MDL_PACK_ALG1, &L2) == MDL_EINVAL);
    // device entry points: the checks that run before any launch
    void* fake = reinterpret_cast<void*>(uintptr_t(1) << 20);
    float* ff = static_cast<float*>(fake);
    const int M0 = MDL_CELL_MDLSTM, M1 = MDL_CELL_LEAKY_LP;
    EXPECT(mdl_forward(L, fake, fake, MDL_F32, 0, 16, M0, ff, ff, ff, ff, nullptr, nullptr, ff, fake, 1 << 20, nullptr) ==
           MDL_EINVAL);
    EXPECT(mdl_forward(L, fake, fake, 7, 4, 16, M0, ff, ff, ff, ff, nullptr, nullptr, ff, fake, 1 << 20, nullptr) ==
           MDL_EINVAL);
    EXPECT(mdl_forward(L, fake, fake, MDL_F32, 4, 16, M0, ff, ff, ff, ff, nullptr, nullptr, ff, fake, 16, nullptr) ==
           MDL_ESIZE);
    EXPECT(mdl_forward(L, fake, fake, MDL_F32, 4, 16, M1, ff, ff, ff, ff, nullptr, nullptr, ff, fake, 1 << 20, nullptr) ==
           MDL_EINVAL);  // Leaky LP without its projections
    EXPECT(mdl_forward(L, fake, fake, MDL_F32, 4, 16, 9, ff, ff, ff, ff, nullptr, nullptr, ff, fake, 1 << 20, nullptr) ==
           MDL_EINVAL);  // unknown cell
    EXPECT(mdl_backward(L, fake, fake, MDL_F32, 4, 16, M0, ff, ff, ff, nullptr, nullptr, ff, ff, ff, ff, nullptr, ff, ff,
                        ff, ff, nullptr, nullptr, fake, 1 << 20, nullptr) == MDL_EINVAL);  // dy_flat and dh_dirs both
    EXPECT(mdl_backward(L, fake, fake, MDL_F32, 4, 16, M1, ff, ff, ff, ff, ff, ff, ff, nullptr, ff, nullptr, ff, ff,
                        ff, ff, nullptr, nullptr, fake, 1 << 20, nullptr) == MDL_EINVAL);  // Leaky LP without dV
    mdl_layout_free(L);
    int32_t hl = 64, wl = 70000;
    EXPECT(mdl_pack(&hl, &wl, 1, 70000, 1, MDL_PACK_ALG1, &L) == MDL_OK);
    EXPECT(mdl_forward(L, fake, fake, MDL_F32, 4, 16, MDL_CELL_MDLSTM, ff, ff, ff, ff, nullptr, nullptr, ff, fake,
                       size_t(1) << 62, nullptr) == MDL_EUNSUPPORTED);
    mdl_layout_free(L);
    mdl_layout_free(nullptr);
    // the timing hooks with nothing recorded
    int32_t count = -1;
    EXPECT(mdl_timing_report(0, nullptr, nullptr, nullptr, &count) == MDL_OK && count == 0);
    EXPECT(mdl_timing_only(nullptr) == MDL_OK);
    EXPECT(mdl_last_error() != nullptr);
    std::printf("host driver: %d failures\n", g_bad);
    return g_bad == 0 ? 0 : 1;
}
