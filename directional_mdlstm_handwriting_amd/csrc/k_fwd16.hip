// k_fwd16.hip — the forward wavefront's shapes other than hidden size 32, the shape table and the launcher
// (the kernel itself is in k_fwd16.h).
#include "k_fwd16.h"

namespace mdl {

namespace {

using namespace f16k;

// Each entry's cell-group count CG was measured per shape. Hidden size 16: four groups of waves, one
// block of units each. Hidden size 32: two groups (the other unit, 16 cells per wave: every row of the
// matrix instruction carries a cell) where the widest diagonal has at most 32 cells, else four (eight
// cells per wave, half of each instruction's rows empty, but room for 64 cells).
const F16Entry kF16[] = {MDL_F16(16, 1, false, 4), MDL_F16(16, 1, true, 4), MDL_F16(32, 1, false, 4),
                         MDL_F16(32, 1, true, 4), MDL_F16(50, 5, false, 1)};
#undef MDL_F16

// the first shape of (H, input K steps, input type) whose groups hold the widest diagonal
const F16Entry* f16_entry(int H, int C, int dtype, int Lmax) {
    const int kx = (C + 3) / 4;
    auto fits = [&](const F16Entry& m) {
        return m.H == H && m.KX == kx && m.bf16 == (dtype != 0) && (Lmax + m.CG - 1) / m.CG <= 16;
    };
    int n32 = 0;
    const F16Entry* e32 = f16_entries_h32(n32);
    for (int i = 0; i < n32; ++i)
        if (fits(e32[i])) return &e32[i];
    for (const auto& m : kF16)
        if (fits(m)) return &m;
    return nullptr;
}

size_t f16_lds(const F16Entry& m) {
    const size_t nrw = 16 * (size_t)m.CG + 2;
    return 2 * nrw * (2 * m.HP + 8) * 2 + 2 * nrw * (m.H + 4) * 4;
}

}  // namespace

bool fwd16_supported(int H, int C, int dtype, int Lmax) { return f16_entry(H, C, dtype, Lmax) != nullptr; }

size_t fwd16_lds(int H, int C, int dtype, int Lmax) {
    const F16Entry* m = f16_entry(H, C, dtype, Lmax);
    return m ? f16_lds(*m) : 0;
}

hipError_t launch_fwd16(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                        const float* b, const float* Ul, const float* Uu, float* stash, float* h_dirs,
                        int32_t* done, hipStream_t st) {
    const F16Entry* m = f16_entry(H, C, dtype, D.max_diag);
    if (!m) return hipErrorInvalidValue;
    const int cells = (D.max_diag + m->CG - 1) / m->CG;  // widest diagonal's cells per group, <= 16
    const int nr = (cells + 3) / 4;
    launch(m->fwd[nr - 1], dim3(4 * D.n), dim3(64 * m->NB * m->CG), f16_lds(*m), st, D, x_canvas, C, Wx,
           b, Ul, Uu, stash, h_dirs, done);
    return hipGetLastError();
}

}  // namespace mdl
