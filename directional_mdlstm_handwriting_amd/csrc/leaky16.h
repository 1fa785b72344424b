// leaky16.h — the Leaky-LP wavefronts on the 16-bit matrix instructions (hidden sizes 16 and 32;
// k_leaky16.hip). The launchers of k_leaky.hip take them whenever leaky16_used says they fit.
#pragma once

#include "kernels.h"

namespace mdl {

bool leaky16_used(int H, int Lmax);
size_t leaky16_fwd_lds(int H, int Lmax);
size_t leaky16_bwd_lds(int H, int Lmax);
hipError_t launch_fwd_leaky16(const Dev& D, const void* x_canvas, int dtype, int C, int H, const float* Wx,
                              const float* b, const float* Ul, const float* Uu, const float* Vl, const float* Vu,
                              float* stash, float* h_dirs, hipStream_t st);
// done: NULL, or [4n] flags, each set (release, device scope) once that unit's gate gradients are stored
hipError_t launch_bwd_leaky16(const Dev& D, int H, const float* Ul, const float* Uu, const float* Vl,
                              const float* Vu, const float* stash, const float* dy_flat, const float* dh_dirs,
                              float* dA, int32_t* done, hipStream_t st);

}  // namespace mdl
