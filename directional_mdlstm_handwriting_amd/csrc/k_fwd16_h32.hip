// k_fwd16_h32.hip — the forward wavefront at hidden size 32 with two cell groups (kernel in k_fwd16.h).
// Built without the ordinary-register form of the matrix-core accumulators that k_fwd16.hip uses: with 16
// cells per wave this shape needs more than 256 registers per lane, which only the accumulation registers
// provide without spilling.
#include "k_fwd16.h"

namespace mdl {
namespace f16k {

const F16Entry* f16_entries_h32(int& n) {
    static const F16Entry k[] = {MDL_F16(32, 1, false, 2), MDL_F16(32, 1, true, 2)};
    n = 2;
    return k;
}

}  // namespace f16k
}  // namespace mdl
