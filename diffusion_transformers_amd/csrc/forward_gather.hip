// forward_gather.hip -- the forward with the relative-position bias on grids whose width is not a
// multiple of 16 ("BinaryAttention" paper notes, CVPR 2026, Method details, key design 2): the
// head-resident and streaming kernels of tile.h / stream.h with each key's table offset gathered
// from LDS (bias kind RELPOS_G).  A translation unit of its own so that the build compiles it in
// parallel with forward.hip.
#include "stream.h"

namespace binattn {

hipError_t launch_forward_gather(const FwdArgs& a, hipStream_t s) {
    switch ((a.d + 15) / 16) {
        case 1: launch_fwd_bk<1, BK_RELPOS_G>(a, s); break;
        case 2: launch_fwd_bk<2, BK_RELPOS_G>(a, s); break;
        case 3: launch_fwd_bk<3, BK_RELPOS_G>(a, s); break;
        case 4: launch_fwd_bk<4, BK_RELPOS_G>(a, s); break;
        case 5: launch_fwd_bk<5, BK_RELPOS_G>(a, s); break;
        case 6: launch_fwd_bk<6, BK_RELPOS_G>(a, s); break;
        case 7: launch_fwd_bk<7, BK_RELPOS_G>(a, s); break;
        default: launch_fwd_bk<8, BK_RELPOS_G>(a, s); break;
    }
    return hipGetLastError();
}

}  // namespace binattn
