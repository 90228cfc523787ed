// attention.hip -- the whole BinaryAttention forward from fp16 Q, K, V in one kernel for short
// rows ("BinaryAttention" paper notes, CVPR 2026, Method details, key designs 1-3 and the
// hardware-implementation bullet): the short-row kernel stages K bits, mu_k and int8 V^ of its
// head and the sign words and mu_q of its queries itself (fused_stage), then runs the same
// two-pass exact-max tile loop as the forward from packed inputs.
#include "tile.h"

namespace binattn {

template <int NT, int BK>
static hipError_t launch_fused_bk(const FwdArgs& a, hipStream_t s) {
    launch_keep<NT, BK, true>(a, s);
    return hipGetLastError();
}

template <int NT>
static hipError_t launch_fused_nt(const FwdArgs& a, int bk, hipStream_t s) {
    switch (bk) {
        case BK_NONE: return launch_fused_bk<NT, BK_NONE>(a, s);
        case BK_DENSE_F16: return launch_fused_bk<NT, BK_DENSE_F16>(a, s);
        case BK_DENSE_F32: return launch_fused_bk<NT, BK_DENSE_F32>(a, s);
        default: return launch_fused_bk<NT, BK_RELPOS>(a, s);
    }
}

bool attention_fused_applies(const FwdArgs& a, int bias_kind) {
    const int ntiles = (a.N + kBC - 1) / kBC;
    if (ntiles > kKeepTiles || (bias_kind == 2 && !keep_window_fits(a))) return false;
    if (bias_kind == 2 && relpos_kind(a.gw) == BK_RELPOS_G) return false;  // gathered grids: two launches
    const int nt = (a.d + 15) / 16;
    return nt == 4 || nt == 5 || nt == 8;
}

hipError_t launch_attention_fused(const FwdArgs& a, int bias_kind, hipStream_t s) {
    if (!attention_fused_applies(a, bias_kind)) return hipErrorNotSupported;
    int bk = BK_NONE;
    if (bias_kind == 1) bk = a.bias_f32 ? BK_DENSE_F32 : BK_DENSE_F16;
    if (bias_kind == 2) bk = BK_RELPOS;
    // head dims of the pages' workloads (64, 72) and the widest supported (128)
    switch ((a.d + 15) / 16) {
        case 4: return launch_fused_nt<4>(a, bk, s);
        case 5: return launch_fused_nt<5>(a, bk, s);
        case 8: return launch_fused_nt<8>(a, bk, s);
        default: return hipErrorNotSupported;
    }
}

}  // namespace binattn
