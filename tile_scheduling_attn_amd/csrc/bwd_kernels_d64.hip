// The bf16 main kernels at head dimension 64.  This translation unit is
// compiled with the MFMA results in architectural registers
// (-mllvm -amdgpu-mfma-vgpr-form): at d = 64 a wave's accumulators and
// operands fit in them, so S and dP come out of the matrix core where the
// softmax reads them, without a copy out of the accumulation registers per
// value (measured: 510 -> 423 instructions per sub-step, about 4% faster at
// b4 h16 s2048 causal).  At d = 128 the same form spills, so the other
// instantiations stay in bwd_kernels.hip.
#include "bwd_main.h"

namespace attn {

int launch_main_bf16_d64(const KParams& kp, const BwdLaunch& L, bool causal, bool det, int tile) {
    if (tile == 64) return launch_main_d<bf16, 64, 64>(kp, L, causal, det, false);
    return launch_main_d<bf16, 64, 128>(kp, L, causal, det, false);
}

// 64-row Q tiles against 128-row KV tiles
int launch_main_bf16_d64_rect(const KParams& kp, const BwdLaunch& L, bool causal, bool det) {
    return launch_main_d<bf16, 64, 128, 64>(kp, L, causal, det, false);
}

}  // namespace attn
