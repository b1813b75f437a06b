// prefill_mfma.hip -- bf16 MFMA chunked prefill (in progress).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
size_t prefill_mfma_workspace(int N, long long T_total, int H, int Dk, int Dv, int C) {
    return prefill_f32_workspace(N, T_total, H, Dk, Dv, C);
}
hipError_t launch_prefill_mfma(const PrefillArgs &a) { return launch_prefill_f32(a); }
}  // namespace kda
