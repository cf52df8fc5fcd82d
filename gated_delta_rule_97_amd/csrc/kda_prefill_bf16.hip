// bf16 instances of the chunked prefill kernels.
#include "kda_prefill_impl.h"

namespace kda {

template <int DK, int DV, int C>
static hipError_t pick_bv(const PrefillArgs &a, int bv, hipStream_t s) {
    if (bv == 16) return launch_prefill_instance<bf16, DK, DV, C, 16>(a, s);
    return launch_prefill_instance<bf16, DK, DV, C, 32>(a, s);
}

hipError_t launch_prefill_bf16(const PrefillArgs &a, int dk, int dv, int C, int bv, hipStream_t s) {
#define KDA_PF(DK_, DV_)                                             \
    if (dk == DK_ && dv == DV_) {                                    \
        if (C == 16) return pick_bv<DK_, DV_, 16>(a, bv, s);         \
        if (C == 64) return pick_bv<DK_, DV_, 64>(a, bv, s);         \
    }
    KDA_PF(32, 32) KDA_PF(32, 64) KDA_PF(32, 128)
    KDA_PF(64, 32) KDA_PF(64, 64) KDA_PF(64, 128)
    KDA_PF(128, 32) KDA_PF(128, 64) KDA_PF(128, 128)
#undef KDA_PF
    return hipErrorInvalidValue;
}

}  // namespace kda
