// fp32 instances of the chunked prefill kernels.  With chunk 64 and dk or
// dv = 128 the intra-chunk kernel takes its compact LDS placement.
#include "kda_prefill_impl.h"

namespace kda {

template <int DK, int DV, int C>
static hipError_t pick_bv(const PrefillArgs &a, int bv, hipStream_t s) {
    if (bv == 16) return launch_prefill_instance<float, DK, DV, C, 16>(a, s);
    return launch_prefill_instance<float, DK, DV, C, 32>(a, s);
}

hipError_t launch_prefill_f32(const PrefillArgs &a, int dk, int dv, int C, int bv, hipStream_t s) {
#define KDA_PF16(DK_, DV_) \
    if (dk == DK_ && dv == DV_ && C == 16) return pick_bv<DK_, DV_, 16>(a, bv, s);
#define KDA_PF64(DK_, DV_) \
    if (dk == DK_ && dv == DV_ && C == 64) return pick_bv<DK_, DV_, 64>(a, bv, s);
    KDA_PF16(32, 32) KDA_PF16(32, 64) KDA_PF16(32, 128)
    KDA_PF16(64, 32) KDA_PF16(64, 64) KDA_PF16(64, 128)
    KDA_PF16(128, 32) KDA_PF16(128, 64) KDA_PF16(128, 128)
    KDA_PF64(32, 32) KDA_PF64(32, 64) KDA_PF64(32, 128)
    KDA_PF64(64, 32) KDA_PF64(64, 64) KDA_PF64(64, 128)
    KDA_PF64(128, 32) KDA_PF64(128, 64) KDA_PF64(128, 128)
#undef KDA_PF16
#undef KDA_PF64
    return hipErrorInvalidValue;
}

}  // namespace kda
