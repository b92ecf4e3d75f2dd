// Gradient of the chunkwise form: the kernels for chunk length 32, every
// (Dk, Dv) and operand type (one translation unit per chunk length, so that
// the instantiations compile in parallel).
#include "kda_bwd.hpp"

namespace kda {

hipError_t launch_bwd_c32(const bwd::Args& a, int Dk, int Dv, kda_dtype dtype, hipStream_t s)
{
#define KDA_BWD_CASE(CC, DK, DV) \
    if (Dk == DK && Dv == DV) \
        return dtype == KDA_BF16 ? bwd::launch3<CC, DK, DV, bf16_t>(a, s) : bwd::launch3<CC, DK, DV, float>(a, s);
    KDA_BWD_CASES(32)
#undef KDA_BWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
