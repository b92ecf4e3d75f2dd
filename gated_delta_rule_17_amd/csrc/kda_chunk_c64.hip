// Chunkwise KDA forward: the kernels for chunk length 64, every (Dk, Dv)
// and operand type (one translation unit per chunk length, so that the
// instantiations compile in parallel).
#include "kda_chunk.hpp"

namespace kda {

hipError_t launch_chunk_c64(const ChunkArgs& a, hipStream_t s)
{
#define KDA_CASE(CC, DK, DV) \
    if (a.Dk == DK && a.Dv == DV) \
        return a.dtype == KDA_BF16 ? launch3<CC, DK, DV, bf16_t>(a, s) : launch3<CC, DK, DV, float>(a, s);
    KDA_FOR_DKDV(KDA_CASE, 64)
#undef KDA_CASE
    return hipErrorInvalidValue;
}

size_t records_bytes_c64(size_t nrec, int Dk, int Dv, kda_dtype dtype)
{
#define KDA_CASE(CC, DK, DV) \
    if (Dk == DK && Dv == DV) \
        return dtype == KDA_BF16 ? records_bytes<CC, DK, DV, bf16_t>(nrec) : records_bytes<CC, DK, DV, float>(nrec);
    KDA_FOR_DKDV(KDA_CASE, 64)
#undef KDA_CASE
    return 0;
}

}  // namespace kda
