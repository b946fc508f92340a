// Explicit instantiations for Kimi Delta Attention: the chunk-parallel
// preparation (bf16 inputs) and the decode step (every dtype pair). The serial
// pass is the delta rule's (kernels_gdn.hip).
#include "decode_impl.hpp"
#include "kda_prep_impl.hpp"

namespace la {

template hipError_t launch_kda_prep<32>(const PrepArgs &, hipStream_t);
template hipError_t launch_kda_prep<64>(const PrepArgs &, hipStream_t);
template hipError_t launch_kda_prep<128>(const PrepArgs &, hipStream_t);

#define LA_KDA_DEC(TI, TO)                                                                  \
    template hipError_t launch_decode<V_KDA, TI, TO, 32, 32>(const DecodeArgs &, hipStream_t);  \
    template hipError_t launch_decode<V_KDA, TI, TO, 32, 64>(const DecodeArgs &, hipStream_t);  \
    template hipError_t launch_decode<V_KDA, TI, TO, 32, 128>(const DecodeArgs &, hipStream_t); \
    template hipError_t launch_decode<V_KDA, TI, TO, 64, 32>(const DecodeArgs &, hipStream_t);  \
    template hipError_t launch_decode<V_KDA, TI, TO, 64, 64>(const DecodeArgs &, hipStream_t);  \
    template hipError_t launch_decode<V_KDA, TI, TO, 64, 128>(const DecodeArgs &, hipStream_t); \
    template hipError_t launch_decode<V_KDA, TI, TO, 128, 32>(const DecodeArgs &, hipStream_t); \
    template hipError_t launch_decode<V_KDA, TI, TO, 128, 64>(const DecodeArgs &, hipStream_t); \
    template hipError_t launch_decode<V_KDA, TI, TO, 128, 128>(const DecodeArgs &, hipStream_t);
LA_KDA_DEC(bf16, bf16)
LA_KDA_DEC(bf16, float)
LA_KDA_DEC(float, float)
#undef LA_KDA_DEC

}  // namespace la
