// Explicit instantiations of the normalized variant's backward kernels (the
// parts around the plain backward, on fp32 operands), every (d_k, d_v).
#include "norm_bwd_impl.hpp"

namespace la {

#define LA_NORM_PRE(TI, DK, DV) template hipError_t launch_norm_bwd_pre<TI, DK, DV>(const NormArgs &, hipStream_t);
#define LA_NORM_DK(TI, DK) LA_NORM_PRE(TI, DK, 32) LA_NORM_PRE(TI, DK, 64) LA_NORM_PRE(TI, DK, 128) \
    template hipError_t launch_norm_bwd_post<TI, DK>(const NormArgs &, hipStream_t);
LA_NORM_DK(float, 32)
LA_NORM_DK(float, 64)
LA_NORM_DK(float, 128)
#undef LA_NORM_DK
#undef LA_NORM_PRE

}  // namespace la
