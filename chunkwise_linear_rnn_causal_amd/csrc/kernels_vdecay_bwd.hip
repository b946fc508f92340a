// Explicit instantiations of the backward pass of the per-key-channel decay
// (bf16 inputs), every (d_k, d_v) pair.
#include "vdecay_bwd_impl.hpp"

namespace la {

#define LA_VD_BWD(DK, DV) template hipError_t launch_vdecay_bwd<DK, DV>(const BwdArgs &, hipStream_t);
LA_VD_BWD(32, 32)
LA_VD_BWD(32, 64)
LA_VD_BWD(32, 128)
LA_VD_BWD(64, 32)
LA_VD_BWD(64, 64)
LA_VD_BWD(64, 128)
LA_VD_BWD(128, 32)
LA_VD_BWD(128, 64)
LA_VD_BWD(128, 128)
#undef LA_VD_BWD

}  // namespace la
