// Explicit instantiations of the backward pass of the gated delta rule (bf16
// inputs), every (d_k, d_v) pair.
#include "gdn_bwd_impl.hpp"

namespace la {

#define LA_GDN_BWD(DK, DV) template hipError_t launch_gdn_bwd<DK, DV>(const BwdArgs &, hipStream_t);
LA_GDN_BWD(32, 32)
LA_GDN_BWD(32, 64)
LA_GDN_BWD(32, 128)
LA_GDN_BWD(64, 32)
LA_GDN_BWD(64, 64)
LA_GDN_BWD(64, 128)
LA_GDN_BWD(128, 32)
LA_GDN_BWD(128, 64)
LA_GDN_BWD(128, 128)
#undef LA_GDN_BWD

}  // namespace la
