// Explicit instantiations of the serial chunk pass of the gated delta rule for
// bf16 inputs (fp32 or bf16 output).
#include "gdn_fwd_impl.hpp"

namespace la {

template hipError_t launch_gdn_fwd<float, 32>(const ChunkArgs &, hipStream_t);
template hipError_t launch_gdn_fwd<float, 64>(const ChunkArgs &, hipStream_t);
template hipError_t launch_gdn_fwd<float, 128>(const ChunkArgs &, hipStream_t);
template hipError_t launch_gdn_fwd<bf16, 32>(const ChunkArgs &, hipStream_t);
template hipError_t launch_gdn_fwd<bf16, 64>(const ChunkArgs &, hipStream_t);
template hipError_t launch_gdn_fwd<bf16, 128>(const ChunkArgs &, hipStream_t);

}  // namespace la
