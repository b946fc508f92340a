// kernels_f32_f32.hip -- explicit instantiations: float inputs, float outputs.
#include "chunk_fwd_impl.hpp"
#include "decode_impl.hpp"
#include "gdn_prep_impl.hpp"

namespace la {

#define LA_CHUNK(VAR, DK, C) template hipError_t launch_chunk<VAR, float, float, DK, kDVT, C>(const ChunkArgs &, hipStream_t);
#define LA_CHUNK_ALL_C(VAR, DK) LA_CHUNK(VAR, DK, 64) LA_CHUNK(VAR, DK, 128)
#define LA_CHUNK_VARS(DK) LA_CHUNK_ALL_C(V_PLAIN, DK) LA_CHUNK_ALL_C(V_NORM, DK) LA_CHUNK_ALL_C(V_DECAY, DK) LA_CHUNK(V_GDN, DK, 64)
LA_CHUNK_VARS(32)
LA_CHUNK_VARS(64)
// fp32 tiles at d_k = 128 with C = 128 exceed the 160 KiB of LDS: C = 64 only.
LA_CHUNK(V_PLAIN, 128, 64) LA_CHUNK(V_NORM, 128, 64) LA_CHUNK(V_DECAY, 128, 64) LA_CHUNK(V_GDN, 128, 64)

#define LA_DEC(VAR, DK, DV) template hipError_t launch_decode<VAR, float, float, DK, DV>(const DecodeArgs &, hipStream_t);
#define LA_DEC_DV(VAR, DK) LA_DEC(VAR, DK, 32) LA_DEC(VAR, DK, 64) LA_DEC(VAR, DK, 128)
#define LA_DEC_ALL(VAR) LA_DEC_DV(VAR, 32) LA_DEC_DV(VAR, 64) LA_DEC_DV(VAR, 128)
LA_DEC_ALL(V_PLAIN)
LA_DEC_ALL(V_DECAY)

template hipError_t launch_gdn_prep<float, 32, 64>(const PrepArgs &, hipStream_t);
template hipError_t launch_gdn_prep<float, 64, 64>(const PrepArgs &, hipStream_t);
template hipError_t launch_gdn_prep<float, 128, 64>(const PrepArgs &, hipStream_t);

}  // namespace la
