// kernels_bf16_bf16.hip -- explicit instantiations: bf16 inputs, bf16 outputs.
#include "chunk_fwd_impl.hpp"
#include "decode_impl.hpp"
#include "gdn_prep_impl.hpp"

namespace la {

#define LA_CHUNK(VAR, DK, C) template hipError_t launch_chunk<VAR, bf16, bf16, DK, kDVT, C>(const ChunkArgs &, hipStream_t);
#define LA_CHUNK_ALL_C(VAR, DK) LA_CHUNK(VAR, DK, 64) LA_CHUNK(VAR, DK, 128)
#define LA_CHUNK_VARS(DK) LA_CHUNK_ALL_C(V_PLAIN, DK) LA_CHUNK_ALL_C(V_NORM, DK) LA_CHUNK_ALL_C(V_DECAY, DK) LA_CHUNK(V_GDN, DK, 64)
LA_CHUNK_VARS(32)
LA_CHUNK_VARS(64)
LA_CHUNK_VARS(128)

#define LA_DEC(VAR, DK, DV) template hipError_t launch_decode<VAR, bf16, bf16, DK, DV>(const DecodeArgs &, hipStream_t);
#define LA_DEC_DV(VAR, DK) LA_DEC(VAR, DK, 32) LA_DEC(VAR, DK, 64) LA_DEC(VAR, DK, 128)
#define LA_DEC_ALL(VAR) LA_DEC_DV(VAR, 32) LA_DEC_DV(VAR, 64) LA_DEC_DV(VAR, 128)
LA_DEC_ALL(V_PLAIN)
LA_DEC_ALL(V_DECAY)

}  // namespace la
