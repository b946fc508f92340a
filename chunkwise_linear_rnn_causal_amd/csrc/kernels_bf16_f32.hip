// kernels_bf16_f32.hip -- explicit instantiations: bf16 inputs, float outputs.
#include "chunk_fwd_impl.hpp"
#include "decode_impl.hpp"
#include "gdn_prep_impl.hpp"
#include "vdecay_fwd_impl.hpp"
#include "bwd_impl.hpp"

namespace la {

// chunk forward: (variant, d_k, value columns per workgroup, chunk, waves)
template hipError_t launch_chunk<V_PLAIN, bf16, float, 32, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, float, 32, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, float, 32, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, float, 32, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, float, 32, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, float, 32, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, float, 32, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, float, 32, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, float, 32, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, float, 64, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, float, 64, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, float, 64, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, float, 64, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, float, 64, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, float, 64, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, float, 64, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, float, 64, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, float, 64, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, float, 128, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, float, 128, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, float, 128, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, float, 128, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, float, 128, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, float, 128, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, float, 128, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, float, 128, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, float, 128, 32, 128, 4>(const ChunkArgs &, hipStream_t);

// decode step: (variant, d_k, d_v)
template hipError_t launch_decode<V_PLAIN, bf16, float, 32, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, float, 32, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, float, 32, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, float, 64, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, float, 64, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, float, 64, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, float, 128, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, float, 128, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, float, 128, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, float, 32, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, float, 32, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, float, 32, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, float, 32, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, float, 32, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, float, 32, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, float, 64, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, float, 64, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, float, 64, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, float, 64, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, float, 64, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, float, 64, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, float, 128, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, float, 128, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, float, 128, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, float, 128, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, float, 128, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, float, 128, 128>(const DecodeArgs &, hipStream_t);

// delta-rule chunk preparation: (d_k, chunk)
template hipError_t launch_gdn_prep<bf16, 32, 64>(const PrepArgs &, hipStream_t);
template hipError_t launch_gdn_prep<bf16, 64, 64>(const PrepArgs &, hipStream_t);
template hipError_t launch_gdn_prep<bf16, 128, 64>(const PrepArgs &, hipStream_t);


// per-key-channel decay: (input, output, d_k)
template hipError_t launch_vdecay<bf16, float, 32>(const ChunkArgs &, hipStream_t);
template hipError_t launch_vdecay<bf16, float, 64>(const ChunkArgs &, hipStream_t);
template hipError_t launch_vdecay<bf16, float, 128>(const ChunkArgs &, hipStream_t);

// per-key-channel decay decode step
template hipError_t launch_decode<V_VDECAY, bf16, float, 32, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, float, 32, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, float, 32, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, float, 64, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, float, 64, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, float, 64, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, float, 128, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, float, 128, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, float, 128, 128>(const DecodeArgs &, hipStream_t);


// backward: (input, d_k, d_v, decayed)
template hipError_t launch_bwd<bf16, 32, 32, false>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 32, 32, true>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 32, 64, false>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 32, 64, true>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 32, 128, false>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 32, 128, true>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 64, 32, false>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 64, 32, true>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 64, 64, false>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 64, 64, true>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 64, 128, false>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 64, 128, true>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 128, 32, false>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 128, 32, true>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 128, 64, false>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 128, 64, true>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 128, 128, false>(const BwdArgs &, hipStream_t);
template hipError_t launch_bwd<bf16, 128, 128, true>(const BwdArgs &, hipStream_t);

}  // namespace la
