// kernels_bf16_bf16.hip -- explicit instantiations: bf16 inputs, bf16 outputs.
#include "chunk_fwd_impl.hpp"
#include "decode_impl.hpp"
#include "gdn_prep_impl.hpp"
#include "vdecay_fwd_impl.hpp"
#include "short_conv_impl.hpp"

namespace la {

// chunk forward: (variant, d_k, value columns per workgroup, chunk, waves)
template hipError_t launch_chunk<V_PLAIN, bf16, bf16, 32, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, bf16, 32, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, bf16, 32, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, bf16, 32, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, bf16, 32, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, bf16, 32, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, bf16, 32, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, bf16, 32, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, bf16, 32, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, bf16, 64, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, bf16, 64, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, bf16, 64, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, bf16, 64, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, bf16, 64, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, bf16, 64, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, bf16, 64, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, bf16, 64, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, bf16, 64, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, bf16, 128, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, bf16, 128, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_PLAIN, bf16, bf16, 128, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, bf16, 128, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, bf16, 128, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_NORM, bf16, bf16, 128, 32, 128, 4>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, bf16, 128, 32, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, bf16, 128, 64, 64, 8>(const ChunkArgs &, hipStream_t);
template hipError_t launch_chunk<V_DECAY, bf16, bf16, 128, 32, 128, 4>(const ChunkArgs &, hipStream_t);

// decode step: (variant, d_k, d_v)
template hipError_t launch_decode<V_PLAIN, bf16, bf16, 32, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, bf16, 32, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, bf16, 32, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, bf16, 64, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, bf16, 64, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, bf16, 64, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, bf16, 128, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, bf16, 128, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_PLAIN, bf16, bf16, 128, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, bf16, 32, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, bf16, 32, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, bf16, 32, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, bf16, 32, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, bf16, 32, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, bf16, 32, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, bf16, 64, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, bf16, 64, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, bf16, 64, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, bf16, 64, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, bf16, 64, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, bf16, 64, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, bf16, 128, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, bf16, 128, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, bf16, 128, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, bf16, 128, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_DECAY, bf16, bf16, 128, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_GDN, bf16, bf16, 128, 128>(const DecodeArgs &, hipStream_t);


// short convolution: (type, taps)
template hipError_t launch_short_conv<bf16, 1>(const ConvArgs &, unsigned, hipStream_t);
template hipError_t launch_short_conv<bf16, 2>(const ConvArgs &, unsigned, hipStream_t);
template hipError_t launch_short_conv<bf16, 3>(const ConvArgs &, unsigned, hipStream_t);
template hipError_t launch_short_conv<bf16, 4>(const ConvArgs &, unsigned, hipStream_t);


// per-key-channel decay: (input, output, d_k)
template hipError_t launch_vdecay<bf16, bf16, 32>(const ChunkArgs &, hipStream_t);
template hipError_t launch_vdecay<bf16, bf16, 64>(const ChunkArgs &, hipStream_t);
template hipError_t launch_vdecay<bf16, bf16, 128>(const ChunkArgs &, hipStream_t);

// per-key-channel decay decode step
template hipError_t launch_decode<V_VDECAY, bf16, bf16, 32, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, bf16, 32, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, bf16, 32, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, bf16, 64, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, bf16, 64, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, bf16, 64, 128>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, bf16, 128, 32>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, bf16, 128, 64>(const DecodeArgs &, hipStream_t);
template hipError_t launch_decode<V_VDECAY, bf16, bf16, 128, 128>(const DecodeArgs &, hipStream_t);

}  // namespace la
