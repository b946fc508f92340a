// la_kernels.hpp -- argument blocks and launcher templates of the gfx950 kernels.
// Launchers are explicitly instantiated in the per-dtype translation units and
// called by the C ABI layer (abi.hip) after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace la {

// One chunkwise forward pass. Pointers are device pointers; sizes are validated.
struct ChunkArgs {
    const void *q, *k, *v;      // [BH, L, DK], [BH, L, DK], [BH, L, dv]
    const float *lg;            // [BH, L] log-gates ([BH, L, DK] per key channel) or nullptr
    const float *s_in;          // [BH, DK, dv] or nullptr
    const float *z_in;          // [BH, DK] or nullptr (normalized only)
    void *o;                    // [BH, L, dv]
    float *s_out;               // [BH, DK, dv] or nullptr
    float *z_out;               // [BH, DK] or nullptr (normalized only)
    const void *w;              // gated delta: W  [BH, Lp, DK] (operand type)
    const void *ut;             // gated delta: U~ [BH, Lp, dv] (operand type)
    const void *mf;             // gated delta, bf16: masked decayed score fragments
                                // [BH, Lp / 64, 6, 64, 8] fp16 (gdn_prep_impl.hpp)
    float *den_out;             // normalized: the per-token denominators [BH, L] (for the
                                // backward pass) or nullptr
    const void *qc, *kc;        // gated delta, bf16, short convolution fused into the
                                // preparation: convolved q, k [BH, Lp, DK] fp16, or nullptr;
                                // KDA: q (.) Gam and k (.) Gam_C / Gam (kda_prep_impl.hpp)
    const float *cdec;          // KDA: the state's per-channel decay per chunk, Gam_C
                                // [BH, Lp / 64, DK], or nullptr
    int BH, L, Lp, dv, nsplit;  // Lp = ceil(L / C) * C; nsplit = dv / DVT (workgroups per head)
    int ld;                     // rows between consecutive heads of q, k, v, o and the gates
                                // (>= L; L unless a piece of a longer sequence is run)
};

// Chunk-parallel preparation of the gated delta rule (one block per chunk).
struct PrepArgs {
    const void *q, *k, *v;      // [BH, L, DK], [BH, L, DK], [BH, L, dv] (q: bf16 inputs only)
    const float *lg, *beta;     // [BH, L] (lg may be nullptr)
    void *w, *ut, *mf;          // outputs, layouts as in ChunkArgs (mf: bf16 inputs only)
    void *t;                    // backward preparation only: T = (I + P)^-1 [BH, nchunks, C, C]
    // short causal convolution fused into the preparation (bf16 inputs, forward):
    // q, k, v are the raw inputs, convolved here with taps cw [H, d, K] (fp32) and
    // the windows cwin [BH, K - 1, d] (bf16, nullptr = zeros) of the inputs before
    // the sequence; the convolved q and k go to qc, kc [BH, Lp, DK] (fp16)
    const float *cw[3];
    const void *cwin[3];
    void *qc, *kc;
    int H, K;
    float *cdec;                // KDA preparation: Gam_C per chunk [BH, nchunks, DK]
    int BH, L, Lp, dv, nchunks;
    int ld;                     // rows between consecutive heads of k, v and the gates (>= L)
};

struct DecodeArgs {
    const void *q, *k, *v;      // [NH, DK], [NH, DK], [NH, DV]
    const float *lg;            // [NH] ([NH, DK] per key channel) or nullptr
    const float *beta;          // [NH] (gated delta rule) or nullptr
    float *S;                   // [NH, DK, DV], updated in place
    void *o;                    // [NH, DV]
    int NH;
};

// Causal depthwise short convolution: up to three tensors (any of q, k, v) in one
// launch; tensor i owns blocks [blk_i, blk_{i+1}).
struct ConvTensor {
    const void *x;              // [BH, L, d] input
    void *y;                    // [BH, L, d] output (same type)
    const void *s_in;           // [BH, K-1, d] incoming window, oldest first, or nullptr (zeros)
    void *s_out;                // [BH, K-1, d] outgoing window or nullptr; may equal s_in
    const float *w;             // [H, d, K] taps, tap tau multiplies x_{t-tau}
    int d;                      // channels, a multiple of 8
};
struct ConvArgs {
    ConvTensor t0, t1, t2;
    unsigned blk1, blk2;        // first block of tensors 1 and 2 (unused ones: past the grid)
    int BH, H, L, NT;           // NT = max(1, ceil(L / TT)) token tiles
    int ldx;                    // rows between consecutive heads of x (>= L)
};

// Backward pass of the chunk forward (C = 64). Gradients are fp32.
struct BwdArgs {
    const void *q, *k, *v, *dout;  // [BH, L, DK], [BH, L, DK], [BH, L, dv], [BH, L, dv] (input type)
    const float *lg;               // [BH, L] log-gates or nullptr (plain); [BH, L, DK] per channel
    const float *s_in;             // [BH, DK, dv] initial state or nullptr
    const float *ds_out;           // [BH, DK, dv] gradient of the final state or nullptr
    float *gq, *gk, *gv;           // gradients of q, k, v: [BH, L, DK], [BH, L, DK], [BH, L, dv]
    float *glg;                    // gradient of the log-gates (the shape of lg) or nullptr
    float *gs_in;                  // gradient of the initial state [BH, DK, dv] or nullptr
    void *hs, *dhs;                // workspace: per-chunk states / state gradients [BH, nchunks, DK, dv] (operand type)
    float *s_last;                 // workspace: final state [BH, DK, dv]
    float *rterm;                  // workspace: q . dq - k . dk per token [BH, L]
    float *xterm;                  // workspace (scalar decay): <dH_c, H_{c+1}> per chunk [BH, nchunks]
                                   // (gated delta rule: q . dq - v . dv)
    int BH, L, dv, nsplit;
    // gated delta rule only (gdn_bwd_impl.hpp); operand-type (fp16) workspace arrays
    const float *beta;             // [BH, L]
    float *gbeta;                  // gradient of beta [BH, L] or nullptr
    void *w;                       // W [BH, Lp, DK]
    void *u;                       // U~ [BH, Lp, dv], overwritten with U by the forward scan
    void *du;                      // A_m^T dO [BH, Lp, dv], overwritten with dU by the reverse scan
    void *t;                       // T [BH, nchunks, C, C]
    int Lp, nchunks;
    // normalized variant (norm_bwd_impl.hpp): rows of dO scaled by rho [BH, L]
    // (1 / denominator) where the plain kernels stage them, or nullptr
    const float *rho;
};

// TI: input type (bf16 or float); TO: output type (float or bf16); DVT: value
// columns per workgroup; NW: waves per workgroup. The instantiated combinations
// are listed in kernels_*.hip and selected by abi.hip.
template <int VAR, typename TI, typename TO, int DK, int DVT, int C, int NW>
hipError_t launch_chunk(const ChunkArgs &a, hipStream_t st);

template <typename TI, int DK, int C>
hipError_t launch_gdn_prep(const PrepArgs &a, hipStream_t st);

// Serial chunk pass of the gated delta rule for bf16 inputs (C = 64, 16-column
// value slices: a.nsplit = dv / 16), after launch_gdn_prep (which writes a.w,
// a.ut and a.mf).
template <typename TO, int DK>
hipError_t launch_gdn_fwd(const ChunkArgs &a, hipStream_t st);

// Chunk forward with one decay gate per key channel (C = 64, 32-column slices).
template <typename TI, typename TO, int DK>
hipError_t launch_vdecay(const ChunkArgs &a, hipStream_t st);

template <int VAR, typename TI, typename TO, int DK, int DV>
hipError_t launch_decode(const DecodeArgs &a, hipStream_t st);

// Tokens per thread of the short convolution (the host sizes the grid with it).
template <typename T> constexpr int conv_tile() { return sizeof(T) == 2 ? 8 : 4; }

template <typename TI, int DK, int DV, bool DECAY>
hipError_t launch_bwd(const BwdArgs &a, hipStream_t st);

// Backward pass of the gated delta rule, bf16 inputs (C = 64): preparation,
// A_m^T dO, the forward and reverse state scans, the per-chunk gradients and the
// log-gate gradient (gdn_bwd_impl.hpp).
template <int DK, int DV>
hipError_t launch_gdn_bwd(const BwdArgs &a, hipStream_t st);

// Chunk-parallel preparation of Kimi Delta Attention, bf16 inputs (C = 64): W, U~,
// the score fragments, the pre-scaled q and k and the per-chunk state decay, for
// the delta rule's serial pass (kda_prep_impl.hpp). PrepArgs::lg is [BH, L, DK].
template <int DK>
hipError_t launch_kda_prep(const PrepArgs &a, hipStream_t st);

// Backward pass of the per-key-channel decay, bf16 inputs (C = 64): the forward
// and reverse state scans, then the per-chunk gradients with the gate gradient
// (vdecay_bwd_impl.hpp). BwdArgs::lg and ::glg are [BH, L, DK] there.
template <int DK, int DV>
hipError_t launch_vdecay_bwd(const BwdArgs &a, hipStream_t st);

// Backward pass of the normalized variant around the plain one
// (norm_bwd_impl.hpp): rho, g and the chunk sums before it, the normalizer terms
// after it.
struct NormArgs;
template <typename TI, int DK, int DV>
hipError_t launch_norm_bwd_pre(const NormArgs &a, hipStream_t st);
template <typename TI, int DK>
hipError_t launch_norm_bwd_post(const NormArgs &a, hipStream_t st);

template <typename T, int K>
hipError_t launch_short_conv(const ConvArgs &a, unsigned blocks, hipStream_t st);

}  // namespace la
