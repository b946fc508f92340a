// abi.hip -- the C ABI of liblinattn (declared in include/linattn.h).
//
// Every entry point validates all arguments on the host before anything is
// launched, selects the compiled kernel instance for (variant, dtype, d_k, C) and
// launches it asynchronously on the caller's stream. Nothing is allocated here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/linattn.h"
#include "la_common.hpp"
#include "la_kernels.hpp"
#include "norm_bwd_impl.hpp"

using namespace la;

// Scratch of la_chunk_fwd_noalloc: every device that loads the library holds
// one copy until the process ends. Host code uses the address that
// hipGetSymbolAddress returns on the current device, never this name.
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const void *p;
    size_t bytes;
};

bool overlap(Span a, Span b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

la_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return LA_ERR_UNSUPPORTED;
    int st = g_device_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LA_ERR_HIP;
        st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_device_ok[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? LA_OK : LA_ERR_UNSUPPORTED;
}

la_status from_hip(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_HIP; }

size_t elem_size(la_dtype dt) { return dt == LA_BF16 ? 2 : 4; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The kernels address the rows of one head with 32-bit element offsets (a
// 64-bit base per head): every element offset inside a head, up to
// ceil(L / C) * C rows of max(d_k, d_v) elements (per-channel gates: d_k per
// token), must stay below 2^31.
bool head_offsets_fit(int L, int C, int d_k, int d_v) {
    const int64_t Lp = ((int64_t)L + C - 1) / C * C;
    return Lp * (d_k > d_v ? d_k : d_v) <= INT32_MAX;
}

// Shape checks shared by the workspace query and the forward call.
la_status check_chunk_shape(la_variant var, la_dtype dt, int B, int H, int L, int d_k, int d_v,
                            int C) {
    if (var < LA_PLAIN || var > LA_KDA) return LA_ERR_INVALID_ARG;
    if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || L < 0) return LA_ERR_INVALID_ARG;
    if (var == LA_KDA && dt != LA_BF16) return LA_ERR_UNSUPPORTED;  // fp16 serial pass only
    if (d_k != 32 && d_k != 64 && d_k != 128) return LA_ERR_UNSUPPORTED;
    if (d_v < 32 || d_v > 128 || d_v % 32 != 0) return LA_ERR_UNSUPPORTED;
    if (C != 64 && C != 128) return LA_ERR_UNSUPPORTED;
    if (var == LA_VECTOR_DECAY && dt == LA_F32 && d_k == 128) return LA_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    if (BH * (d_v / 16) > INT32_MAX || BH * ((L + C - 1) / C) > INT32_MAX) return LA_ERR_UNSUPPORTED;
    if (!head_offsets_fit(L, C, d_k, d_v)) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

// Chunk length the kernels run for a requested C. The chunk form gives the same
// result for every C (tensorplay "Talk Linear Attention", section 3.3: C sets
// the schedule, not the value). A 128-token chunk of the delta rule, the
// per-key-channel decay, and fp32 inputs with d_k = 128 (whose fp32 tiles do
// not fit in LDS at 128 tokens) runs as two 64-token sub-chunks: for the delta
// rule that is the block forward substitution of the chunk's 128 x 128 UT
// system over its two halves, U_b = T_b (beta V_b - beta a K_b S_0 - P_ba U_a),
// which is what the second sub-chunk evaluates with the state carried from the
// first.
int kernel_chunk(la_variant var, la_dtype dt, int d_k, int C) {
    if (C == 128 && (var == LA_GATED_DELTA || var == LA_KDA || var == LA_VECTOR_DECAY || (dt == LA_F32 && d_k == 128)))
        return 64;
    return C;
}

size_t gdn_w_bytes(la_dtype dt, int64_t BH, int64_t Lp, int d_k) {
    return round_up((size_t)BH * Lp * d_k * elem_size(dt), 256);
}

// U~ bytes, rounded up to 256 like W (the score fragments follow it).
size_t gdn_ut_bytes(la_dtype dt, int64_t BH, int64_t Lp, int d_v) {
    return round_up((size_t)BH * Lp * d_v * elem_size(dt), 256);
}

// Score fragments of the bf16 serial pass: 6 fragments of 64 lanes x 8 fp16
// per 64-token chunk, i.e. 96 bytes per token.
size_t gdn_mf_bytes(la_dtype dt, int64_t BH, int64_t Lp) {
    return dt == LA_BF16 ? (size_t)BH * Lp * 96 : 0;
}

// KDA adds the pre-scaled q and k (fp16 [BH, Lp, d_k] each) and the per-chunk
// state decay (fp32 [BH, Lp / 64, d_k]) after the delta rule's arrays.
size_t kda_qk_bytes(int64_t BH, int64_t Lp, int d_k) { return round_up((size_t)BH * Lp * d_k * 2, 256); }
size_t kda_cdec_bytes(int64_t BH, int64_t Lp, int d_k) { return round_up((size_t)BH * (Lp / 64) * d_k * 4, 256); }

size_t chunk_workspace(la_variant var, la_dtype dt, int B, int H, int L, int d_k, int d_v, int C) {
    if ((var != LA_GATED_DELTA && var != LA_KDA) || L == 0) return 0;
    C = kernel_chunk(var, dt, d_k, C);
    const int64_t BH = (int64_t)B * H, Lp = (int64_t)((L + C - 1) / C) * C;
    size_t b = gdn_w_bytes(dt, BH, Lp, d_k) + gdn_ut_bytes(dt, BH, Lp, d_v) + gdn_mf_bytes(dt, BH, Lp);
    if (var == LA_KDA) b += 2 * kda_qk_bytes(BH, Lp, d_k) + kda_cdec_bytes(BH, Lp, d_k);
    return b;
}

// Workgroup geometry of the chunk kernel: value columns per workgroup (DVT) and
// waves per workgroup (NW). fp32 inputs and C = 128 use 4 waves over 32 columns.
// For bf16 inputs and C = 64, 8-wave workgroups (four waves compute the 16-row
// blocks, four stage the tiles and update the state) take 64 columns when that
// still gives at least one
// workgroup per CU (fewer duplicate Q/K loads), else 32. The delta rule, whose
// serial pass is the heaviest, falls back to 16-column workgroups when
// 32-column ones would leave CUs idle.
struct Geometry {
    int dvt, nw;
};
constexpr int kNumCU = 256;

Geometry choose_geometry(la_variant var, la_dtype dt, int64_t BH, int d_v, int C) {
    if (dt == LA_F32 || C == 128) return {32, 4};
    if (var == LA_GATED_DELTA || var == LA_KDA) return {16, 8};  // the chain kernel: 16-column slices
    if (d_v % 64 == 0 && BH * (d_v / 64) >= kNumCU) return {64, 8};
    return {32, 8};
}

template <typename TI, typename TO, int DK, int DVT, int C, int NW>
hipError_t launch_var(la_variant var, const ChunkArgs &a, hipStream_t st) {
    switch (var) {
        case LA_PLAIN: return launch_chunk<V_PLAIN, TI, TO, DK, DVT, C, NW>(a, st);
        case LA_NORMALIZED: return launch_chunk<V_NORM, TI, TO, DK, DVT, C, NW>(a, st);
        case LA_DECAY: return launch_chunk<V_DECAY, TI, TO, DK, DVT, C, NW>(a, st);
        default: break;
    }
    return hipErrorInvalidValue;
}

template <typename TI, typename TO, int DK>
hipError_t dispatch_chunk(la_variant var, int C, Geometry geo, const ChunkArgs &a, hipStream_t st) {
    constexpr bool F32 = sizeof(TI) == 4;
    if (var == LA_GATED_DELTA) {
        if constexpr (F32) return launch_chunk<V_GDN, TI, TO, DK, 32, 64, 4>(a, st);
        if constexpr (!F32) return launch_gdn_fwd<TO, DK>(a, st);
    }
    if (var == LA_KDA) {  // bf16 only (checked); the prepared q, k and decay are in a
        if constexpr (!F32) return launch_gdn_fwd<TO, DK>(a, st);
        return hipErrorInvalidValue;
    }
    if (C == 128) {
        if constexpr (!(F32 && DK == 128)) return launch_var<TI, TO, DK, 32, 128, 4>(var, a, st);
        return hipErrorInvalidValue;
    }
    if constexpr (F32) return launch_var<TI, TO, DK, 32, 64, 4>(var, a, st);
    if constexpr (!F32) {
        if (geo.dvt == 64) return launch_var<TI, TO, DK, 64, 64, 8>(var, a, st);
        return launch_var<TI, TO, DK, 32, 64, 8>(var, a, st);
    }
    return hipErrorInvalidValue;
}

template <typename TI, typename TO>
hipError_t dispatch_vdecay(int d_k, const ChunkArgs &a, hipStream_t st) {
    switch (d_k) {
        case 32: return launch_vdecay<TI, TO, 32>(a, st);
        case 64: return launch_vdecay<TI, TO, 64>(a, st);
        case 128:
            if constexpr (sizeof(TI) == 2) return launch_vdecay<TI, TO, 128>(a, st);
            break;
    }
    return hipErrorInvalidValue;
}

template <typename TI, typename TO>
hipError_t dispatch_chunk_dk(la_variant var, int d_k, int C, Geometry geo, const ChunkArgs &a,
                             hipStream_t st) {
    switch (d_k) {
        case 32: return dispatch_chunk<TI, TO, 32>(var, C, geo, a, st);
        case 64: return dispatch_chunk<TI, TO, 64>(var, C, geo, a, st);
        case 128: return dispatch_chunk<TI, TO, 128>(var, C, geo, a, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t dispatch_prep(int d_k, const PrepArgs &a, hipStream_t st) {
    switch (d_k) {
        case 32: return launch_gdn_prep<T, 32, 64>(a, st);
        case 64: return launch_gdn_prep<T, 64, 64>(a, st);
        case 128: return launch_gdn_prep<T, 128, 64>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int VAR, typename TI, typename TO, int DK>
hipError_t dispatch_decode_dv(int d_v, const DecodeArgs &a, hipStream_t st) {
    switch (d_v) {
        case 32: return launch_decode<VAR, TI, TO, DK, 32>(a, st);
        case 64: return launch_decode<VAR, TI, TO, DK, 64>(a, st);
        case 128: return launch_decode<VAR, TI, TO, DK, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int VAR, typename TI, typename TO>
hipError_t dispatch_decode(int d_k, int d_v, const DecodeArgs &a, hipStream_t st) {
    switch (d_k) {
        case 32: return dispatch_decode_dv<VAR, TI, TO, 32>(d_v, a, st);
        case 64: return dispatch_decode_dv<VAR, TI, TO, 64>(d_v, a, st);
        case 128: return dispatch_decode_dv<VAR, TI, TO, 128>(d_v, a, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t dispatch_short_conv(int K, const ConvArgs &a, unsigned blocks, hipStream_t st) {
    switch (K) {
        case 1: return launch_short_conv<T, 1>(a, blocks, st);
        case 2: return launch_short_conv<T, 2>(a, blocks, st);
        case 3: return launch_short_conv<T, 3>(a, blocks, st);
        case 4: return launch_short_conv<T, 4>(a, blocks, st);
        default: break;
    }
    return hipErrorInvalidValue;
}

// ---- backward pass
// fp32 inputs keep fp32 operand tiles in LDS; the chunk kernel then fits 160 KB
// only for d_k * d_v <= 4096 or the (32, 128) / (128, 32) shapes.
constexpr int kBwdF32MaxState = 4096;
bool bwd_f32_fits(int d_k, int d_v) { return d_k * d_v <= kBwdF32MaxState || d_k + d_v == 160; }

la_status check_bwd_shape(la_variant var, la_dtype dt, int B, int H, int L, int d_k, int d_v, int C) {
    if (var < LA_PLAIN || var > LA_KDA) return LA_ERR_INVALID_ARG;
    if (var == LA_KDA) return LA_ERR_UNSUPPORTED;  // no KDA backward
    if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || L < 0) return LA_ERR_INVALID_ARG;
    if ((var == LA_GATED_DELTA || var == LA_VECTOR_DECAY) && dt != LA_BF16) return LA_ERR_UNSUPPORTED;
    if (C != 64) return LA_ERR_UNSUPPORTED;
    if ((d_k != 32 && d_k != 64 && d_k != 128) || (d_v != 32 && d_v != 64 && d_v != 128))
        return LA_ERR_UNSUPPORTED;
    // fp32 operand tiles (the normalized variant always computes on them)
    if ((dt == LA_F32 || var == LA_NORMALIZED) && !bwd_f32_fits(d_k, d_v)) return LA_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H, nch = (L + C - 1) / C;
    if (BH * nch > INT32_MAX || BH * 2 > INT32_MAX) return LA_ERR_UNSUPPORTED;
    if (!head_offsets_fit(L, C, d_k, d_v)) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

struct BwdLayout {
    size_t hs, dhs, s_last, rterm, xterm, w, u, du, t, o, den, rho, g, ksum, gqsum, up, total;
};
// Every array starts on a 256-byte boundary. The delta rule adds W [BH, Lp, d_k],
// U~ / U and A_m^T dO / dU [BH, Lp, d_v] and T [BH, nchunks, 64, 64], in fp16.
BwdLayout bwd_layout(la_variant var, la_dtype dt, int64_t BH, int L, int d_k, int d_v) {
    const int64_t nch = (L + 63) / 64, Lp = nch * 64;
    BwdLayout w{};
    const la_dtype in_dt = dt;
    if (var == LA_NORMALIZED) dt = LA_F32;  // states in the fp32 operand precision
    const size_t st = (size_t)BH * nch * d_k * d_v * elem_size(dt);
    w.hs = 0;
    w.dhs = round_up(st, 256);
    w.s_last = w.dhs + round_up(st, 256);
    w.rterm = w.s_last + round_up((size_t)BH * d_k * d_v * 4, 256);
    w.xterm = w.rterm + round_up((size_t)BH * L * 4, 256);
    w.total = w.xterm + round_up((size_t)BH * nch * 4, 256);
    if (var == LA_GATED_DELTA) {
        w.w = w.total;
        w.u = w.w + round_up((size_t)BH * Lp * d_k * 2, 256);
        w.du = w.u + round_up((size_t)BH * Lp * d_v * 2, 256);
        w.t = w.du + round_up((size_t)BH * Lp * d_v * 2, 256);
        w.total = w.t + round_up((size_t)BH * nch * 64 * 64 * 2, 256);
    }
    if (var == LA_NORMALIZED) {  // the forward's output and denominators, rho, g, chunk sums
        const size_t tok = round_up((size_t)BH * L * 4, 256), cs = round_up((size_t)BH * nch * d_k * 4, 256);
        w.o = w.total;
        w.den = w.o + round_up((size_t)BH * L * d_v * 4, 256);
        w.rho = w.den + tok;
        w.g = w.rho + tok;
        w.ksum = w.g + tok;
        w.gqsum = w.ksum + cs;
        w.total = w.gqsum + cs;
        if (in_dt == LA_BF16) {  // fp32 copies of q, k, v and d_o
            const size_t qk = round_up((size_t)BH * L * d_k * 4, 256), vb = round_up((size_t)BH * L * d_v * 4, 256);
            w.up = w.total;
            w.total += 2 * qk + 2 * vb;
        }
    }
    return w;
}

template <typename TI>
hipError_t dispatch_norm_pre(int d_k, int d_v, const NormArgs &a, hipStream_t st) {
#define LA_NORM_DV(DK)                                                   \
    switch (d_v) {                                                       \
        case 32: return launch_norm_bwd_pre<TI, DK, 32>(a, st);          \
        case 64: return launch_norm_bwd_pre<TI, DK, 64>(a, st);          \
        case 128: return launch_norm_bwd_pre<TI, DK, 128>(a, st);        \
    }                                                                    \
    break;
    switch (d_k) {
        case 32: LA_NORM_DV(32)
        case 64: LA_NORM_DV(64)
        case 128: LA_NORM_DV(128)
    }
#undef LA_NORM_DV
    return hipErrorInvalidValue;
}

template <typename TI>
hipError_t dispatch_norm_post(int d_k, const NormArgs &a, hipStream_t st) {
    switch (d_k) {
        case 32: return launch_norm_bwd_post<TI, 32>(a, st);
        case 64: return launch_norm_bwd_post<TI, 64>(a, st);
        case 128: return launch_norm_bwd_post<TI, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t dispatch_vdecay_bwd(int d_k, int d_v, const BwdArgs &a, hipStream_t st) {
#define LA_VD_BWD_DV(DK)                                           \
    switch (d_v) {                                                 \
        case 32: return launch_vdecay_bwd<DK, 32>(a, st);          \
        case 64: return launch_vdecay_bwd<DK, 64>(a, st);          \
        case 128: return launch_vdecay_bwd<DK, 128>(a, st);        \
    }                                                              \
    break;
    switch (d_k) {
        case 32: LA_VD_BWD_DV(32)
        case 64: LA_VD_BWD_DV(64)
        case 128: LA_VD_BWD_DV(128)
    }
#undef LA_VD_BWD_DV
    return hipErrorInvalidValue;
}

hipError_t dispatch_gdn_bwd(int d_k, int d_v, const BwdArgs &a, hipStream_t st) {
#define LA_GDN_BWD_DV(DK)                                          \
    switch (d_v) {                                                 \
        case 32: return launch_gdn_bwd<DK, 32>(a, st);             \
        case 64: return launch_gdn_bwd<DK, 64>(a, st);             \
        case 128: return launch_gdn_bwd<DK, 128>(a, st);           \
    }                                                              \
    break;
    switch (d_k) {
        case 32: LA_GDN_BWD_DV(32)
        case 64: LA_GDN_BWD_DV(64)
        case 128: LA_GDN_BWD_DV(128)
    }
#undef LA_GDN_BWD_DV
    return hipErrorInvalidValue;
}

template <typename TI, bool DECAY>
hipError_t dispatch_bwd(int d_k, int d_v, const BwdArgs &a, hipStream_t st) {
#define LA_BWD_DV(DK)                                                            \
    switch (d_v) {                                                               \
        case 32: return launch_bwd<TI, DK, 32, DECAY>(a, st);                    \
        case 64:                                                                 \
            if constexpr (sizeof(TI) == 2 || DK * 64 <= kBwdF32MaxState)         \
                return launch_bwd<TI, DK, 64, DECAY>(a, st);                     \
            break;                                                               \
        case 128:                                                                \
            if constexpr (sizeof(TI) == 2 || DK * 128 <= kBwdF32MaxState)        \
                return launch_bwd<TI, DK, 128, DECAY>(a, st);                    \
            break;                                                               \
    }                                                                            \
    break;
    switch (d_k) {
        case 32: LA_BWD_DV(32)
        case 64: LA_BWD_DV(64)
        case 128: LA_BWD_DV(128)
    }
#undef LA_BWD_DV
    return hipErrorInvalidValue;
}

// Supported (input, output) dtype pairs: bf16 -> fp32, bf16 -> bf16, fp32 -> fp32.
bool dtype_pair_ok(la_dtype dt, la_dtype o_dt) {
    return (dt == LA_BF16 && (o_dt == LA_F32 || o_dt == LA_BF16)) || (dt == LA_F32 && o_dt == LA_F32);
}

// ---- chunk forward: validation and launch, shared by la_chunk_fwd and
// la_chunk_fwd_noalloc
struct FwdCall {
    la_variant var;
    la_dtype dt, o_dt;
    const void *q, *k, *v;
    const float *log_gate, *beta, *state_in, *z_in;
    void *o;
    float *state_out, *z_out;
    int B, H, L, d_k, d_v, C;
};

struct FwdSpans {
    Span sp[10];
    const Span *begin() const { return sp; }
    const Span *end() const { return sp + 10; }
};
// Every buffer the call reads or writes (for overlap checks against a workspace).
FwdSpans fwd_spans(const FwdCall &f) {
    const int64_t BH = (int64_t)f.B * f.H;
    const size_t es = elem_size(f.dt), g_b = (size_t)BH * f.L * 4;
    const size_t s_b = (size_t)BH * f.d_k * f.d_v * 4, z_b = (size_t)BH * f.d_k * 4;
    return FwdSpans{{{f.q, (size_t)BH * f.L * f.d_k * es}, {f.k, (size_t)BH * f.L * f.d_k * es},
                     {f.v, (size_t)BH * f.L * f.d_v * es},
                     {f.log_gate, (f.var == LA_VECTOR_DECAY || f.var == LA_KDA) ? g_b * f.d_k : g_b}, {f.beta, g_b},
                     {f.o, (size_t)BH * f.L * f.d_v * elem_size(f.o_dt)}, {f.state_in, s_b},
                     {f.state_out, s_b}, {f.z_in, z_b}, {f.z_out, z_b}}};
}

la_status validate_fwd(const FwdCall &f) {
    la_status s = check_chunk_shape(f.var, f.dt, f.B, f.H, f.L, f.d_k, f.d_v, f.C);
    if (s != LA_OK) return s;
    const la_variant var = f.var;
    if (f.o_dt != LA_F32 && f.o_dt != LA_BF16) return LA_ERR_INVALID_ARG;
    if (!dtype_pair_ok(f.dt, f.o_dt)) return LA_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)f.B * f.H;
    const size_t es = elem_size(f.dt), oes = elem_size(f.o_dt);
    const bool has_tokens = f.L > 0;
    // required / forbidden pointers
    if (has_tokens && (!f.q || !f.k || !f.o)) return LA_ERR_INVALID_ARG;
    if (has_tokens && !f.v) return LA_ERR_INVALID_ARG;
    if ((var == LA_DECAY || var == LA_VECTOR_DECAY || var == LA_KDA) && has_tokens && !f.log_gate)
        return LA_ERR_INVALID_ARG;
    if ((var == LA_PLAIN || var == LA_NORMALIZED) && f.log_gate) return LA_ERR_INVALID_ARG;
    const bool delta = var == LA_GATED_DELTA || var == LA_KDA;
    if (delta && has_tokens && !f.beta) return LA_ERR_INVALID_ARG;
    if (!delta && f.beta) return LA_ERR_INVALID_ARG;
    if (var != LA_NORMALIZED && (f.z_in || f.z_out)) return LA_ERR_INVALID_ARG;
    // alignment
    const void *ptrs[] = {f.q, f.k, f.v, f.o, f.log_gate, f.beta, f.state_in, f.z_in, f.state_out, f.z_out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
    // aliasing: outputs must not overlap inputs (state_out == state_in is allowed)
    const int L = f.L, d_k = f.d_k, d_v = f.d_v;
    const size_t qk_b = (size_t)BH * L * d_k * es, v_b = (size_t)BH * L * d_v * es;
    const size_t g_b = (size_t)BH * L * 4, s_b = (size_t)BH * d_k * d_v * 4, z_b = (size_t)BH * d_k * 4;
    const size_t lg_b = (var == LA_VECTOR_DECAY || var == LA_KDA) ? g_b * d_k : g_b;
    const Span o_sp{f.o, (size_t)BH * L * d_v * oes}, so_sp{f.state_out, s_b}, zo_sp{f.z_out, z_b};
    const Span ins[] = {{f.q, qk_b}, {f.k, qk_b}, {f.v, v_b}, {f.log_gate, lg_b}, {f.beta, g_b}, {f.z_in, z_b}};
    for (const Span &in : ins) {
        if (overlap(o_sp, in) || overlap(so_sp, in) || overlap(zo_sp, in)) return LA_ERR_INVALID_ARG;
    }
    if (overlap(o_sp, Span{f.state_in, s_b}) || overlap(o_sp, so_sp) || overlap(o_sp, zo_sp) ||
        overlap(so_sp, zo_sp) || overlap(zo_sp, Span{f.state_in, s_b}))
        return LA_ERR_INVALID_ARG;
    if (f.state_out && f.state_in && f.state_out != f.state_in && overlap(so_sp, Span{f.state_in, s_b}))
        return LA_ERR_INVALID_ARG;
    return LA_OK;
}

// Launch the forward over tokens [p0, p0 + n) of every head (a piece of the
// sequence; the whole sequence when p0 = 0 and n = L): pointers are advanced to
// the piece, heads stay f.L rows apart, the state comes from s_in and goes to
// s_out. ws: the delta rule's per-chunk products for this piece.
// The short convolution fused into the delta rule's preparation: taps, windows
// and the workspace arrays of the convolved q and k.
struct ConvSpec {
    const float *w[3];
    const void *win[3];
    void *qc, *kc;
    int H, K;
};

la_status run_fwd(const FwdCall &f, int p0, int n, const float *s_in, float *s_out, void *ws,
                  hipStream_t st, const ConvSpec *cv = nullptr, float *den_out = nullptr) {
    const la_variant var = f.var;
    const la_dtype dt = f.dt;
    const int64_t BH = (int64_t)f.B * f.H;
    const size_t es = elem_size(dt), oes = elem_size(f.o_dt);
    const int C = kernel_chunk(var, dt, f.d_k, f.C), d_k = f.d_k, d_v = f.d_v;
    const int nchunks = (n + C - 1) / C;
    const int Lp = nchunks * C;
    const int gw = (var == LA_VECTOR_DECAY || var == LA_KDA) ? d_k : 1;  // gates per token
    auto adv = [&](const void *p, size_t per_row) -> const void * {
        return p ? static_cast<const char *>(p) + (size_t)p0 * per_row : nullptr;
    };
    ChunkArgs a{};
    a.q = adv(f.q, d_k * es); a.k = adv(f.k, d_k * es); a.v = adv(f.v, d_v * es);
    a.lg = static_cast<const float *>(adv(f.log_gate, 4 * gw));
    a.s_in = s_in; a.z_in = f.z_in;
    a.o = const_cast<void *>(adv(f.o, d_v * oes));
    a.s_out = s_out; a.z_out = f.z_out;
    a.den_out = den_out ? den_out + p0 : nullptr;
    const Geometry geo = choose_geometry(var, dt, BH, d_v, C);
    a.BH = (int)BH; a.L = n; a.Lp = Lp; a.dv = d_v; a.nsplit = d_v / geo.dvt; a.ld = f.L;

    if (var == LA_KDA && n > 0) {
        // the preparation folds the per-channel gates into W, the scores, q and k
        // and the per-chunk state decay; the serial pass runs without a scalar gate
        char *w = static_cast<char *>(ws);
        const size_t wb = gdn_w_bytes(dt, BH, Lp, d_k), ub = gdn_ut_bytes(dt, BH, Lp, d_v);
        const size_t mb = gdn_mf_bytes(dt, BH, Lp), qkb = kda_qk_bytes(BH, Lp, d_k);
        PrepArgs p{};
        p.q = a.q; p.k = a.k; p.v = a.v; p.lg = a.lg; p.beta = static_cast<const float *>(adv(f.beta, 4));
        p.w = w; p.ut = w + wb; p.mf = w + wb + ub;
        p.qc = w + wb + ub + mb; p.kc = w + wb + ub + mb + qkb;
        p.cdec = reinterpret_cast<float *>(w + wb + ub + mb + 2 * qkb);
        p.BH = (int)BH; p.L = n; p.Lp = Lp; p.dv = d_v; p.nchunks = nchunks; p.ld = f.L;
        hipError_t e = hipErrorInvalidValue;
        switch (d_k) {
            case 32: e = launch_kda_prep<32>(p, st); break;
            case 64: e = launch_kda_prep<64>(p, st); break;
            case 128: e = launch_kda_prep<128>(p, st); break;
        }
        if (e != hipSuccess) return LA_ERR_HIP;
        a.w = p.w; a.ut = p.ut; a.mf = p.mf; a.qc = p.qc; a.kc = p.kc; a.cdec = p.cdec;
        a.lg = nullptr;
    }
    if (var == LA_GATED_DELTA && n > 0) {
        char *w = static_cast<char *>(ws);
        a.w = w;
        a.ut = w + gdn_w_bytes(dt, BH, Lp, d_k);
        a.mf = dt == LA_BF16 ? w + gdn_w_bytes(dt, BH, Lp, d_k) + gdn_ut_bytes(dt, BH, Lp, d_v) : nullptr;
        PrepArgs p{};
        p.q = a.q; p.k = a.k; p.v = a.v; p.lg = a.lg; p.beta = static_cast<const float *>(adv(f.beta, 4));
        p.w = const_cast<void *>(a.w); p.ut = const_cast<void *>(a.ut); p.mf = const_cast<void *>(a.mf);
        p.BH = (int)BH; p.L = n; p.Lp = Lp; p.dv = d_v; p.nchunks = nchunks; p.ld = f.L;
        if (cv) {  // bf16 only (validated by the caller)
            for (int i = 0; i < 3; ++i) {
                p.cw[i] = cv->w[i];
                p.cwin[i] = cv->win[i];
            }
            p.qc = cv->qc; p.kc = cv->kc; p.H = cv->H; p.K = cv->K;
            a.qc = cv->qc; a.kc = cv->kc;
        }
        const hipError_t e = (dt == LA_BF16) ? dispatch_prep<bf16>(d_k, p, st)
                                             : dispatch_prep<float>(d_k, p, st);
        if (e != hipSuccess) return LA_ERR_HIP;
    }
    hipError_t e;
    if (var == LA_VECTOR_DECAY) {  // the launcher picks its own value slices
        if (dt == LA_F32)
            e = dispatch_vdecay<float, float>(d_k, a, st);
        else if (f.o_dt == LA_F32)
            e = dispatch_vdecay<bf16, float>(d_k, a, st);
        else
            e = dispatch_vdecay<bf16, bf16>(d_k, a, st);
        return from_hip(e);
    }
    if (dt == LA_F32)
        e = dispatch_chunk_dk<float, float>(var, d_k, C, geo, a, st);
    else if (f.o_dt == LA_F32)
        e = dispatch_chunk_dk<bf16, float>(var, d_k, C, geo, a, st);
    else
        e = dispatch_chunk_dk<bf16, bf16>(var, d_k, C, geo, a, st);
    return from_hip(e);
}

// ---- la_chunk_fwd_noalloc: the delta rule's per-chunk products (W, U~) live
// in a static device array instead of a caller workspace.
constexpr size_t kScratchBytes = sizeof(scratch);
// Device address of `scratch` per device, from hipGetSymbolAddress on that
// device (the host-side name of the array is not a device address).
std::atomic<char *> g_scratch[kMaxDevices];

la_status scratch_for_current_device(char **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LA_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return LA_ERR_UNSUPPORTED;
    char *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return LA_ERR_HIP;
        p = static_cast<char *>(addr);
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return LA_OK;
}

// Piece length (tokens, a multiple of C) whose delta-rule products fit the
// scratch, with room for a carried state when the caller passes no state_out;
// rows >= L means the whole sequence in one piece, 0 that one chunk does not fit.
struct PiecePlan {
    int rows;
    size_t ws_bytes;  // products of one full piece (the carried state follows them)
};
PiecePlan plan_pieces(const FwdCall &f) {
    const size_t whole = chunk_workspace(f.var, f.dt, f.B, f.H, f.L, f.d_k, f.d_v, f.C);
    if (whole <= kScratchBytes) return PiecePlan{f.L > 0 ? f.L : 1, whole};
    const int64_t BH = (int64_t)f.B * f.H;
    const size_t carry = f.state_out ? 0 : round_up((size_t)BH * f.d_k * f.d_v * 4, 256);
    const size_t per_row = (size_t)BH * ((f.d_k + f.d_v) * elem_size(f.dt) + (f.dt == LA_BF16 ? 96 : 0));
    const int kc = kernel_chunk(f.var, f.dt, f.d_k, f.C);
    if (carry >= kScratchBytes) return PiecePlan{0, 0};
    int64_t rows = (int64_t)((kScratchBytes - carry) / per_row) / kc * kc;
    while (rows >= kc) {
        const size_t ws = chunk_workspace(f.var, f.dt, f.B, f.H, (int)rows, f.d_k, f.d_v, f.C);
        if (ws + carry <= kScratchBytes) return PiecePlan{(int)rows, ws};
        rows -= kc;
    }
    return PiecePlan{0, 0};
}

}  // namespace

extern "C" {

int la_abi_version(void) { return LA_ABI_VERSION; }

const char *la_status_str(la_status s) {
    switch (s) {
        case LA_OK: return "LA_OK";
        case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
        case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
        case LA_ERR_HIP: return "LA_ERR_HIP";
    }
    return "LA_ERR_UNKNOWN";
}

la_status la_chunk_fwd_workspace_size(la_variant var, la_dtype dt, int B, int H, int L, int d_k,
                                      int d_v, int C, size_t *bytes) {
    if (!bytes) return LA_ERR_INVALID_ARG;
    const la_status s = check_chunk_shape(var, dt, B, H, L, d_k, d_v, C);
    if (s != LA_OK) return s;
    *bytes = chunk_workspace(var, dt, B, H, L, d_k, d_v, C);
    return LA_OK;
}

la_status la_chunk_fwd(la_variant var, la_dtype dt, la_dtype o_dt, const void *q, const void *k,
                       const void *v, const float *log_gate, const float *beta,
                       const float *state_in, const float *z_in, void *o, float *state_out,
                       float *z_out, int B, int H, int L, int d_k, int d_v, int C, void *workspace,
                       size_t workspace_bytes, void *stream) {
    const FwdCall f{var, dt, o_dt, q, k, v, log_gate, beta, state_in, z_in, o, state_out, z_out,
                    B, H, L, d_k, d_v, C};
    la_status s = validate_fwd(f);
    if (s != LA_OK) return s;
    const size_t need = chunk_workspace(var, dt, B, H, L, d_k, d_v, C);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return LA_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LA_ERR_INVALID_ARG;
        const Span ws{workspace, need};
        for (const Span &sp : fwd_spans(f))
            if (overlap(ws, sp)) return LA_ERR_INVALID_ARG;
    }
    s = check_device();
    if (s != LA_OK) return s;
    return run_fwd(f, 0, L, state_in, state_out, workspace, reinterpret_cast<hipStream_t>(stream));
}

la_status la_chunk_fwd_noalloc(la_variant var, la_dtype dt, la_dtype o_dt, const void *q,
                               const void *k, const void *v, const float *log_gate,
                               const float *beta, const float *state_in, const float *z_in, void *o,
                               float *state_out, float *z_out, int B, int H, int L, int d_k,
                               int d_v, int C, void *stream) {
    const FwdCall f{var, dt, o_dt, q, k, v, log_gate, beta, state_in, z_in, o, state_out, z_out,
                    B, H, L, d_k, d_v, C};
    la_status s = validate_fwd(f);
    if (s != LA_OK) return s;
    const PiecePlan plan = plan_pieces(f);
    if (plan.rows == 0) return LA_ERR_UNSUPPORTED;  // one chunk of every head exceeds the scratch
    s = check_device();
    if (s != LA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (plan.rows >= L) {  // no workspace needed, or one piece
        char *scr = nullptr;
        if (chunk_workspace(var, dt, B, H, L, d_k, d_v, C) > 0) {
            s = scratch_for_current_device(&scr);
            if (s != LA_OK) return s;
        }
        return run_fwd(f, 0, L, state_in, state_out, scr, st);
    }
    // Pieces of plan.rows tokens (a multiple of C), chained through the fp32
    // state: in state_out when the caller wants it (in place from the second
    // piece on), else in the scratch after the per-chunk products.
    char *scr = nullptr;
    s = scratch_for_current_device(&scr);
    if (s != LA_OK) return s;
    float *carry = state_out ? state_out : reinterpret_cast<float *>(scr + plan.ws_bytes);
    for (int p0 = 0; p0 < L; p0 += plan.rows) {
        const int n = L - p0 < plan.rows ? L - p0 : plan.rows;
        const bool last = p0 + n == L;
        const float *sin = p0 == 0 ? state_in : carry;
        float *sout = last ? state_out : carry;
        s = run_fwd(f, p0, n, sin, sout, scr, st);
        if (s != LA_OK) return s;
    }
    return LA_OK;
}

// ---- la_chunk_fwd_conv: the delta rule with the short convolution fused into
// its preparation. Workspace: la_chunk_fwd's, then the convolved q and k (fp16,
// [BH, Lp, d_k] each), then the discarded outputs of the window update (at most
// 3 rows of q, k, v per head).
size_t conv_fused_workspace(int B, int H, int L, int d_k, int d_v, int C) {
    const int64_t BH = (int64_t)B * H, Lp = (int64_t)((L + 63) / 64) * 64;
    return chunk_workspace(LA_GATED_DELTA, LA_BF16, B, H, L, d_k, d_v, C) +
           2 * round_up((size_t)BH * Lp * d_k * 2, 256) + round_up((size_t)BH * 3 * (2 * d_k + d_v) * 2, 256);
}

la_status check_conv_fused(la_variant var, la_dtype dt, int B, int H, int L, int d_k, int d_v, int C, int K) {
    const la_status s = check_chunk_shape(var, dt, B, H, L, d_k, d_v, C);
    if (s != LA_OK) return s;
    if (K < 1) return LA_ERR_INVALID_ARG;
    if (var != LA_GATED_DELTA || dt != LA_BF16 || K > 4) return LA_ERR_UNSUPPORTED;
    return LA_OK;
}

la_status la_chunk_fwd_conv_workspace_size(la_variant var, la_dtype dt, int B, int H, int L, int d_k,
                                           int d_v, int C, int K, size_t *bytes) {
    if (!bytes) return LA_ERR_INVALID_ARG;
    const la_status s = check_conv_fused(var, dt, B, H, L, d_k, d_v, C, K);
    if (s != LA_OK) return s;
    *bytes = conv_fused_workspace(B, H, L, d_k, d_v, C);
    return LA_OK;
}

la_status la_chunk_fwd_conv(la_variant var, la_dtype dt, la_dtype o_dt, const void *q, const void *k,
                            const void *v, const float *w_q, const float *w_k, const float *w_v, int K,
                            const void *q_win_in, const void *k_win_in, const void *v_win_in,
                            void *q_win_out, void *k_win_out, void *v_win_out, const float *log_gate,
                            const float *beta, const float *state_in, void *o, float *state_out, int B,
                            int H, int L, int d_k, int d_v, int C, void *workspace,
                            size_t workspace_bytes, void *stream) {
    la_status s = check_conv_fused(var, dt, B, H, L, d_k, d_v, C, K);
    if (s != LA_OK) return s;
    const FwdCall f{var, dt, o_dt, q, k, v, log_gate, beta, state_in, nullptr, o, state_out, nullptr,
                    B, H, L, d_k, d_v, C};
    s = validate_fwd(f);
    if (s != LA_OK) return s;
    if (!w_q || !w_k || !w_v) return LA_ERR_INVALID_ARG;
    const int64_t BH = (int64_t)B * H;
    const int d[3] = {d_k, d_k, d_v};
    const float *taps[3] = {w_q, w_k, w_v};
    const void *win_in[3] = {q_win_in, k_win_in, v_win_in};
    void *win_out[3] = {q_win_out, k_win_out, v_win_out};
    const void *ptrs[] = {w_q, w_k, w_v, q_win_in, k_win_in, v_win_in, q_win_out, k_win_out, v_win_out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
    const size_t need = conv_fused_workspace(B, H, L, d_k, d_v, C);
    if (!workspace || workspace_bytes < need) return LA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LA_ERR_INVALID_ARG;
    // aliasing: the workspace and the outgoing windows overlap no other buffer;
    // an outgoing window may equal its own incoming window (updated in place)
    Span in_sp[16], out_sp[4];
    int ni = 0, no = 0;
    for (const Span &sp : fwd_spans(f)) in_sp[ni++] = sp;  // includes o and state_out
    for (int i = 0; i < 3; ++i) {
        const size_t wb = (size_t)BH * (K - 1) * d[i] * 2;
        in_sp[ni++] = Span{taps[i], (size_t)H * d[i] * K * 4};
        if (win_in[i] != win_out[i]) in_sp[ni++] = Span{win_in[i], wb};
        out_sp[no++] = Span{win_out[i], wb};
        if (win_out[i] && win_in[i] && win_out[i] != win_in[i] && overlap(Span{win_out[i], wb}, Span{win_in[i], wb}))
            return LA_ERR_INVALID_ARG;
    }
    out_sp[no++] = Span{workspace, need};
    for (int o2 = 0; o2 < no; ++o2) {
        for (int i = 0; i < ni; ++i)
            if (overlap(out_sp[o2], in_sp[i])) return LA_ERR_INVALID_ARG;
        for (int o3 = o2 + 1; o3 < no; ++o3)
            if (overlap(out_sp[o2], out_sp[o3])) return LA_ERR_INVALID_ARG;
    }
    // the forward's own outputs must not overlap the taps or incoming windows
    const Span fo[] = {{o, (size_t)BH * L * d_v * elem_size(o_dt)}, {state_out, (size_t)BH * d_k * d_v * 4}};
    for (const Span &x : fo)
        for (int i = 0; i < 3; ++i)
            if (overlap(x, Span{taps[i], (size_t)H * d[i] * K * 4}) ||
                overlap(x, Span{win_in[i], (size_t)BH * (K - 1) * d[i] * 2}))
                return LA_ERR_INVALID_ARG;

    s = check_device();
    if (s != LA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(workspace);
    const int64_t Lp = (int64_t)((L + 63) / 64) * 64;
    const size_t base = chunk_workspace(var, dt, B, H, L, d_k, d_v, C);
    const size_t qk = round_up((size_t)BH * Lp * d_k * 2, 256);
    ConvSpec cv{};
    for (int i = 0; i < 3; ++i) {
        cv.w[i] = taps[i];
        cv.win[i] = K > 1 ? win_in[i] : nullptr;
    }
    cv.qc = w + base; cv.kc = w + base + qk; cv.H = H; cv.K = K;
    s = run_fwd(f, 0, L, state_in, state_out, workspace, st, &cv);
    if (s != LA_OK) return s;
    // outgoing windows: the short convolution kernel over the last min(L, K - 1)
    // tokens (the incoming window as well when L < K - 1); its outputs are dropped
    if (K > 1 && (q_win_out || k_win_out || v_win_out)) {
        const int n = L < K - 1 ? L : K - 1;
        char *ydrop = w + base + 2 * qk;
        ConvArgs a{};
        ConvTensor *slots[3] = {&a.t0, &a.t1, &a.t2};
        const void *xs[3] = {q, k, v};
        int nt = 0;
        int64_t blk[3] = {0, 0, 0}, total = 0;
        const int tt = conv_tile<bf16>();
        const int64_t NT = n > 0 ? ((int64_t)n + tt - 1) / tt : 1;
        size_t yoff = 0;
        for (int i = 0; i < 3; ++i) {
            if (!win_out[i]) continue;
            const void *x = xs[i] ? static_cast<const char *>(xs[i]) + (size_t)(L - n) * d[i] * 2 : nullptr;
            *slots[nt] = ConvTensor{x, ydrop + yoff, n < K - 1 ? win_in[i] : nullptr, win_out[i], taps[i], d[i]};
            yoff += (size_t)BH * 3 * d[i] * 2;
            blk[nt] = (BH * NT * (d[i] / 8) + 255) / 256;
            total += blk[nt];
            ++nt;
        }
        a.blk1 = (unsigned)(nt > 1 ? blk[0] : total);
        a.blk2 = (unsigned)(nt > 2 ? blk[0] + blk[1] : total);
        a.BH = (int)BH; a.H = H; a.L = n; a.NT = (int)NT; a.ldx = L;
        if (dispatch_short_conv<bf16>(K, a, (unsigned)total, st) != hipSuccess) return LA_ERR_HIP;
    }
    return LA_OK;
}

la_status la_decode_step(la_variant var, la_dtype dt, la_dtype o_dt, const void *q, const void *k,
                         const void *v, const float *log_gate, const float *beta, float *state,
                         void *o, int N, int H, int d_k, int d_v, void *stream) {
    if (var < LA_PLAIN || var > LA_KDA) return LA_ERR_INVALID_ARG;
    if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_INVALID_ARG;
    if (o_dt != LA_F32 && o_dt != LA_BF16) return LA_ERR_INVALID_ARG;
    if (!dtype_pair_ok(dt, o_dt)) return LA_ERR_UNSUPPORTED;
    if (var == LA_NORMALIZED) return LA_ERR_UNSUPPORTED;
    if (N < 1 || H < 1) return LA_ERR_INVALID_ARG;
    // (the delta rules launch two workgroups per sequence-head)
    const bool delta = var == LA_GATED_DELTA || var == LA_KDA;
    if ((int64_t)N * H > (delta ? INT32_MAX / 2 : INT32_MAX)) return LA_ERR_UNSUPPORTED;
    if ((d_k != 32 && d_k != 64 && d_k != 128) || (d_v != 32 && d_v != 64 && d_v != 128))
        return LA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !state || !o) return LA_ERR_INVALID_ARG;
    if ((var == LA_DECAY || var == LA_VECTOR_DECAY || var == LA_KDA) && !log_gate) return LA_ERR_INVALID_ARG;
    if (var == LA_PLAIN && log_gate) return LA_ERR_INVALID_ARG;
    if (delta != (beta != nullptr)) return LA_ERR_INVALID_ARG;
    const void *ptrs[] = {q, k, v, o, log_gate, beta, state};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
    const int64_t NH = (int64_t)N * H;
    const size_t es = elem_size(dt);
    const Span o_sp{o, (size_t)NH * d_v * elem_size(o_dt)}, s_sp{state, (size_t)NH * d_k * d_v * 4};
    const Span ins[] = {{q, (size_t)NH * d_k * es}, {k, (size_t)NH * d_k * es},
                        {v, (size_t)NH * d_v * es},
                        {log_gate, (size_t)NH * 4 * ((var == LA_VECTOR_DECAY || var == LA_KDA) ? d_k : 1)},
                        {beta, (size_t)NH * 4}};
    for (const Span &in : ins)
        if (overlap(o_sp, in) || overlap(s_sp, in)) return LA_ERR_INVALID_ARG;
    if (overlap(o_sp, s_sp)) return LA_ERR_INVALID_ARG;

    const la_status s = check_device();
    if (s != LA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    DecodeArgs a{q, k, v, log_gate, beta, state, o, (int)NH};
    hipError_t e;
    if (var == LA_VECTOR_DECAY) {
        if (dt == LA_F32) e = dispatch_decode<V_VDECAY, float, float>(d_k, d_v, a, st);
        else if (o_dt == LA_F32) e = dispatch_decode<V_VDECAY, bf16, float>(d_k, d_v, a, st);
        else e = dispatch_decode<V_VDECAY, bf16, bf16>(d_k, d_v, a, st);
    } else if (var == LA_KDA) {
        if (dt == LA_F32) e = dispatch_decode<V_KDA, float, float>(d_k, d_v, a, st);
        else if (o_dt == LA_F32) e = dispatch_decode<V_KDA, bf16, float>(d_k, d_v, a, st);
        else e = dispatch_decode<V_KDA, bf16, bf16>(d_k, d_v, a, st);
    } else if (var == LA_GATED_DELTA) {
        if (dt == LA_F32) e = dispatch_decode<V_GDN, float, float>(d_k, d_v, a, st);
        else if (o_dt == LA_F32) e = dispatch_decode<V_GDN, bf16, float>(d_k, d_v, a, st);
        else e = dispatch_decode<V_GDN, bf16, bf16>(d_k, d_v, a, st);
    } else if (var == LA_DECAY) {
        if (dt == LA_F32) e = dispatch_decode<V_DECAY, float, float>(d_k, d_v, a, st);
        else if (o_dt == LA_F32) e = dispatch_decode<V_DECAY, bf16, float>(d_k, d_v, a, st);
        else e = dispatch_decode<V_DECAY, bf16, bf16>(d_k, d_v, a, st);
    } else {
        if (dt == LA_F32) e = dispatch_decode<V_PLAIN, float, float>(d_k, d_v, a, st);
        else if (o_dt == LA_F32) e = dispatch_decode<V_PLAIN, bf16, float>(d_k, d_v, a, st);
        else e = dispatch_decode<V_PLAIN, bf16, bf16>(d_k, d_v, a, st);
    }
    return from_hip(e);
}

la_status la_short_conv(la_dtype dt, const void *q, const void *k, const void *v,
                        const float *w_q, const float *w_k, const float *w_v,
                        const void *q_state_in, const void *k_state_in, const void *v_state_in,
                        void *q_out, void *k_out, void *v_out, void *q_state_out,
                        void *k_state_out, void *v_state_out, int B, int H, int L, int d_k,
                        int d_v, int K, void *stream) {
    if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || L < 0 || K < 1 || d_k < 1 || d_v < 1) return LA_ERR_INVALID_ARG;
    if (K > 4) return LA_ERR_UNSUPPORTED;
    if (d_k % 8 || d_v % 8 || d_k > 4096 || d_v > 4096) return LA_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)B * H;
    const size_t es = elem_size(dt);
    struct Tensor {
        const void *x;
        const float *w;
        const void *si;
        void *y;
        void *so;
        int d;
    };
    const Tensor all[3] = {{q, w_q, q_state_in, q_out, q_state_out, d_k},
                           {k, w_k, k_state_in, k_out, k_state_out, d_k},
                           {v, w_v, v_state_in, v_out, v_state_out, d_v}};
    Tensor use[3];
    int n = 0;
    for (const Tensor &t : all) {  // a tensor is convolved when its taps are given
        if (!t.w) {
            if (t.x || t.si || t.y || t.so) return LA_ERR_INVALID_ARG;
            continue;
        }
        if (L > 0 && (!t.x || !t.y)) return LA_ERR_INVALID_ARG;
        use[n++] = t;
    }
    if (n == 0) return LA_ERR_INVALID_ARG;
    // alignment, then aliasing: outputs overlap nothing except that a window may
    // be updated in place (state_out == state_in of the same tensor)
    Span in_sp[9], out_sp[6];
    int ni = 0, no = 0;
    for (int i = 0; i < n; ++i) {
        const Tensor &t = use[i];
        const void *ptrs[] = {t.x, t.w, t.si, t.y, t.so};
        for (const void *p : ptrs)
            if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
        const size_t xb = (size_t)BH * L * t.d * es, wb = (size_t)H * t.d * K * 4;
        const size_t sb = (size_t)BH * (K - 1) * t.d * es;
        if (t.so && t.si && t.so != t.si && overlap(Span{t.so, sb}, Span{t.si, sb}))
            return LA_ERR_INVALID_ARG;
        in_sp[ni++] = Span{t.x, xb};
        in_sp[ni++] = Span{t.w, wb};
        if (t.si != t.so) in_sp[ni++] = Span{t.si, sb};
        out_sp[no++] = Span{t.y, xb};
        out_sp[no++] = Span{t.so, sb};
    }
    for (int o = 0; o < no; ++o) {
        for (int i = 0; i < ni; ++i)
            if (overlap(out_sp[o], in_sp[i])) return LA_ERR_INVALID_ARG;
        for (int o2 = o + 1; o2 < no; ++o2)
            if (overlap(out_sp[o], out_sp[o2])) return LA_ERR_INVALID_ARG;
    }
    const int tt = dt == LA_BF16 ? conv_tile<bf16>() : conv_tile<float>();
    const int64_t NT = L > 0 ? ((int64_t)L + tt - 1) / tt : 1;
    int64_t blk[3] = {0, 0, 0}, total = 0;
    for (int i = 0; i < n; ++i) {
        blk[i] = (BH * NT * (use[i].d / 8) + 255) / 256;
        total += blk[i];
    }
    if (total * 256 > (int64_t)UINT32_MAX || NT > INT32_MAX || BH > INT32_MAX)
        return LA_ERR_UNSUPPORTED;

    const la_status s = check_device();
    if (s != LA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    ConvArgs a{};
    ConvTensor *slots[3] = {&a.t0, &a.t1, &a.t2};
    for (int i = 0; i < n; ++i)
        *slots[i] = ConvTensor{use[i].x, use[i].y, use[i].si, use[i].so, use[i].w, use[i].d};
    a.blk1 = (unsigned)(n > 1 ? blk[0] : total);
    a.blk2 = (unsigned)(n > 2 ? blk[0] + blk[1] : total);
    a.BH = (int)BH; a.H = H; a.L = L; a.NT = (int)NT; a.ldx = L;
    const hipError_t e = dt == LA_BF16 ? dispatch_short_conv<bf16>(K, a, (unsigned)total, st)
                                       : dispatch_short_conv<float>(K, a, (unsigned)total, st);
    return from_hip(e);
}

la_status la_chunk_bwd_workspace_size(la_variant var, la_dtype dt, int B, int H, int L, int d_k,
                                      int d_v, int C, size_t *bytes) {
    const la_status s = check_bwd_shape(var, dt, B, H, L, d_k, d_v, C);
    if (s != LA_OK) return s;
    if (!bytes) return LA_ERR_INVALID_ARG;
    *bytes = bwd_layout(var, dt, (int64_t)B * H, L, d_k, d_v).total;
    return LA_OK;
}

la_status la_chunk_bwd(la_variant var, la_dtype dt, const void *q, const void *k, const void *v,
                       const float *log_gate, const float *beta, const float *state_in,
                       const float *z_in, const void *d_o, const float *d_state_out,
                       const float *d_z_out, float *dq, float *dk, float *dv, float *d_log_gate,
                       float *d_beta, float *d_state_in, float *d_z_in, int B, int H, int L,
                       int d_k, int d_v, int C, void *workspace, size_t workspace_bytes,
                       void *stream) {
    la_status s = check_bwd_shape(var, dt, B, H, L, d_k, d_v, C);
    if (s != LA_OK) return s;
    const bool tok = L > 0, gdn = var == LA_GATED_DELTA, norm = var == LA_NORMALIZED;
    const bool vec = var == LA_VECTOR_DECAY;
    if (tok && (!q || !k || !v || !d_o || !dq || !dk || !dv)) return LA_ERR_INVALID_ARG;
    if ((var == LA_DECAY || vec) && tok && !log_gate) return LA_ERR_INVALID_ARG;
    if ((var == LA_PLAIN || norm) && (log_gate || d_log_gate)) return LA_ERR_INVALID_ARG;
    if (d_log_gate && !log_gate && tok) return LA_ERR_INVALID_ARG;
    if (gdn ? (tok && !beta) : (beta || d_beta)) return LA_ERR_INVALID_ARG;
    if (!norm && (z_in || d_z_out || d_z_in)) return LA_ERR_INVALID_ARG;
    const void *ptrs[] = {q, k, v, log_gate, beta, state_in, z_in, d_o, d_state_out, d_z_out, dq, dk, dv,
                          d_log_gate, d_beta, d_state_in, d_z_in};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return LA_ERR_INVALID_ARG;
    const int64_t BH = (int64_t)B * H;
    const size_t es = elem_size(dt);
    const size_t qk_b = (size_t)BH * L * d_k * es, v_b = (size_t)BH * L * d_v * es;
    const size_t g_b = (size_t)BH * L * 4, s_b = (size_t)BH * d_k * d_v * 4, z_b = (size_t)BH * d_k * 4;
    const size_t lg_b = vec ? g_b * d_k : g_b;  // per-channel gates: [B, H, L, d_k]
    const BwdLayout lay = bwd_layout(var, dt, BH, L, d_k, d_v);
    if (!workspace || workspace_bytes < lay.total) return LA_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return LA_ERR_INVALID_ARG;
    const Span ins[] = {{q, qk_b},    {k, qk_b},        {v, v_b},    {log_gate, lg_b},   {beta, g_b},
                        {state_in, s_b}, {z_in, z_b},   {d_o, v_b},  {d_state_out, s_b}, {d_z_out, z_b}};
    const Span outs[] = {{dq, (size_t)BH * L * d_k * 4}, {dk, (size_t)BH * L * d_k * 4},
                         {dv, (size_t)BH * L * d_v * 4}, {d_log_gate, lg_b}, {d_beta, g_b},
                         {d_state_in, s_b}, {d_z_in, z_b}, {workspace, lay.total}};
    for (size_t o = 0; o < sizeof(outs) / sizeof(outs[0]); ++o) {
        for (const Span &in : ins)
            if (overlap(outs[o], in)) return LA_ERR_INVALID_ARG;
        for (size_t o2 = o + 1; o2 < sizeof(outs) / sizeof(outs[0]); ++o2)
            if (overlap(outs[o], outs[o2])) return LA_ERR_INVALID_ARG;
    }

    s = check_device();
    if (s != LA_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.dout = d_o; a.lg = log_gate;
    a.s_in = state_in; a.ds_out = d_state_out;
    a.gq = dq; a.gk = dk; a.gv = dv; a.glg = d_log_gate; a.gs_in = d_state_in;
    a.hs = ws + lay.hs; a.dhs = ws + lay.dhs;
    a.s_last = reinterpret_cast<float *>(ws + lay.s_last);
    a.rterm = reinterpret_cast<float *>(ws + lay.rterm);
    a.xterm = reinterpret_cast<float *>(ws + lay.xterm);
    a.BH = (int)BH; a.L = L; a.dv = d_v; a.nsplit = 1;
    const int nch = (L + 63) / 64;
    hipError_t e;
    if (vec) return from_hip(dispatch_vdecay_bwd(d_k, d_v, a, st));
    if (gdn) {
        a.beta = beta; a.gbeta = d_beta;
        a.w = ws + lay.w; a.u = ws + lay.u; a.du = ws + lay.du; a.t = ws + lay.t;
        a.nchunks = nch; a.Lp = nch * 64;
        return from_hip(dispatch_gdn_bwd(d_k, d_v, a, st));
    }
    NormArgs na{};
    la_dtype idt = dt;  // the dtype the kernels read
    if (norm && dt == LA_BF16) {
        // fp32 copies of the inputs and of d_o (fp32 operands, see norm_bwd_impl.hpp)
        float *up = reinterpret_cast<float *>(ws + lay.up);
        const size_t nq = (size_t)BH * L * d_k, nv = (size_t)BH * L * d_v;
        float *q32 = up, *k32 = up + round_up(nq * 4, 256) / 4;
        float *v32 = k32 + round_up(nq * 4, 256) / 4, *o32 = v32 + round_up(nv * 4, 256) / 4;
        if (launch_upcast4(q, k, v, d_o, q32, k32, v32, o32, nq, nv, st) != hipSuccess) return LA_ERR_HIP;
        q = q32; k = k32; v = v32; d_o = o32;
        a.q = q; a.k = k; a.v = v; a.dout = d_o;
        idt = LA_F32;
    }
    if (norm) {
        // the forward pass (its output in fp32 and its denominators), then rho, g
        // and the chunk sums, the plain backward on rho-scaled dO rows, and the
        // normalizer terms
        na.q = q; na.k = k; na.dout = d_o;
        na.o = reinterpret_cast<const float *>(ws + lay.o);
        na.den = reinterpret_cast<const float *>(ws + lay.den);
        na.z_in = z_in; na.dz_out = d_z_out; na.dz_in = d_z_in;
        na.rho = reinterpret_cast<float *>(ws + lay.rho);
        na.g = reinterpret_cast<float *>(ws + lay.g);
        na.ksum = reinterpret_cast<float *>(ws + lay.ksum);
        na.gqsum = reinterpret_cast<float *>(ws + lay.gqsum);
        na.gq = dq; na.gk = dk; na.BH = (int)BH; na.L = L; na.nchunks = nch;
        if (tok) {
            const FwdCall f{LA_NORMALIZED, idt, LA_F32, q, k, v, nullptr, nullptr, state_in, z_in,
                            ws + lay.o, nullptr, nullptr, B, H, L, d_k, d_v, 64};
            s = run_fwd(f, 0, L, state_in, nullptr, nullptr, st, nullptr, reinterpret_cast<float *>(ws + lay.den));
            if (s != LA_OK) return s;
            e = dispatch_norm_pre<float>(d_k, d_v, na, st);
            if (e != hipSuccess) return LA_ERR_HIP;
        }
        a.rho = na.rho;
    }
    if (idt == LA_BF16)
        e = var == LA_DECAY ? dispatch_bwd<bf16, true>(d_k, d_v, a, st) : dispatch_bwd<bf16, false>(d_k, d_v, a, st);
    else
        e = var == LA_DECAY ? dispatch_bwd<float, true>(d_k, d_v, a, st) : dispatch_bwd<float, false>(d_k, d_v, a, st);
    if (e != hipSuccess || !norm) return from_hip(e);
    return from_hip(dispatch_norm_post<float>(d_k, na, st));
}

}  // extern "C"
