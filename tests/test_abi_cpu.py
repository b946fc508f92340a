"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before touching the HIP runtime."""
import ctypes
import re

import pytest

import chunkwise_linear_rnn_causal_amd as la

PLAIN, NORM, DECAY, GDN, VDECAY, KDA = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
INVALID, UNSUPPORTED = la.LA_ERR_INVALID_ARG, la.LA_ERR_UNSUPPORTED
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def header_functions():
    src = open(la.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_binding_names():
    assert header_functions() == sorted(la.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = la.load_library()
    for name in header_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert la.la_abi_version() == 3
    assert la.la_status_str(0) == "LA_OK"
    assert la.la_status_str(1) == "LA_ERR_INVALID_ARG"
    assert la.la_status_str(2) == "LA_ERR_UNSUPPORTED"
    assert la.la_status_str(3) == "LA_ERR_HIP"


def chunk(var=PLAIN, dt=BF16, odt=F32, q=FAKE, k=FAKE, v=FAKE, lg=None, beta=None, s_in=None, z_in=None,
          o=0x800000000, s_out=None, z_out=None, B=1, H=1, L=128, dk=64, dv=64, C=64, ws=None,
          ws_bytes=0):
    return la.load_library().la_chunk_fwd(var, dt, odt, q, k, v, lg, beta, s_in, z_in, o, s_out, z_out,
                                          B, H, L, dk, dv, C, ws, ws_bytes, None)


def wsize(var=GDN, dt=BF16, B=2, H=3, L=100, dk=64, dv=32, C=64):
    out = ctypes.c_size_t(123)
    st = la.load_library().la_chunk_fwd_workspace_size(var, dt, B, H, L, dk, dv, C, ctypes.byref(out))
    return st, out.value


def test_workspace_sizes():
    # one fused pass for the variants without the delta rule
    for var in (PLAIN, NORM, DECAY):
        assert wsize(var=var) == (0, 0)
    # delta rule: W [BH, Lp, dk] + U~ [BH, Lp, dv] (each rounded to 256 B), Lp = 128,
    # and for bf16 the score fragments, 96 bytes per token
    up = lambda x: -(-x // 256) * 256
    st, n = wsize()
    assert st == 0 and n == up(2 * 3 * 128 * 64 * 2) + up(2 * 3 * 128 * 32 * 2) + 2 * 3 * 128 * 96
    st, n = wsize(dt=F32, L=37, dv=32)
    assert st == 0 and n == up(2 * 3 * 64 * 64 * 4) + up(2 * 3 * 64 * 32 * 4)
    assert wsize(L=0) == (0, 0)
    # C = 128: the delta rule runs its 128-token chunks as two 64-token sub-chunks
    assert wsize(C=128) == wsize(C=64)
    assert la.load_library().la_chunk_fwd_workspace_size(GDN, BF16, 1, 1, 8, 64, 64, 64, None) == INVALID
    # the largest head the 32-bit row offsets address, and one chunk more
    assert wsize(B=1, H=1, L=2 ** 24 - 64, dk=128, dv=128)[0] == 0
    assert wsize(B=1, H=1, L=2 ** 24 - 63, dk=128, dv=128)[0] == UNSUPPORTED
    # KDA (bf16 only): the delta rule's arrays, then q and k with the gates folded in
    # (fp16 [BH, Lp, dk] each) and the per-chunk state decay (fp32 [BH, Lp / 64, dk])
    st, n = wsize(var=KDA)
    assert st == 0 and n == (up(2 * 3 * 128 * 64 * 2) + up(2 * 3 * 128 * 32 * 2) + 2 * 3 * 128 * 96
                             + 2 * up(2 * 3 * 128 * 64 * 2) + up(2 * 3 * 2 * 64 * 4))
    assert wsize(var=KDA, dt=F32)[0] == UNSUPPORTED
    assert wsize(var=KDA, C=128) == wsize(var=KDA, C=64)


@pytest.mark.parametrize("kw,expect", [
    (dict(var=7), INVALID),
    (dict(var=KDA, beta=FAKE + 0x200000), INVALID),   # KDA needs its gates
    (dict(var=KDA, lg=FAKE + 0x100000), INVALID),     # and beta
    (dict(var=KDA, lg=FAKE + 0x100000, beta=FAKE + 0x200000, dt=F32), UNSUPPORTED),
    (dict(var=KDA, lg=FAKE + 0x100000, beta=FAKE + 0x200000, o=FAKE + 0x100000 + 0x7000), INVALID),  # o in the gates
    (dict(var=KDA, lg=FAKE + 0x100000, beta=FAKE + 0x200000), INVALID),  # workspace missing (dict(dt=5), INVALID), (dict(odt=5), INVALID),
    (dict(var=VDECAY), INVALID),                      # per-channel decay needs its gates
    (dict(var=VDECAY, lg=FAKE + 0x100000, dt=F32, dk=128), UNSUPPORTED),
    (dict(var=VDECAY, lg=FAKE + 0x100000, o=FAKE + 0x100000 + 0x7000), INVALID),  # o inside the gates
    (dict(dt=F32, odt=BF16), UNSUPPORTED),
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(L=-3), INVALID),
    (dict(dk=48), UNSUPPORTED), (dict(dk=256), UNSUPPORTED),
    (dict(dv=48), UNSUPPORTED), (dict(dv=256), UNSUPPORTED),
    (dict(C=32), UNSUPPORTED), (dict(C=256), UNSUPPORTED),
    # row offsets inside one head are 32-bit: ceil(L/C)*C*max(d_k, d_v) < 2^31
    (dict(L=2 ** 24, dk=128, dv=32), UNSUPPORTED), (dict(L=2 ** 24 - 63, dk=32, dv=128), UNSUPPORTED),
    (dict(L=2 ** 25 - 63, dk=64, dv=64), UNSUPPORTED),
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(var=DECAY), INVALID),                       # decay needs a log-gate
    (dict(var=PLAIN, lg=FAKE + 0x100000), INVALID),   # gate given to an ungated variant
    (dict(var=GDN, lg=FAKE + 0x100000), INVALID),     # delta rule needs beta
    (dict(var=DECAY, lg=FAKE + 0x100000, beta=FAKE + 0x200000), INVALID),
    (dict(var=PLAIN, z_in=FAKE + 0x100000), INVALID), # normalizer given to another variant
    (dict(q=FAKE + 2), INVALID),                      # misaligned
    (dict(o=FAKE), INVALID),                          # output aliases an input
    (dict(s_in=0x900000000, s_out=0x900000010), INVALID),  # partial state overlap
    (dict(var=GDN, beta=FAKE + 0x100000), INVALID),   # workspace missing
    (dict(var=GDN, beta=FAKE + 0x100000, ws=0x700000000, ws_bytes=16), INVALID),  # too small
])
def test_chunk_fwd_rejects(kw, expect):
    assert chunk(**kw) == expect


def test_kda_valid_arguments_reach_the_device_check():
    assert chunk(var=KDA, lg=FAKE + 0x100000, beta=FAKE + 0x200000, ws=0x700000000,
                 ws_bytes=1 << 30) not in (INVALID, UNSUPPORTED)
    assert dec(var=KDA, beta=FAKE + 0x5000) not in (INVALID, UNSUPPORTED)


def test_noalloc_refuses_problems_whose_chunk_exceeds_the_scratch():
    lib = la.load_library()
    G = 1 << 32  # fake, 16-byte aligned, far apart: validation fails first
    # 4096 heads of d = 128: one chunk of products is 128 MiB, above the 64 MiB scratch
    st = lib.la_chunk_fwd_noalloc(GDN, BF16, F32, G, 2 * G, 3 * G, None, 4 * G, None, None, 5 * G,
                                  None, None, 64, 64, 64, 128, 128, 64, None)
    assert st == UNSUPPORTED
    # the same shape checks as la_chunk_fwd
    assert lib.la_chunk_fwd_noalloc(GDN, BF16, F32, G, 2 * G, 3 * G, None, None, None, None, 5 * G,
                                    None, None, 1, 1, 64, 64, 64, 64, None) == INVALID  # beta missing
    assert lib.la_chunk_fwd_noalloc(GDN, BF16, F32, G, 2 * G, 3 * G, None, 4 * G, None, None, 5 * G,
                                    None, None, 1, 1, 64, 48, 64, 64, None) == UNSUPPORTED


def dec(var=DECAY, dt=BF16, odt=F32, q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000, lg=FAKE + 0x3000, beta=None,
        S=0x900000000, o=0x800000000, N=4, H=2, dk=128, dv=128):
    return la.load_library().la_decode_step(var, dt, odt, q, k, v, lg, beta, S, o, N, H, dk, dv, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(var=9), INVALID), (dict(var=NORM), UNSUPPORTED),
    (dict(var=VDECAY, lg=None), INVALID),             # per-channel decay needs its gates
    (dict(var=VDECAY, o=FAKE + 0x3800), INVALID),     # o inside the [N,H,d_k] gates
    (dict(var=GDN), INVALID),                         # delta rule needs beta
    (dict(var=GDN, beta=FAKE + 0x5000, o=FAKE + 0x5000), INVALID),  # o overlaps beta
    (dict(var=KDA), INVALID),                         # KDA needs beta
    (dict(var=KDA, beta=FAKE + 0x5000, lg=None), INVALID),  # and its gates
    (dict(var=KDA, beta=FAKE + 0x5000, o=FAKE + 0x3800), INVALID),  # o inside the [N,H,d_k] gates
    (dict(odt=7), INVALID), (dict(dt=F32, odt=BF16), UNSUPPORTED),
    (dict(N=0), INVALID), (dict(dk=96), UNSUPPORTED), (dict(dv=16), UNSUPPORTED),
    (dict(q=None), INVALID), (dict(S=None), INVALID), (dict(lg=None), INVALID),
    (dict(var=PLAIN), INVALID),                       # plain step takes no gate
    (dict(beta=FAKE + 0x4000), INVALID),
    (dict(o=FAKE), INVALID),                          # o overlaps q
    (dict(o=0x900000000 + 64), INVALID),              # o inside the state
    (dict(S=0x900000008), INVALID),                   # misaligned state
])
def test_decode_step_rejects(kw, expect):
    assert dec(**kw) == expect


def conv(dt=BF16, q=FAKE, k=None, v=None, wq=0x200000, wk=None, wv=None, qsi=None, ksi=None, vsi=None,
         qo=0x800000000, ko=None, vo=None, qso=None, kso=None, vso=None, B=1, H=2, L=64, dk=64, dv=64,
         K=4):
    return la.load_library().la_short_conv(dt, q, k, v, wq, wk, wv, qsi, ksi, vsi, qo, ko, vo, qso, kso,
                                           vso, B, H, L, dk, dv, K, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(dt=5), INVALID), (dict(B=0), INVALID), (dict(L=-1), INVALID), (dict(K=0), INVALID),
    (dict(K=5), UNSUPPORTED), (dict(dk=12), UNSUPPORTED), (dict(dk=8192), UNSUPPORTED),
    (dict(q=None, wq=None, qo=None), INVALID),            # nothing to convolve
    (dict(wq=None), INVALID),                             # input without taps
    (dict(q=None), INVALID),                              # taps without input (L > 0)
    (dict(qo=None), INVALID),                             # output missing
    (dict(ko=0x900000000), INVALID),                      # output for a skipped tensor
    (dict(ksi=0x900000000), INVALID),                     # window for a skipped tensor
    (dict(q=FAKE + 8), INVALID),                          # misaligned
    (dict(qo=FAKE), INVALID),                             # in place y = x
    (dict(qo=FAKE + 0x1000), INVALID),                    # output overlaps the input
    (dict(k=0x300000, wk=0x400000, ko=0x800000000 + 0x2000), INVALID),  # outputs overlap
    (dict(k=0x300000, wk=0x400000, ko=0x300000 + 0x100), INVALID),      # k output overlaps k
    (dict(v=0x300000, wv=0x400000, vo=FAKE + 0x10), INVALID),           # v output overlaps q
    (dict(qsi=0xA00000000, qso=0xA00000010), INVALID),    # partial window overlap
    (dict(qso=0x200000), INVALID),                        # window written over the taps
])
def test_short_conv_rejects(kw, expect):
    assert conv(**kw) == expect


@pytest.mark.parametrize("kw", [
    dict(), dict(qsi=0xA00000000, qso=0xA00000000),       # window updated in place
    dict(L=0, qo=None), dict(L=0, q=None, qo=None), dict(K=1), dict(q=None, wq=None, qo=None, v=0x300000, wv=0x400000,
                                        vo=0x900000000, dv=32),
])
def test_short_conv_valid_arguments_reach_the_device_check(kw):
    # on a host without a usable gfx950 device the call fails only at the device
    # check, after every argument was accepted
    assert conv(**kw) not in (INVALID,)


def bwd(var=DECAY, dt=BF16, q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, lg=FAKE + 0x300000, beta=None,
        s_in=None, z_in=None, do=FAKE + 0x400000, dso=None, dzo=None, dq=0x800000000, dk=0x810000000,
        dv=0x820000000, dlg=None, dbeta=None, dsi=None, dzi=None, B=1, H=2, L=128, dk_=64, dv_=64, C=64,
        ws=0x900000000, ws_bytes=1 << 30):
    return la.load_library().la_chunk_bwd(var, dt, q, k, v, lg, beta, s_in, z_in, do, dso, dzo, dq, dk, dv, dlg,
                                          dbeta, dsi, dzi, B, H, L, dk_, dv_, C, ws, ws_bytes, None)


def bwd_wsize(var=DECAY, dt=BF16, B=2, H=3, L=100, dk_=64, dv_=32, C=64):
    out = ctypes.c_size_t(123)
    st = la.load_library().la_chunk_bwd_workspace_size(var, dt, B, H, L, dk_, dv_, C, ctypes.byref(out))
    return st, out.value


def test_bwd_workspace_size():
    # per-chunk states and state gradients (fp16 operands for bf16), final state, one float per
    # token, one float per chunk (<dH_c, H_{c+1}>, where the gate gradient's suffix restarts)
    st, n = bwd_wsize()
    r = lambda x: -(-x // 256) * 256
    states = r(6 * 2 * 64 * 32 * 2)
    base = 2 * states + r(6 * 64 * 32 * 4) + r(6 * 100 * 4) + r(6 * 2 * 4)
    assert st == 0 and n == base
    # delta rule (bf16 only): also W [BH, Lp, dk], U~ and A_m^T dO [BH, Lp, dv] and T [BH, nch, 64, 64], fp16
    st, n = bwd_wsize(var=GDN)
    assert st == 0 and n == base + r(6 * 128 * 64 * 2) + 2 * r(6 * 128 * 32 * 2) + r(6 * 2 * 64 * 64 * 2)
    assert bwd_wsize(var=GDN, dt=F32)[0] == UNSUPPORTED
    # per-channel decay (bf16 only): the decay layout
    assert bwd_wsize(var=VDECAY) == bwd_wsize()
    assert bwd_wsize(var=VDECAY, dt=F32)[0] == UNSUPPORTED
    # normalized: also the forward's fp32 output, den, rho, g per token, two d_k sums per chunk
    # (fp32 operands: fp32 states, and for bf16 inputs fp32 copies of q, k, v, d_o)
    st, n = bwd_wsize(var=NORM)
    states32 = r(6 * 2 * 64 * 32 * 4)
    assert st == 0 and n == (2 * states32 + r(6 * 64 * 32 * 4) + r(6 * 100 * 4) + r(6 * 2 * 4) + r(6 * 100 * 32 * 4)
                             + 3 * r(6 * 100 * 4) + 2 * r(6 * 2 * 64 * 4)
                             + 2 * r(6 * 100 * 64 * 4) + 2 * r(6 * 100 * 32 * 4))
    assert bwd_wsize(var=NORM, dk_=128, dv_=128)[0] == UNSUPPORTED
    assert bwd_wsize(C=128)[0] == UNSUPPORTED
    assert bwd_wsize(dt=F32, dk_=128, dv_=128)[0] == UNSUPPORTED
    assert bwd_wsize(dt=F32, dk_=128, dv_=32)[0] == 0
    assert bwd_wsize(L=2 ** 24 - 63, dk_=128, dv_=128)[0] == UNSUPPORTED   # 32-bit head offsets


@pytest.mark.parametrize("kw,expect", [
    (dict(var=9), INVALID), (dict(var=NORM), INVALID), (dict(var=VDECAY, dt=F32), UNSUPPORTED),
    (dict(var=VDECAY, lg=None), INVALID),               # the per-channel decay needs its gates
    (dict(var=VDECAY, dlg=FAKE + 0x300000 + 0x8000), INVALID),  # d_log_gate inside the [B,H,L,d_k] gates
    (dict(z_in=FAKE + 0x600000), INVALID),              # the normalizer is the normalized variant's
    (dict(var=NORM, lg=None, dzi=FAKE + 0x400000), INVALID),   # d_z_in inside d_o
    (dict(C=128), UNSUPPORTED), (dict(dk_=96), UNSUPPORTED), (dict(B=0), INVALID),
    (dict(lg=None), INVALID),                           # decay needs its gates
    (dict(var=PLAIN), INVALID),                         # plain takes no gates
    (dict(var=PLAIN, lg=None, dlg=0x830000000), INVALID),
    (dict(do=None), INVALID), (dict(dq=None), INVALID),
    (dict(ws=None), INVALID), (dict(ws_bytes=1024), INVALID), (dict(ws=0x900000010), INVALID),
    (dict(dq=FAKE + 0x400000 + 0x100), INVALID),        # dq inside d_o
    (dict(dk=0x800000000 + 0x1000), INVALID),           # dk inside dq
    (dict(dsi=0x900000000 + 0x100), INVALID),           # d_state_in inside the workspace
    (dict(q=FAKE + 4), INVALID),
    (dict(beta=FAKE + 0x500000), INVALID),              # beta is the delta rule's
    (dict(dbeta=0x830000000), INVALID),
    (dict(var=GDN), INVALID),                           # the delta rule needs beta
    (dict(var=GDN, dt=F32, beta=FAKE + 0x500000), UNSUPPORTED),
    (dict(var=GDN, lg=None, beta=FAKE + 0x500000, dlg=0x830000000), INVALID),  # no gates, no gate gradient
    (dict(var=GDN, beta=FAKE + 0x500000, dbeta=FAKE + 0x500000 + 0x40), INVALID),  # d_beta inside beta
    (dict(var=GDN, beta=FAKE + 0x500008), INVALID),     # misaligned beta
])
def test_chunk_bwd_rejects(kw, expect):
    assert bwd(**kw) == expect


def test_chunk_bwd_valid_arguments_reach_the_device_check():
    assert bwd() not in (INVALID, UNSUPPORTED)
    assert bwd(var=PLAIN, lg=None) not in (INVALID, UNSUPPORTED)
    assert bwd(L=0, q=None, k=None, v=None, do=None, dq=None, dk=None, dv=None) not in (INVALID, UNSUPPORTED)
    assert bwd(var=GDN, beta=FAKE + 0x500000, dbeta=0x830000000, dlg=0x840000000) not in (INVALID, UNSUPPORTED)
    assert bwd(var=GDN, lg=None, beta=FAKE + 0x500000) not in (INVALID, UNSUPPORTED)
    assert bwd(var=VDECAY, dlg=0x830000000) not in (INVALID, UNSUPPORTED)
    assert bwd(var=KDA, beta=FAKE + 0x500000) == UNSUPPORTED  # no KDA backward
    assert bwd(var=NORM, lg=None, z_in=FAKE + 0x600000, dzo=FAKE + 0x610000,
               dzi=0x830000000) not in (INVALID, UNSUPPORTED)


def conv_fwd(var=GDN, dt=BF16, odt=F32, q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, wq=FAKE + 0x300000,
             wk=FAKE + 0x310000, wv=FAKE + 0x320000, K=4, qwi=None, kwi=None, vwi=None, qwo=None, kwo=None,
             vwo=None, lg=FAKE + 0x400000, beta=FAKE + 0x410000, s_in=None, o=0x800000000, s_out=None,
             B=1, H=2, L=128, dk=64, dv=64, C=64, ws=0x900000000, ws_bytes=1 << 30):
    return la.load_library().la_chunk_fwd_conv(var, dt, odt, q, k, v, wq, wk, wv, K, qwi, kwi, vwi, qwo, kwo,
                                               vwo, lg, beta, s_in, o, s_out, B, H, L, dk, dv, C, ws,
                                               ws_bytes, None)


def test_conv_fused_workspace_size():
    out = ctypes.c_size_t(0)
    lib = la.load_library()
    assert lib.la_chunk_fwd_conv_workspace_size(GDN, BF16, 2, 3, 100, 64, 32, 64, 4, ctypes.byref(out)) == 0
    up = lambda x: -(-x // 256) * 256
    base = up(6 * 128 * 64 * 2) + up(6 * 128 * 32 * 2) + 6 * 128 * 96
    assert out.value == base + 2 * up(6 * 128 * 64 * 2) + up(6 * 3 * (2 * 64 + 32) * 2)
    for var, dt, K in ((DECAY, BF16, 4), (GDN, F32, 4), (GDN, BF16, 5)):
        assert lib.la_chunk_fwd_conv_workspace_size(var, dt, 2, 3, 100, 64, 32, 64, K, ctypes.byref(out)) == UNSUPPORTED
    assert lib.la_chunk_fwd_conv_workspace_size(GDN, BF16, 2, 3, 100, 64, 32, 64, 0, ctypes.byref(out)) == INVALID


@pytest.mark.parametrize("kw,expect", [
    (dict(var=DECAY, beta=None), UNSUPPORTED), (dict(dt=F32), UNSUPPORTED), (dict(K=5), UNSUPPORTED),
    (dict(K=0), INVALID), (dict(wq=None), INVALID), (dict(wv=None), INVALID), (dict(beta=None), INVALID),
    (dict(ws=None), INVALID), (dict(ws_bytes=1024), INVALID), (dict(ws=0x900000010), INVALID),
    (dict(qwi=FAKE + 0x500008), INVALID),                         # misaligned window
    (dict(kwo=FAKE + 0x100000), INVALID),                         # outgoing window inside k
    (dict(qwo=0x800000000 + 0x100), INVALID),                     # outgoing window inside o
    (dict(vwo=0x900000000 + 0x1000), INVALID),                    # outgoing window inside the workspace
    (dict(o=FAKE + 0x300000), INVALID),                           # o over the taps
    (dict(qwi=FAKE + 0x600000, kwo=FAKE + 0x600000 + 0x10), INVALID),  # window out inside another's window in
])
def test_conv_fused_rejects(kw, expect):
    assert conv_fwd(**kw) == expect


def test_conv_fused_valid_arguments_reach_the_device_check():
    assert conv_fwd() not in (INVALID, UNSUPPORTED)
    assert conv_fwd(qwi=FAKE + 0x600000, qwo=FAKE + 0x600000) not in (INVALID, UNSUPPORTED)  # in place
    assert conv_fwd(lg=None, K=1) not in (INVALID, UNSUPPORTED)
    assert conv_fwd(L=0, q=None, k=None, v=None, o=None, beta=None) not in (INVALID, UNSUPPORTED)
