"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/hta.h declares, and rejects bad arguments with the
documented status before anything is enqueued (fake pointers are never
dereferenced because validation fails first)."""
import ctypes
import os
import re
import subprocess

import pytest

from hybrid_linear_temporal_hta_amd import hta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hta.h")

F = ctypes.c_void_p(0x10000000)   # fake device pointers (never touched)
G = ctypes.c_void_p(0x20000000)
Hh = ctypes.c_void_p(0x30000000)
O = ctypes.c_void_p(0x40000000)
A = ctypes.c_void_p(0x50000000)
Bt = ctypes.c_void_p(0x60000000)
S = ctypes.c_void_p(0x70000000)
W = ctypes.c_void_p(0x80000000)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\**(hta_[a-z0-9_]+)\s*\(",
                                 text, flags=re.M)))


def test_header_declarations_are_exported():
    names = declared_functions()
    assert set(names) == set(hta.EXPORTED), names
    lib = hta.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", hta.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hta_[a-z0-9_]+)$", out, flags=re.M))
    assert set(names) <= exported, set(names) - exported


def test_peaks_header_declarations_are_exported():
    from hybrid_linear_temporal_hta_amd import peaks
    text = open(os.path.join(ROOT, "include", "hta_peaks.h")).read()
    names = sorted(set(re.findall(r"^\s*[a-z_]+\*?\s+\**(hta_[a-z0-9_]+)\s*\(", text, flags=re.M)))
    assert set(names) == set(peaks.EXPORTED), names
    out = subprocess.run(["nm", "-D", "--defined-only", peaks.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hta_[a-z0-9_]+)$", out, flags=re.M))
    assert set(names) <= exported, set(names) - exported


def test_peaks_argument_errors():
    """The microbenchmarks check their arguments before launching (fake pointers)."""
    from hybrid_linear_temporal_hta_amd import peaks
    L = peaks.lib()
    assert L.hta_peak_mfma_chains() == 4
    assert L.hta_peak_mfma(1, 1, None, None) == -1
    assert L.hta_peak_mfma(0, 1, F, None) == -2
    assert L.hta_peak_mfma(1, 0, F, None) == -2
    assert L.hta_peak_copy(None, G, 16384, None) == -1
    assert L.hta_peak_copy(F, G, 0, None) == -2
    assert L.hta_peak_copy(F, G, 16384 + 64, None) == -2
    assert L.hta_peak_copy(ctypes.c_void_p(F.value + 8), G, 16384, None) == -10
    assert L.hta_peak_copy(F, ctypes.c_void_p(F.value + 16384), 32768, None) == -9
    assert L.hta_peak_lds_dma(None, 1 << 21, 1, 1, 0, None) == -1
    assert L.hta_peak_lds_dma(F, 1 << 21, 0, 1, 0, None) == -2
    assert L.hta_peak_lds_dma(F, 1 << 21, 1, 0, 0, None) == -2
    assert L.hta_peak_lds_dma(F, 1 << 21, 1, 1, 2, None) == -2
    assert L.hta_peak_lds_dma(F, 4096, 1, 1, 0, None) == -2
    assert L.hta_peak_lds_dma(F, (1 << 21) + 8192, 1, 1, 0, None) == -2
    assert L.hta_peak_lds_dma(ctypes.c_void_p(F.value + 8), 1 << 21, 1, 1, 1, None) == -10
    assert L.hta_peak_lds_read(1, 1, 0, None, None) == -1
    assert L.hta_peak_lds_read(0, 1, 1, F, None) == -2
    assert L.hta_peak_lds_read(1, 0, 0, F, None) == -2


def test_version_and_status_strings():
    lib = hta.lib()
    assert b"gfx950" in lib.hta_version()
    for code in range(-9, 1):
        assert lib.hta_status_string(code)
    assert lib.hta_status_string(hta.HTA_ERR_ALIAS).startswith(b"HTA_ERR_ALIAS")


def shape(B=1, H=2, T=4, P=16, d=128, dtype=hta.HTA_BF16, out=None):
    return hta.Shape(B, H, T, P, d, d, dtype, dtype if out is None else out)


def swa(s, window=3, scale=0.0, q=F, k=G, v=Hh, o=O):
    return hta.lib().hta_swa_fwd(ctypes.byref(s) if s is not None else None, q, k, v, o,
                                 window, scale, None)


@pytest.mark.parametrize("mut,code", [
    (dict(B=0), hta.HTA_ERR_SHAPE), (dict(T=0), hta.HTA_ERR_SHAPE), (dict(P=0), hta.HTA_ERR_SHAPE),
    (dict(dtype=7), hta.HTA_ERR_DTYPE), (dict(d=96), hta.HTA_ERR_UNSUPPORTED),
    (dict(out=5), hta.HTA_ERR_DTYPE), (dict(dtype=hta.HTA_F32, d=64, out=hta.HTA_BF16), hta.HTA_ERR_DTYPE),
    (dict(d=64), hta.HTA_ERR_UNSUPPORTED),   # bf16 needs d = 128
])
def test_shape_errors(mut, code):
    assert swa(shape(**mut)) == code


def test_null_and_window_errors():
    assert swa(None) == hta.HTA_ERR_NULL
    assert swa(shape(), q=None) == hta.HTA_ERR_NULL
    assert swa(shape(), window=0) == hta.HTA_ERR_WINDOW
    assert swa(shape(), window=17) == hta.HTA_ERR_WINDOW
    assert swa(shape(), scale=-1.0) == hta.HTA_ERR_UNSUPPORTED
    assert swa(shape(), scale=float("nan")) == hta.HTA_ERR_UNSUPPORTED
    lib = hta.lib()
    s = shape()
    assert lib.hta_dswa_fwd(ctypes.byref(s), F, G, Hh, O, 0, 2, 0.0, None) == hta.HTA_ERR_WINDOW
    assert lib.hta_dswa_fwd(ctypes.byref(s), F, G, Hh, O, 4, 0, 0.0, None) == hta.HTA_ERR_WINDOW
    assert lib.hta_dswa_fwd(ctypes.byref(s), F, G, Hh, O, 4, 2000, 0.0, None) == hta.HTA_ERR_WINDOW


def test_alias_detected():
    s = shape()
    assert swa(s, o=F) == hta.HTA_ERR_ALIAS
    nbytes = 1 * 2 * 4 * 16 * 128 * 2
    assert swa(s, o=ctypes.c_void_p(F.value + nbytes - 16)) == hta.HTA_ERR_ALIAS
    # adjacent but not overlapping is accepted up to the launch; not called here


def test_alignment_errors():
    """Sequence tensors, states and workspaces need 16-byte alignment, gates 4-byte."""
    s = shape()
    assert swa(s, o=ctypes.c_void_p(O.value + 8)) == hta.HTA_ERR_ALIGN
    assert swa(s, q=ctypes.c_void_p(F.value + 2)) == hta.HTA_ERR_ALIGN
    lib = hta.lib()
    prm = hta.make_params(chunk=64)
    need = hta.hta_workspace_bytes(hta.HTA_OP_GLA, s, prm)
    call = lambda q=F, a=A, st=S, ws=W: lib.hta_gla_fwd(
        ctypes.byref(s), q, G, Hh, a, Bt, st, O, 64, 0.0, ws, need, None)
    assert call(st=ctypes.c_void_p(S.value + 4)) == hta.HTA_ERR_ALIGN
    assert call(ws=ctypes.c_void_p(W.value + 8)) == hta.HTA_ERR_ALIGN
    assert call(a=ctypes.c_void_p(A.value + 2)) == hta.HTA_ERR_ALIGN
    # a gate only needs float alignment: this call is refused later, for aliasing
    assert call(a=ctypes.c_void_p(A.value + 4), st=ctypes.c_void_p(A.value + 64)) == hta.HTA_ERR_ALIAS
    assert hta.HTA_ERR_ALIGN == -10
    assert b"ALIGN" in hta.lib().hta_status_string(hta.HTA_ERR_ALIGN)


def test_gla_argument_errors():
    lib = hta.lib()
    s = shape()
    prm = hta.make_params(chunk=64)
    need = hta.hta_workspace_bytes(hta.HTA_OP_GLA, s, prm)
    assert need >= 256
    call = lambda chunk=64, ws=W, wsb=need, **kw: lib.hta_gla_fwd(
        ctypes.byref(s), kw.get("q", F), G, Hh, A, Bt, kw.get("st", S), O, chunk, 0.0, ws, wsb,
        None)
    assert call(chunk=48) == hta.HTA_ERR_UNSUPPORTED
    assert call(chunk=32) == hta.HTA_ERR_UNSUPPORTED      # bf16 path runs chunk 64
    assert call(ws=None) == hta.HTA_ERR_WORKSPACE
    assert call(wsb=need - 1) == hta.HTA_ERR_WORKSPACE
    assert call(q=None) == hta.HTA_ERR_NULL
    assert call(st=F) == hta.HTA_ERR_ALIAS


def test_workspace_bytes_rules():
    s = shape()
    prm = hta.make_params()
    assert hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, s, prm) > \
        hta.hta_workspace_bytes(hta.HTA_OP_GLA, s, prm)
    assert hta.hta_workspace_bytes(99, s, prm) == 0
    assert hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, s, hta.make_params(window=0)) == 0
    assert hta.hta_workspace_bytes(hta.HTA_OP_STREAM_STEP, s, prm) == 0     # T must be 1
    s1 = shape(T=1)
    assert hta.hta_workspace_bytes(hta.HTA_OP_STREAM_STEP, s1, prm) > 0
    # bf16 inputs: the GLA branch runs first into an fp32 partial of its own; a bf16
    # o also needs an fp32 buffer for the SWA branch's output. The one-pass
    # attention parks each wave's own-frame softmax state: 68 floats per lane,
    # 4 waves of 64 lanes per workgroup of 128 query rows.
    so = shape(out=hta.HTA_F32)
    part = so.B * so.H * so.T * so.P * so.dv * 4
    part = (part + 255) // 256 * 256
    park = so.B * so.H * so.T * ((so.P + 127) // 128) * 4 * 64 * 68 * 4
    park = (park + 255) // 256 * 256
    # the GLA branch's operand blocks: 42496 bytes per 64-token chunk and head
    up = lambda n: (n + 255) // 256 * 256
    gla = hta.hta_workspace_bytes(hta.HTA_OP_GLA, so, prm)
    assert gla == up(so.B * so.H * ((so.T * so.P + 63) // 64) * 42496)
    assert hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, so, prm) == gla + part + park
    assert hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, shape(), prm) == gla + 2 * part + park
    assert hta.hta_workspace_bytes(hta.HTA_OP_SWA_DSWA, so, None) == park + part
    # fp32 inputs run the branches in sequence with the GLA partial in o
    f32 = shape(dtype=hta.HTA_F32, d=64)
    prm16 = hta.make_params(chunk=16)
    assert hta.hta_workspace_bytes(hta.HTA_OP_GLA, f32, prm16) > 0
    assert hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, f32, prm16) == \
        hta.hta_workspace_bytes(hta.HTA_OP_GLA, f32, prm16)


def test_stream_ring_too_small():
    lib = hta.lib()
    ctx = hta.StreamCtx(shape(T=1), hta.make_params(3, 4, 4, 64), 12, F.value, G.value, S.value, 0)
    assert lib.hta_stream_step(ctypes.byref(ctx), F, G, Hh, A, Bt, O, W, 1 << 30, None) == \
        hta.HTA_ERR_RING
    assert ctx.n_frames == 0
    ctx.R = 13
    assert lib.hta_stream_step(ctypes.byref(ctx), F, G, Hh, A, Bt, O, W, 16, None) == \
        hta.HTA_ERR_WORKSPACE
    assert lib.hta_stream_init(ctypes.byref(ctx), None, None, 3, None, None) == hta.HTA_ERR_NULL
    assert ctx.n_frames == 0


def test_stream_step_noalloc_rejects_oversized_steps():
    """The no-allocation step refuses a step whose workspace exceeds the fixed
    scratch (before any HIP call), and passes the context checks through."""
    lib = hta.lib()
    prm = hta.make_params(3, 4, 4, 64)
    big = hta.Shape(4, 16, 1, 4096, 128, 128, hta.HTA_BF16, hta.HTA_BF16)
    assert hta.hta_workspace_bytes(hta.HTA_OP_STREAM_STEP, big, prm) > hta.HTA_NOALLOC_SCRATCH_BYTES
    ctx = hta.StreamCtx(big, prm, 13, F.value, G.value, S.value, 5)
    assert lib.hta_stream_step_noalloc(ctypes.byref(ctx), F, G, Hh, A, Bt, O, None) == \
        hta.HTA_ERR_SCRATCH
    assert ctx.n_frames == 5
    ctx.R = 12                                   # the ring check comes first
    assert lib.hta_stream_step_noalloc(ctypes.byref(ctx), F, G, Hh, A, Bt, O, None) == \
        hta.HTA_ERR_RING
    assert "HTA_ERR_SCRATCH" in lib.hta_status_string(hta.HTA_ERR_SCRATCH).decode()
    # the serving workload (B2 H16, 1560 tokens per frame) fits, with either output dtype
    for out in (hta.HTA_F32, hta.HTA_BF16):
        s = hta.Shape(2, 16, 1, 1560, 128, 128, hta.HTA_BF16, out)
        assert hta.hta_workspace_bytes(hta.HTA_OP_STREAM_STEP, s, prm) <= \
            hta.HTA_NOALLOC_SCRATCH_BYTES


def test_gla_form_validation():
    """gla_form must be one of the two update forms; hta_gla_fwd_ex checks it
    before anything else touches the buffers."""
    s = shape()
    assert hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, s, hta.make_params(gla_form=2)) == 0
    assert hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, s,
                                   hta.make_params(gla_form=hta.HTA_GLA_PRINTED)) > 0
    lib = hta.lib()
    need = hta.hta_workspace_bytes(hta.HTA_OP_GLA, s, hta.make_params())
    call = lambda form, ws=W, p=True: lib.hta_gla_fwd_ex(
        ctypes.byref(s), ctypes.byref(hta.make_params(gla_form=form)) if p else None,
        F, G, Hh, A, Bt, S, O, ws, need, None)
    assert call(2) == hta.HTA_ERR_UNSUPPORTED
    assert call(-1) == hta.HTA_ERR_UNSUPPORTED
    assert call(0, p=False) == hta.HTA_ERR_NULL
    assert call(hta.HTA_GLA_PRINTED, ws=None) == hta.HTA_ERR_WORKSPACE


def test_project_argument_checks():
    """hta_project_fwd rejects what its kernel does not cover, before any launch."""
    lib = hta.lib()
    X, Wt = ctypes.c_void_p(0x90000000), ctypes.c_void_p(0xA0000000)
    Q, K, V = ctypes.c_void_p(0xB0000000), ctypes.c_void_p(0xC0000000), ctypes.c_void_p(0xD0000000)
    Al, Be = ctypes.c_void_p(0xE0000000), ctypes.c_void_p(0xF0000000)
    call = lambda s, dm=256, flags=3, **kw: lib.hta_project_fwd(
        ctypes.byref(s) if s is not None else None, dm, kw.get("x", X), Wt, kw.get("q", Q), K, V,
        Al, Be, flags, None)
    ok = shape(B=1, H=4, T=2, P=16)
    assert call(None) == hta.HTA_ERR_NULL
    assert call(ok, x=None) == hta.HTA_ERR_NULL
    assert call(shape(B=1, H=4, T=2, P=16, dtype=hta.HTA_F32, d=128)) == hta.HTA_ERR_UNSUPPORTED
    assert call(shape(B=1, H=2, T=2, P=16)) == hta.HTA_ERR_UNSUPPORTED      # H % 4
    assert call(shape(B=1, H=68, T=2, P=16)) == hta.HTA_ERR_UNSUPPORTED     # 2H > 128
    assert call(ok, dm=100) == hta.HTA_ERR_UNSUPPORTED                      # d_model % 64
    assert call(ok, flags=4) == hta.HTA_ERR_UNSUPPORTED
    assert call(ok, q=K) == hta.HTA_ERR_ALIAS                               # q overlaps k
    assert call(ok, q=X) == hta.HTA_ERR_ALIAS                               # output on input



# ---- backward entry points: argument checks before any launch

Z1 = ctypes.c_void_p(0x90000000)
Z2 = ctypes.c_void_p(0xa0000000)
Z3 = ctypes.c_void_p(0xb0000000)
L1 = ctypes.c_void_p(0xc0000000)
D1 = ctypes.c_void_p(0xd0000000)


def test_attention_backward_argument_checks():
    lib = hta.lib()
    s = shape()
    need = hta.hta_workspace_bytes(hta.HTA_OP_ATTN_BWD, s, None)
    assert need > 0
    # bf16 inputs with an fp32 dout need room for its bf16 copy as well
    assert hta.hta_workspace_bytes(hta.HTA_OP_ATTN_BWD, shape(out=hta.HTA_F32), None) > need

    def call(fn="hta_swa_bwd", ws=W, wsb=need, a=3, **kw):
        args = [ctypes.byref(s), kw.get("q", F), G, Hh, kw.get("o", O), kw.get("lse", L1),
                kw.get("dout", D1), kw.get("dq", Z1), Z2, Z3]
        tail = [a] if fn == "hta_swa_bwd" else [4, kw.get("dil", 2)]
        return getattr(lib, fn)(*args, *tail, 0.0, ws, wsb, None)

    assert call(q=None) == hta.HTA_ERR_NULL
    assert call(lse=None) == hta.HTA_ERR_NULL
    assert call(dout=None) == hta.HTA_ERR_NULL
    assert call(ws=None) == hta.HTA_ERR_WORKSPACE
    assert call(wsb=need - 1) == hta.HTA_ERR_WORKSPACE
    assert call(a=0) == hta.HTA_ERR_WINDOW
    assert call(fn="hta_dswa_bwd", dil=0) == hta.HTA_ERR_WINDOW
    assert call(dq=F) == hta.HTA_ERR_ALIAS            # a gradient over an input
    assert call(dq=D1) == hta.HTA_ERR_ALIAS           # over dout
    assert call(dq=W) == hta.HTA_ERR_ALIAS            # over the workspace
    # the forward with log-sum-exp: lse must not overlap q, k, v or o
    assert lib.hta_swa_fwd_lse(ctypes.byref(s), F, G, Hh, O, None, 3, 0.0, None) == hta.HTA_ERR_NULL
    assert lib.hta_swa_fwd_lse(ctypes.byref(s), F, G, Hh, O, O, 3, 0.0, None) == hta.HTA_ERR_ALIAS
    assert lib.hta_dswa_fwd_lse(ctypes.byref(s), F, G, Hh, O, L1, 0, 2, 0.0, None) == \
        hta.HTA_ERR_WINDOW


def test_gla_backward_argument_checks():
    lib = hta.lib()
    s = shape()
    prm = hta.make_params(chunk=64)
    need = hta.hta_workspace_bytes(hta.HTA_OP_GLA_BWD, s, prm)
    assert need > hta.hta_workspace_bytes(hta.HTA_OP_GLA, s, prm)
    assert hta.hta_workspace_bytes(hta.HTA_OP_GLA_BWD, s, hta.make_params(chunk=32)) == 0

    def call(p=prm, ws=W, wsb=need, **kw):
        return lib.hta_gla_bwd(ctypes.byref(s), ctypes.byref(p), F, G, Hh, A, Bt,
                               kw.get("s0", S), kw.get("dout", D1), kw.get("dst", L1),
                               kw.get("dq", Z1), Z2, Z3, kw.get("da", O),
                               ctypes.c_void_p(0xe0000000), ws, wsb, None)

    assert call(s0=None) == hta.HTA_ERR_NULL
    assert call(dst=None) == hta.HTA_ERR_NULL
    assert call(wsb=need - 1) == hta.HTA_ERR_WORKSPACE
    assert call(p=hta.make_params(chunk=64, gla_form=2)) == hta.HTA_ERR_UNSUPPORTED
    assert call(dq=S) == hta.HTA_ERR_ALIAS            # a gradient over the initial state
    assert call(da=A) == hta.HTA_ERR_ALIAS            # dalpha over alpha
    assert call(dst=S) == hta.HTA_ERR_ALIAS           # dstate over the initial state


def test_hybrid_training_argument_checks():
    lib = hta.lib()
    s = shape()
    prm = hta.make_params()
    saved = hta.hta_hybrid_saved_bytes(s)
    # two fp32 branch outputs, two log-sum-exp rows, the initial state
    L = s.B * s.H * s.T * s.P
    al = lambda n: (n + 255) // 256 * 256
    assert saved == 2 * al(L * s.dv * 4) + 2 * al(L * 4) + al(s.B * s.H * s.dk * s.dv * 4)
    assert hta.hta_hybrid_saved_bytes(shape(B=0)) == 0
    need_f = hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, s, prm)
    need_b = hta.hta_workspace_bytes(hta.HTA_OP_HYBRID_BWD, s, prm)
    assert need_b > hta.hta_workspace_bytes(hta.HTA_OP_GLA_BWD, s, prm)
    SV = ctypes.c_void_p(0xf0000000)
    fwd = lambda sv=SV, o=O: lib.hta_hybrid_fwd_train(ctypes.byref(s), ctypes.byref(prm), F, G, Hh,
                                                      A, Bt, S, o, sv, W, need_f, None)
    assert fwd(sv=None) == hta.HTA_ERR_NULL
    assert fwd(sv=O) == hta.HTA_ERR_ALIAS             # saved over o
    bwd = lambda wsb=need_b, dq=Z1, sv=SV: lib.hta_hybrid_bwd(
        ctypes.byref(s), ctypes.byref(prm), F, G, Hh, A, Bt, sv, D1, L1, dq, Z2, Z3, O,
        ctypes.c_void_p(0xe0000000), W, wsb, None)
    assert bwd(sv=None) == hta.HTA_ERR_NULL
    assert bwd(wsb=need_b - 1) == hta.HTA_ERR_WORKSPACE
    assert bwd(dq=SV) == hta.HTA_ERR_ALIAS            # a gradient over the saved activations
