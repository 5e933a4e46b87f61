"""C-ABI contract checks that need no GPU: the library loads, exports every
declared symbol, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prism.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from gated_delta_rule_prologue_amd import binding
    if not os.path.exists(binding.lib_path()):
        pytest.fail("libprism.so is not built (run __graft_entry__.build())")
    return binding.lib()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("prism_fwd", "prism_prologue", "prism_scan", "prism_workspace_bytes",
              "prism_status_str", "prism_abi_version", "prism_fwd_resume", "prism_decode_step",
              "prism_prologue_ex", "prism_scan_ex", "prism_scan_workspace_bytes", "prism_bwd",
              "prism_bwd_workspace_bytes", "prism_bwd_ex", "prism_scan_wait_giveups",
              "prism_fwd_noalloc", "prism_checkpoint_bytes", "prism_fwd_ckpt", "prism_bwd_ckpt"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_abi_version(lib):
    assert lib.prism_abi_version() == 2


def test_status_strings(lib):
    from gated_delta_rule_prologue_amd import binding
    assert binding.status_str(0) == "ok"
    assert "invalid" in binding.status_str(1)
    assert "unsupported" in binding.status_str(2)
    assert "HIP" in binding.status_str(3)


def test_fwd_noalloc_rejects_bad_arguments(lib):
    from gated_delta_rule_prologue_amd import binding as B
    ok = B.make_dims(1, 10, 1, 64, 64, B.PRISM_BF16)
    call = lambda d, L=2: lib.prism_fwd_noalloc(ctypes.byref(d), *([FAKE] * 10), L, FAKE, FAKE,
                                                None)
    assert call(ok, L=0) == B.PRISM_EINVAL
    assert call(B.make_dims(0, 10, 1, 64, 64, B.PRISM_BF16)) == B.PRISM_EINVAL
    # the scratch bound is checked before the device is touched
    big = B.make_dims(1, 65536, 16, 128, 128, B.PRISM_BF16)
    assert B.workspace_bytes(big, 4) > B.NOALLOC_MAX_BYTES
    assert call(big, L=4) == B.PRISM_ENOSPACE
    assert "scratch" in B.status_str(B.PRISM_ENOSPACE)


def test_wait_giveups_rejects_null(lib):
    from gated_delta_rule_prologue_amd import binding as B
    assert lib.prism_scan_wait_giveups(None, 0) == B.PRISM_EINVAL


def test_workspace_bytes(lib, monkeypatch):
    """prism_workspace_bytes: the write keys (input dtype, 256-byte rounded)
    plus, for the opt-in two-pass bf16 scan, the per-chunk matrices: 20 KB (T,
    A_kkw, A_qkw, -A_qk as ten bf16 16x16 blocks each) per head and virtual
    chunk, floor(T / 64) + n_seqs virtual chunks; plus, at the bf16 shapes the
    in-scan write-key producers serve (L = 4, or 8 at dk = 64), one int32
    readiness flag per head and virtual chunk (256-byte rounded)."""
    from gated_delta_rule_prologue_amd import binding as B
    up = lambda x: (x + 255) // 256 * 256
    d = B.make_dims(8, 16384, 6, 128, 128, B.PRISM_BF16)
    monkeypatch.delenv("PRISM_SCAN_TWOPASS", raising=False)
    monkeypatch.delenv("PRISM_KW_PRODUCERS", raising=False)
    assert B.workspace_bytes(d, 4) == 16384 * 6 * 128 * 2
    assert B.scan_workspace_bytes(d) == 0
    monkeypatch.setenv("PRISM_SCAN_TWOPASS", "1")
    assert B.workspace_bytes(d, 4) == 16384 * 6 * 128 * 2 + up((16384 // 64 + 8) * 6 * 20480)
    assert B.scan_workspace_bytes(d) == up((16384 // 64 + 8) * 6 * 20480)
    monkeypatch.delenv("PRISM_SCAN_TWOPASS")
    # the opt-in write-key producers add their flags at the shapes they serve
    monkeypatch.setenv("PRISM_KW_PRODUCERS", "1")
    flags = up((16384 // 64 + 8) * 6 * 4)
    assert B.workspace_bytes(d, 4) == 16384 * 6 * 128 * 2 + flags
    assert B.workspace_bytes(d, 3) == 16384 * 6 * 128 * 2              # none at L = 3
    d64 = B.make_dims(3, 1000, 2, 64, 64, B.PRISM_BF16)
    assert B.workspace_bytes(d64, 8) == up(1000 * 2 * 64 * 2) + up((1000 // 64 + 3) * 2 * 4)
    assert B.workspace_bytes(B.make_dims(3, 1000, 2, 128, 64, B.PRISM_BF16), 8) == up(1000 * 2 * 128 * 2)
    monkeypatch.delenv("PRISM_KW_PRODUCERS")
    d32 = B.make_dims(1, 3, 1, 64, 64, B.PRISM_F32)
    assert B.workspace_bytes(d32, 2) == 768
    assert B.workspace_bytes(B.make_dims(1, 0, 1, 64, 64, B.PRISM_BF16), 1) == 256
    assert B.workspace_bytes(d, 0) == 0 and B.workspace_bytes(d, 17) == 0
    assert B.workspace_bytes(B.make_dims(0, 0, 1, 64, 64, B.PRISM_BF16), 1) == 0


FAKE = 0x10000          # aligned, never dereferenced: every call below fails validation first


def _fwd(lib, d, L=2, ws=1 << 30, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, g=FAKE, b=FAKE, a=FAKE, h=FAKE, conv_w=FAKE,
                cu=FAKE, o=FAKE, s=FAKE, w=FAKE)
    args.update(over)
    return lib.prism_fwd(ctypes.byref(d), args["q"], args["k"], args["v"], args["u"], args["g"],
                         args["b"], args["a"], args["h"], args["conv_w"], args["cu"], L, args["o"],
                         args["s"], args["w"], ws, None)


def test_fwd_rejects_bad_arguments(lib):
    from gated_delta_rule_prologue_amd import binding as B
    # unsupported widths are reported as such (before any launch)
    assert _fwd(lib, B.make_dims(1, 10, 1, 96, 64, B.PRISM_BF16)) == B.PRISM_EUNSUPPORTED
    assert _fwd(lib, B.make_dims(1, 10, 1, 96, 128, B.PRISM_F32)) == B.PRISM_EUNSUPPORTED
    assert _fwd(lib, B.make_dims(1, 10, 1, 128, 48, B.PRISM_F32)) == B.PRISM_EUNSUPPORTED
    ok = B.make_dims(1, 10, 1, 64, 64, B.PRISM_BF16)
    # null / misaligned pointers, bad L, small workspace, bad dims
    assert _fwd(lib, ok, q=None) == B.PRISM_EINVAL
    assert _fwd(lib, ok, k=FAKE + 2) == B.PRISM_EINVAL
    assert _fwd(lib, ok, u=None) == B.PRISM_EINVAL
    assert _fwd(lib, ok, L=0) == B.PRISM_EINVAL
    assert _fwd(lib, ok, L=17) == B.PRISM_EINVAL
    assert _fwd(lib, ok, ws=16) == B.PRISM_EINVAL
    assert _fwd(lib, ok, cu=None) == B.PRISM_EINVAL
    assert _fwd(lib, ok, s=None) == B.PRISM_EINVAL
    assert _fwd(lib, B.make_dims(0, 10, 1, 64, 64, B.PRISM_BF16)) == B.PRISM_EINVAL
    assert _fwd(lib, B.make_dims(1, -1, 1, 64, 64, B.PRISM_BF16)) == B.PRISM_EINVAL
    assert _fwd(lib, B.make_dims(1, 10, 0, 64, 64, B.PRISM_BF16)) == B.PRISM_EINVAL
    assert _fwd(lib, B.make_dims(1, 10, 1, 64, 64, 7)) == B.PRISM_EINVAL
    assert lib.prism_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2,
                         FAKE, FAKE, FAKE, 1 << 30, None) == B.PRISM_EINVAL


def test_prologue_and_scan_reject_bad_arguments(lib):
    from gated_delta_rule_prologue_amd import binding as B
    d = B.make_dims(1, 10, 1, 64, 64, B.PRISM_BF16)
    assert lib.prism_prologue(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 3, FAKE,
                              None) == B.PRISM_EINVAL
    assert lib.prism_prologue(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE,
                              None) == B.PRISM_EINVAL
    d12 = B.make_dims(1, 10, 1, 12, 64, B.PRISM_BF16)
    assert lib.prism_prologue(ctypes.byref(d12), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, FAKE,
                              None) == B.PRISM_EUNSUPPORTED
    assert lib.prism_scan(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          None) == B.PRISM_EINVAL
    d96 = B.make_dims(1, 10, 1, 64, 96, B.PRISM_BF16)
    assert lib.prism_scan(ctypes.byref(d96), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          None) == B.PRISM_EUNSUPPORTED


def _resume(lib, d, L=2, ws=1 << 30, residual=0, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, g=FAKE, b=FAKE, a=FAKE, h=FAKE, conv_w=FAKE,
                cu=FAKE, s0=None, hist=None, o=FAKE, s=FAKE, hout=None, w=FAKE)
    args.update(over)
    A = args
    return lib.prism_fwd_resume(ctypes.byref(d), A["q"], A["k"], A["v"], A["u"], A["g"], A["b"],
                                A["a"], A["h"], A["conv_w"], A["cu"], L, residual, A["s0"], A["hist"],
                                A["o"], A["s"], A["hout"], A["w"], ws, None)


def test_fwd_resume_rejects_bad_arguments(lib):
    from gated_delta_rule_prologue_amd import binding as B
    ok = B.make_dims(1, 10, 1, 64, 64, B.PRISM_BF16)
    # the optional pointers must be aligned when given
    assert _resume(lib, ok, s0=FAKE + 4) == B.PRISM_EINVAL
    assert _resume(lib, ok, hist=FAKE + 2) == B.PRISM_EINVAL
    assert _resume(lib, ok, hout=FAKE + 8) == B.PRISM_EINVAL
    assert _resume(lib, ok, s=None) == B.PRISM_EINVAL
    assert _resume(lib, ok, L=0) == B.PRISM_EINVAL
    assert _resume(lib, ok, ws=16) == B.PRISM_EINVAL
    assert _resume(lib, B.make_dims(1, 10, 1, 96, 64, B.PRISM_BF16)) == B.PRISM_EUNSUPPORTED
    assert _resume(lib, ok, residual=2) == B.PRISM_EINVAL
    assert _resume(lib, ok, residual=-1) == B.PRISM_EINVAL


def _decode(lib, d, L=2, residual=0, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, u=FAKE, g=FAKE, b=FAKE, a=FAKE, h=FAKE, conv_w=FAKE,
                S=FAKE, hist=FAKE, o=FAKE)
    args.update(over)
    A = args
    return lib.prism_decode_step(ctypes.byref(d), A["q"], A["k"], A["v"], A["u"], A["g"], A["b"],
                                 A["a"], A["h"], A["conv_w"], L, residual, A["S"], A["hist"],
                                 A["o"], None)


def test_decode_step_rejects_bad_arguments(lib):
    from gated_delta_rule_prologue_amd import binding as B
    ok = B.make_dims(4, 4, 2, 64, 64, B.PRISM_BF16)
    assert _decode(lib, B.make_dims(4, 5, 2, 64, 64, B.PRISM_BF16)) == B.PRISM_EINVAL  # one token each
    assert _decode(lib, ok, S=None) == B.PRISM_EINVAL
    assert _decode(lib, ok, hist=None) == B.PRISM_EINVAL
    assert _decode(lib, ok, hist=FAKE + 2) == B.PRISM_EINVAL
    assert _decode(lib, ok, u=None) == B.PRISM_EINVAL
    assert _decode(lib, ok, L=17) == B.PRISM_EINVAL
    assert _decode(lib, B.make_dims(4, 4, 2, 96, 64, B.PRISM_BF16)) == B.PRISM_EUNSUPPORTED
    assert _decode(lib, B.make_dims(4, 4, 2, 64, 32, B.PRISM_F32)) == B.PRISM_EUNSUPPORTED
    assert _decode(lib, ok, residual=5) == B.PRISM_EINVAL


def test_prologue_ex_rejects_bad_arguments(lib):
    from gated_delta_rule_prologue_amd import binding as B
    d = B.make_dims(1, 10, 1, 64, 64, B.PRISM_BF16)
    call = lambda L=3, residual=1, hist=None, kw=FAKE: lib.prism_prologue_ex(
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, hist, FAKE, L, residual, kw, None)
    assert call(residual=2) == B.PRISM_EINVAL
    assert call(hist=FAKE + 2) == B.PRISM_EINVAL
    assert call(kw=None) == B.PRISM_EINVAL
    assert call(L=17) == B.PRISM_EINVAL


def test_bwd_ex_rejects_bad_arguments(lib):
    from gated_delta_rule_prologue_amd import binding as B
    d = B.make_dims(1, 10, 1, 64, 64, B.PRISM_BF16)
    call = lambda L=3, residual=1, dq=FAKE, ws=1 << 30: lib.prism_bwd_ex(
        ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, L, residual,
        None, FAKE, None, dq, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None)
    assert call(residual=2) == B.PRISM_EINVAL
    assert call(residual=-1) == B.PRISM_EINVAL
    assert call(L=0) == B.PRISM_EINVAL
    assert call(dq=None) == B.PRISM_EINVAL
    assert call(ws=16) == B.PRISM_EINVAL
    d96 = B.make_dims(1, 10, 1, 96, 64, B.PRISM_BF16)
    assert lib.prism_bwd_ex(
        ctypes.byref(d96), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 1,
        None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
        1 << 30, None) == B.PRISM_EUNSUPPORTED


def test_binding_checks_shapes_before_calling():
    torch = pytest.importorskip("torch")
    from gated_delta_rule_prologue_amd import binding as B
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        B.scan(q, q, q, q, torch.zeros(4, 3, dtype=torch.bfloat16), torch.zeros(4, 2), cu)
    with pytest.raises(ValueError):
        B.prologue(q, None, None, None, torch.zeros(4, 2, dtype=torch.bfloat16),
                   torch.zeros(2, 64, 4, dtype=torch.bfloat16), cu.to(torch.int64), 1)


def test_scan_workspace_bytes_for_forced_split(lib, monkeypatch):
    """With PRISM_SPLIT=P the scan workspace holds o' (bf16 [T, H, dk]), S_loc and
    S_in (fp32 [n P, H, dk, dv]), M (fp32 [n P, H, dk, dk]) and the segment
    offsets, each rounded up to 256 bytes; prism_workspace_bytes adds the write
    keys.  Off (PRISM_SPLIT=0), and for fp32 inputs, it is zero (the
    opt-in two-pass scan then needs its per-chunk matrices)."""
    from gated_delta_rule_prologue_amd import binding as B
    up = lambda x: (x + 255) // 256 * 256
    n, T, H, dk, dv, P = 2, 1000, 3, 128, 64, 3
    d = B.make_dims(n, T, H, dk, dv, B.PRISM_BF16)
    monkeypatch.setenv("PRISM_SPLIT", str(P))
    segs = n * P
    want = (up(T * H * dk * 2) + 2 * up(segs * H * dk * dv * 4) + up(segs * H * dk * dk * 4)
            + up((segs + 1) * 4))
    assert B.scan_workspace_bytes(d) == want
    assert B.workspace_bytes(d, 4) == up(T * H * dk * 2) + want
    monkeypatch.setenv("PRISM_SPLIT", "0")
    assert B.scan_workspace_bytes(d) == 0
    monkeypatch.setenv("PRISM_SCAN_TWOPASS", "1")
    assert B.scan_workspace_bytes(d) == up((T // 64 + n) * H * 20480)   # two-pass matrices
    monkeypatch.delenv("PRISM_SCAN_TWOPASS")
    monkeypatch.setenv("PRISM_SPLIT", str(P))
    assert B.scan_workspace_bytes(B.make_dims(n, T, H, 64, 64, B.PRISM_F32)) == 0


def test_bwd_workspace_bytes_both_paths(lib, monkeypatch):
    """prism_bwd_workspace_bytes.  bf16 (the chunkwise backward, default): write
    keys, per-chunk matrices (20 KB per head and virtual chunk), four bf16 state
    checkpoints (dk x dv per head and virtual chunk), dkw (fp32 [T, H, dk]) and
    the dconv_w partials (per 64-token block and per slab of 16 blocks, 4 H dk
    floats each), every part rounded up to 256 bytes.  fp32, or
    PRISM_BWD_CHUNKED=0: the token walk's checkpoints, segment gradients, dkw and
    the same partials, after the write keys."""
    up = lambda x: (x + 255) // 256 * 256
    n, T, H, dk, dv, L = 3, 1000, 2, 128, 64, 4
    nv = (T // 64 + n) * H
    nb = (T + 63) // 64
    wk = (nb + (nb + 15) // 16) * H * dk * 4
    chunked = (up(T * H * dk * 2) + up(nv * 20480) + 4 * up(nv * dk * dv * 2) + up(T * H * dk * 4)
               + up(wk * 4))
    walk = lambda e, s: up(T * H * dk * e) + 4 * ((T // s + n + 1) * H * dk * dv + n * 8 * H * dk * dv
                                                  + T * H * dk + wk)
    from gated_delta_rule_prologue_amd import binding as B
    d16 = B.make_dims(n, T, H, dk, dv, B.PRISM_BF16)
    d32 = B.make_dims(n, T, H, dk, dv, B.PRISM_F32)
    lib.prism_bwd_workspace_bytes.restype = ctypes.c_size_t
    monkeypatch.delenv("PRISM_BWD_CHUNKED", raising=False)
    assert lib.prism_bwd_workspace_bytes(ctypes.byref(d16), L) == chunked
    assert lib.prism_bwd_workspace_bytes(ctypes.byref(d32), L) == walk(4, 4)
    monkeypatch.setenv("PRISM_BWD_CHUNKED", "0")
    assert lib.prism_bwd_workspace_bytes(ctypes.byref(d16), L) == walk(2, 4)
    monkeypatch.setenv("PRISM_BWD_CHUNKED", "1")
    # no tokens: the token walk (the chunkwise form needs at least one chunk)
    e16 = B.make_dims(n, 0, H, dk, dv, B.PRISM_BF16)
    assert lib.prism_bwd_workspace_bytes(ctypes.byref(e16), L) == 256 + 4 * ((n + 1) * H * dk * dv
                                                                           + n * 8 * H * dk * dv)


def test_checkpoint_bytes_and_argument_checks(lib):
    """prism_checkpoint_bytes: two bf16 arrays of floor(T / 64) + n_seqs
    chunk-start states per head (rows and transposes) and the bf16 write keys
    [T, H, dk], each 256-byte rounded (kw at least 256), for the shapes the
    chunkwise backward serves; 0 elsewhere.  The checkpoint entry points reject
    a null buffer and unserved shapes before touching the device."""
    from gated_delta_rule_prologue_amd import binding as B
    up = lambda x: (x + 255) // 256 * 256
    d = B.make_dims(8, 16384, 6, 128, 128, B.PRISM_BF16)
    assert B.checkpoint_bytes(d) == 2 * up((16384 // 64 + 8) * 6 * 128 * 128 * 2) + up(16384 * 6 * 128 * 2)
    assert B.checkpoint_bytes(B.make_dims(3, 100, 2, 64, 128, B.PRISM_BF16)) == \
        2 * up((1 + 3) * 2 * 64 * 128 * 2) + up(100 * 2 * 64 * 2)
    assert B.checkpoint_bytes(B.make_dims(2, 0, 1, 64, 64, B.PRISM_BF16)) == 2 * up(2 * 64 * 64 * 2) + 256
    assert B.checkpoint_bytes(B.make_dims(1, 100, 1, 64, 64, B.PRISM_F32)) == 0
    assert B.checkpoint_bytes(B.make_dims(1, 100, 1, 32, 64, B.PRISM_BF16)) == 0
    assert B.checkpoint_bytes(B.make_dims(0, 0, 1, 64, 64, B.PRISM_BF16)) == 0
    fwd = lambda d, ck: lib.prism_fwd_ckpt(ctypes.byref(d), *([FAKE] * 10), 2, 0, None, FAKE, FAKE, ck,
                                           FAKE, 1 << 30, None)
    bwd = lambda d, ck, gd=B.PRISM_F32: lib.prism_bwd_ckpt(ctypes.byref(d), *([FAKE] * 10), 2, 0, gd, None,
                                                           FAKE, None, *([FAKE] * 9), None, ck, FAKE,
                                                           1 << 30, None)
    ok = B.make_dims(2, 100, 2, 64, 64, B.PRISM_BF16)
    assert fwd(ok, None) == B.PRISM_EINVAL and bwd(ok, None) == B.PRISM_EINVAL
    assert bwd(ok, FAKE, 2) == B.PRISM_EINVAL and bwd(ok, FAKE, -1) == B.PRISM_EINVAL
    f32 = B.make_dims(2, 100, 2, 64, 64, B.PRISM_F32)
    assert fwd(f32, FAKE) == B.PRISM_EUNSUPPORTED and bwd(f32, FAKE) == B.PRISM_EUNSUPPORTED
