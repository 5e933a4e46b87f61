"""GPU parity: libprism (HIP, gfx950) against the fp64 oracle, through the C ABI.

Every test compares every element of o and S_final, the five full-size
workloads included (in the launch configuration the benchmark times).
"""
import os

import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import WORKLOADS, Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs, to_float, f32_to_bf16_bits
from tests.gpu_common import TOL, TOL_KW, gpu_fwd, gpu_prologue, max_rel, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()          # fails loudly if libprism.so is missing


def W(name="t", H=2, dk=64, dv=64, L=4, dtype="bf16", lengths=(100,), seed=5, g_mu=3.0):
    return Workload(name, heads=H, dk=dk, dv=dv, L=L, dtype=dtype, seed=seed,
                    lengths=list(lengths), g_mu=g_mu)


# ----------------------------------------------------------------------------- prologue
PROLOGUE_CASES = [
    W(dtype="f32", dk=64, L=2, lengths=(256,)),
    W(dtype="f32", dk=64, L=5, lengths=(3, 0, 70, 1, 2, 129)),
    W(dtype="bf16", dk=64, L=4, lengths=(17, 0, 64, 5)),
    W(dtype="bf16", dk=128, L=4, lengths=(300, 33)),
    W(dtype="bf16", dk=128, L=1, lengths=(40,)),
    W(dtype="bf16", dk=64, L=16, lengths=(20, 9)),
    W(dtype="bf16", dk=16, L=3, H=3, lengths=(31, 0, 2)),
]


@pytest.mark.parametrize("w", PROLOGUE_CASES, ids=lambda w: f"{w.dtype}-dk{w.dk}-L{w.L}-{len(w.lengths)}seq")
def test_prologue_matches_oracle(w):
    inp = make_inputs(w)
    say(f"prologue {w}")
    kw = gpu_prologue(inp)
    ref = oracle.prologue(inp)
    err = max_rel(kw, ref)
    say(f"  kw max-rel err {err:.3e}")
    assert err <= TOL_KW[w.dtype]


def test_prologue_residual_amplified():
    """u unnormalised x10 and a ~ U(0,1): the residual levels dominate kw."""
    inp = make_inputs(W(dtype="bf16", dk=128, L=4, lengths=(90, 7)))
    rng = np.random.default_rng(9)
    inp.u[:] = f32_to_bf16_bits(10.0 * to_float(inp.u) * np.sqrt(inp.dk))
    inp.a[:] = f32_to_bf16_bits(rng.uniform(0, 1, inp.a.shape).astype(np.float32))
    kw = gpu_prologue(inp)
    ref = oracle.prologue(inp)
    bk = to_float(inp.b)[:, :, None].astype(np.float64) * to_float(inp.k)
    assert np.max(np.abs(ref - bk)) > 5 * np.max(np.abs(bk))      # residual part dominates
    assert max_rel(kw, ref) <= TOL_KW["bf16"]


# ----------------------------------------------------------------------------- forward
FWD_CASES = [
    W(dtype="f32", dk=64, dv=64, L=2, lengths=(256,)),
    W(dtype="f32", dk=64, dv=64, L=4, lengths=(256,)),              # strict-tolerance run of h
    W(dtype="f32", dk=64, dv=64, L=3, lengths=(1, 64, 65, 0, 130)),
    W(dtype="f32", dk=128, dv=128, L=4, lengths=(300, 1, 0, 77, 64)),  # token-recurrent fp32
    W(dtype="f32", dk=128, dv=64, L=2, lengths=(129, 5)),
    W(dtype="bf16", dk=64, dv=64, L=4, lengths=(200, 64, 1, 0, 77)),
    W(dtype="bf16", dk=128, dv=128, L=4, lengths=(300, 63)),
    W(dtype="bf16", dk=128, dv=128, L=1, lengths=(257,)),           # exact GDN
    W(dtype="bf16", dk=128, dv=64, L=2, lengths=(150,)),
    W(dtype="bf16", dk=64, dv=128, L=2, lengths=(150,)),
    W(dtype="bf16", dk=64, dv=64, L=3, lengths=(190,), g_mu=-2.0),  # strong decay
    W(dtype="bf16", dk=128, dv=128, L=8, lengths=(129,), H=1),
]


@pytest.mark.parametrize("w", FWD_CASES,
                         ids=lambda w: f"{w.dtype}-dk{w.dk}-dv{w.dv}-L{w.L}-g{w.g_mu}-{len(w.lengths)}seq")
def test_fwd_matches_oracle(w):
    inp = make_inputs(w)
    say(f"fwd {w}")
    o, s = gpu_fwd(inp)
    o_ref, s_ref = oracle.fwd(inp)
    eo, es = max_rel(o, o_ref), max_rel(s, s_ref)
    say(f"  o err {eo:.3e}  S err {es:.3e}")
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


SCAN_KERNELS = {                 # environment selecting each bf16 scan kernel
    "twopass": {"PRISM_SCAN_GENERIC": "0", "PRISM_SCAN_TWOPASS": "1"},
    "specialised": {"PRISM_SCAN_GENERIC": "0", "PRISM_SCAN_TWOPASS": "0", "PRISM_SCAN_SPECIALISED": "1",
                    "PRISM_SCAN_WAVES": "8"},
    "specialised4": {"PRISM_SCAN_GENERIC": "0", "PRISM_SCAN_TWOPASS": "0", "PRISM_SCAN_SPECIALISED": "1",
                     "PRISM_SCAN_WAVES": "4"},
    "register": {"PRISM_SCAN_GENERIC": "0", "PRISM_SCAN_TWOPASS": "0", "PRISM_SCAN_SPECIALISED": "0"},
    "generic": {"PRISM_SCAN_GENERIC": "1"},
}


# (kernel, slice width) pairs that exist: the two-pass scan takes slices of 32
# value columns, the wavefront-specialised kernels 16 and 32, the others 16, 32
# and 64
SLICE_CASES = [(k, dvs) for k in SCAN_KERNELS for dvs in (16, 32, 64)
               if not (k.startswith("specialised") and dvs == 64) and not (k == "twopass" and dvs != 32)]


@pytest.mark.parametrize("kernel,dvs", SLICE_CASES, ids=[f"{k}-{d}" for k, d in SLICE_CASES])
@pytest.mark.parametrize("dk", [64, 128])
def test_every_value_slice_width(dk, dvs, kernel, monkeypatch):
    """Every bf16 scan kernel at every value-slice width it has; sequences of
    0, 1, 2 and 3 chunks with full and ragged last chunks."""
    monkeypatch.setenv("PRISM_DV_SLICE", str(dvs))
    for key, val in SCAN_KERNELS[kernel].items():
        monkeypatch.setenv(key, val)
    inp = make_inputs(W(dtype="bf16", dk=dk, dv=64, L=3, lengths=(140, 3, 0, 64, 128, 65)))
    o, s = gpu_fwd(inp)
    o_ref, s_ref = oracle.fwd(inp)
    say(f"{kernel} dk {dk} dvs {dvs}: o {max_rel(o, o_ref):.3e} S {max_rel(s, s_ref):.3e}")
    assert max_rel(o, o_ref) <= TOL["bf16"] and max_rel(s, s_ref) <= TOL["bf16"]


@pytest.mark.parametrize("kernel", ["twopass", "specialised", "specialised4", "register"])
def test_bf16_kernels_long_sequence(kernel, monkeypatch):
    """Dozens of chunks through one chain: the double-buffered matrices and the
    staged rows alternate many times."""
    monkeypatch.setenv("PRISM_DV_SLICE", "32")
    for key, val in SCAN_KERNELS[kernel].items():
        monkeypatch.setenv(key, val)
    inp = make_inputs(W(dtype="bf16", dk=128, dv=128, L=4, H=1, lengths=(2000, 37)))
    o, s = gpu_fwd(inp)
    o_ref, s_ref = oracle.fwd(inp)
    say(f"{kernel} long: o {max_rel(o, o_ref):.3e} S {max_rel(s, s_ref):.3e}")
    assert max_rel(o, o_ref) <= TOL["bf16"] and max_rel(s, s_ref) <= TOL["bf16"]


@pytest.mark.parametrize("dvs", [16, 32])
@pytest.mark.parametrize("lengths", [(130, 0, 64, 300), (65, 1, 128, 7, 200, 0, 90, 33)],
                         ids=["8-chains", "16-chains"])
def test_slices_grouped_per_xcd(dvs, lengths, monkeypatch):
    """Chain counts divisible by eight take the XCD-grouped workgroup order."""
    monkeypatch.setenv("PRISM_DV_SLICE", str(dvs))
    inp = make_inputs(W(dtype="bf16", dk=128, dv=128, L=4, H=2, lengths=lengths))
    o, s = gpu_fwd(inp)
    o_ref, s_ref = oracle.fwd(inp)
    say(f"xcd-grouped dvs {dvs} {lengths}: o {max_rel(o, o_ref):.3e} S {max_rel(s, s_ref):.3e}")
    assert max_rel(o, o_ref) <= TOL["bf16"] and max_rel(s, s_ref) <= TOL["bf16"]


def test_fp32_recurrent_kernel_at_dk64(monkeypatch):
    """The token-recurrent fp32 scan (the fp32 path at dk = 128) forced at
    dk = 64 as well: the same strict tolerance on ragged and empty sequences."""
    monkeypatch.setenv("PRISM_SCAN_RECURRENT", "1")
    inp = make_inputs(W(dtype="f32", dk=64, dv=64, L=4, lengths=(200, 0, 1, 63)))
    o, s = gpu_fwd(inp)
    o_ref, s_ref = oracle.fwd(inp)
    say(f"f32 recurrent dk64: o {max_rel(o, o_ref):.3e} S {max_rel(s, s_ref):.3e}")
    assert max_rel(o, o_ref) <= TOL["f32"] and max_rel(s, s_ref) <= TOL["f32"]


def test_fp32_ignores_unsupported_slice_request(monkeypatch):
    """fp32 has one value-slice width (16); a request for another falls back to it."""
    monkeypatch.setenv("PRISM_DV_SLICE", "32")
    inp = make_inputs(W(dtype="f32", dk=64, dv=128, L=4, lengths=(200,)))
    o, s = gpu_fwd(inp)
    o_ref, s_ref = oracle.fwd(inp)
    assert max_rel(o, o_ref) <= TOL["f32"] and max_rel(s, s_ref) <= TOL["f32"]


def test_scan_alone_from_oracle_write_keys():
    """prism_scan fed with the oracle's write keys (rounded to the input dtype)."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    inp = make_inputs(W(dtype="bf16", dk=128, dv=128, L=4, lengths=(192, 50)))
    kw_ref = oracle.prologue(inp)
    dev = binding.to_device(inp)
    kw = torch.from_numpy(f32_to_bf16_bits(kw_ref.astype(np.float32))).view(torch.bfloat16).cuda()
    o, s = binding.scan(dev["q"], dev["k"], kw, dev["v"], dev["g"], dev["b"], dev["cu_seqlens"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd(inp)
    assert max_rel(to_host(o), o_ref) <= TOL["bf16"]
    assert max_rel(to_host(s), s_ref) <= TOL["bf16"]


def test_all_sequences_empty():
    import torch
    from gated_delta_rule_prologue_amd import binding
    inp = make_inputs(W(dtype="bf16", dk=64, dv=64, L=2, lengths=(0, 0, 0)))
    dev = binding.to_device(inp)
    s = torch.full((3, 2, 64, 64), 7.0, device="cuda")
    o, s = binding.fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"],
                       dev["h"], dev["conv_w"], dev["cu_seqlens"], inp.L, S_final=s)
    torch.cuda.synchronize()
    assert o.numel() == 0 and not s.any()


@pytest.mark.parametrize("w", [FWD_CASES[3], FWD_CASES[4], FWD_CASES[8]],
                         ids=["dk64-varlen", "dk128", "strong-decay"])
def test_generic_bf16_kernel(w, monkeypatch):
    monkeypatch.setenv("PRISM_SCAN_GENERIC", "1")
    inp = make_inputs(w)
    o, s = gpu_fwd(inp)
    o_ref, s_ref = oracle.fwd(inp)
    assert max_rel(o, o_ref) <= TOL["bf16"] and max_rel(s, s_ref) <= TOL["bf16"]


def test_deterministic():
    inp = make_inputs(W(dtype="bf16", dk=128, dv=128, L=4, lengths=(333, 21)))
    o1, s1 = gpu_fwd(inp)
    o2, s2 = gpu_fwd(inp)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


# ----------------------------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("idx", range(len(WORKLOADS)), ids=[w.name for w in WORKLOADS])
def test_workload_parity(idx):
    """The five workloads at full size: every element of o and S_final of every
    (sequence, head) chain against the oracle."""
    w = WORKLOADS[idx]
    say(f"workload {w.name}: generating")
    inp = make_inputs(w)
    say(f"workload {w.name}: T={inp.total_tokens} chains={inp.n_seqs * inp.heads}")
    o, s = gpu_fwd(inp)
    say(f"workload {w.name}: oracle")
    o_ref, s_ref = oracle.fwd(inp)
    eo, es = max_rel(o, o_ref), max_rel(s, s_ref)
    say(f"workload {w.name}: o err {eo:.3e} S err {es:.3e}")
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]
