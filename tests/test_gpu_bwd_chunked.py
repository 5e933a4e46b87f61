"""GPU parity of the two bf16 backward paths, each selected explicitly: the
chunkwise form (PRISM_BWD_CHUNKED=1, the default: the forward state products
again with each chunk's start state kept, the carried state gradient chunk by
chunk, then every input gradient of all chunks at once on MFMA) and the token
walk (PRISM_BWD_CHUNKED=0).  Checked against the fp64 oracle's backward
(pinned against finite differences and torch autograd), every gradient, at
the bf16 tolerance, and against each other."""
import numpy as np
import pytest

from gated_delta_rule_prologue_amd.configs import BY_NAME, Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs
from tests.gpu_common import TOL, max_rel, say
from tests.test_gpu_bwd import NAMES, W, check, run

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_prologue_amd import binding
    binding.lib()


@pytest.fixture
def chunked(monkeypatch):
    monkeypatch.setenv("PRISM_BWD_CHUNKED", "1")


@pytest.fixture
def token_walk(monkeypatch):
    monkeypatch.setenv("PRISM_BWD_CHUNKED", "0")


def _chunked_ws_bytes(inp):
    """The chunkwise path's workspace, laid out as the library lays it out
    (write keys, per-chunk matrices, four bf16 state checkpoints, dkw, the
    write-key backward's partial sums of dconv_w; 256-byte parts)."""
    r = lambda n: (n + 255) // 256 * 256
    T, H, dk, dv, n = inp.total_tokens, inp.heads, inp.dk, inp.dv, inp.n_seqs
    nv = (T // 64 + n) * H
    nb = (T + 63) // 64                            # write-key blocks and their slabs of 16
    wk = (nb + (nb + 15) // 16) * H * dk * 4 * 4
    return (max(r(T * H * dk * 2), 256) + r(nv * 20480) + 4 * r(nv * dk * dv * 2)
            + r(T * H * dk * 4) + r(wk))


CASES = [
    # ragged chunks, empty and one-token sequences, a sequence of exactly one chunk
    W(dk=64, dv=64, L=4, lengths=(150, 1, 0, 70, 64)),
    W(dk=128, dv=128, L=4, lengths=(200, 65)),
    W(dk=64, dv=128, L=1, lengths=(90, 3)),
    W(dk=128, dv=64, L=8, lengths=(70, 129), H=3),
    W(dk=64, dv=64, L=16, lengths=(40, 3)),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: f"dk{w.dk}-dv{w.dv}-L{w.L}-{len(w.lengths)}seq")
def test_chunked_bwd_matches_oracle(w, chunked):
    from gated_delta_rule_prologue_amd import binding
    inp = make_inputs(w)
    d = binding.make_dims(inp.n_seqs, inp.total_tokens, inp.heads, inp.dk, inp.dv, binding.PRISM_BF16)
    assert int(binding.lib().prism_bwd_workspace_bytes(d, inp.L)) == _chunked_ws_bytes(inp), \
        "the chunkwise path is not the one taken"
    say(f"chunked bwd {w}")
    got, ref = run(inp)
    check(got, ref, "bf16")


@pytest.mark.parametrize("w", CASES[:2], ids=lambda w: f"dk{w.dk}-dv{w.dv}-L{w.L}")
def test_token_walk_bwd_matches_oracle(w, token_walk):
    inp = make_inputs(w)
    say(f"token-walk bwd {w}")
    got, ref = run(inp)
    check(got, ref, "bf16")


def test_chunked_bwd_without_carried_state(chunked):
    inp = make_inputs(W(dk=64, dv=64, L=2, lengths=(100, 40)))
    got, ref = run(inp, with_state=False)
    check(got, ref, "bf16")


@pytest.mark.parametrize("g_mu", [-1.0, -3.0])
def test_chunked_bwd_strong_decay(g_mu, chunked):
    """Forget gates near zero: the in-chunk cumulative decay underflows fp32
    within a chunk, so every factor of it must stay finite."""
    inp = make_inputs(W(dk=64, dv=64, L=4, lengths=(300, 17), g_mu=g_mu))
    got, ref = run(inp)
    check(got, ref, "bf16")


def test_chunked_bwd_gelu(chunked):
    from tests.test_gpu_gelu import amplify
    inp = amplify(make_inputs(W(dk=128, dv=128, L=5, lengths=(200, 65))))
    got, ref = run(inp, residual="gelu")
    check(got, ref, "bf16")


def test_chunked_agrees_with_token_recurrent(monkeypatch):
    """Both backward paths on the same inputs: they differ by rounding only."""
    import torch
    from gated_delta_rule_prologue_amd import binding
    from tests.test_gpu_state import dev_tensor
    inp = make_inputs(W(dk=64, dv=64, L=4, lengths=(300, 64, 5)))
    rng = np.random.default_rng(9)
    from gated_delta_rule_prologue_amd.inputs import f32_to_bf16_bits
    d_o = dev_tensor(f32_to_bf16_bits(rng.standard_normal(
        (inp.total_tokens, inp.heads, inp.dv)).astype(np.float32)))
    dev = binding.to_device(inp)

    def go():
        g = binding.bwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"],
                        dev["h"], dev["conv_w"], dev["cu_seqlens"], inp.L, d_o)
        torch.cuda.synchronize()
        return {n: g[n].cpu().numpy().astype(np.float64) for n in NAMES if g[n] is not None}

    monkeypatch.setenv("PRISM_BWD_CHUNKED", "0")
    a = go()
    monkeypatch.setenv("PRISM_BWD_CHUNKED", "1")
    b = go()
    for n in a:
        err = max_rel(b[n], a[n])
        say(f"  d{n} chunked vs token-recurrent {err:.3e}")
        assert err <= TOL["bf16"], (n, err)


@pytest.mark.parametrize("name,chains", [("lm-130m-layer", [5, 37]),
                                         ("recsys-history", [0, 77, 130, 255])])
def test_token_walk_bwd_full_size_sampled_chains(name, chains, token_walk):
    """The LM layer (B=8, T=2048, H=6, d=128, L=4) and the recommendation
    histories (B=64, T=1024, H=4, d=64, L=4) on the token walk (the default
    path's full-size cases are in test_gpu_bwd.py): every gradient of sampled
    chains."""
    w = BY_NAME[name]
    inp = make_inputs(w)
    say(f"chunked {name}: chains {chains}")
    got, ref = run(inp, with_state=False, chains=chains)
    H = inp.heads
    rows = np.zeros((inp.total_tokens, H), dtype=bool)
    for c in chains:
        n, e = divmod(c, H)
        rows[inp.cu_seqlens[n]:inp.cu_seqlens[n + 1], e] = True
    masks = {n: rows for n in ("q", "k", "v", "u", "a", "h", "g", "b")}
    smask = np.zeros((inp.n_seqs, H), dtype=bool)
    for c in chains:
        smask[divmod(c, H)] = True
    masks["S_init"] = smask
    ref["conv_w"] = None
    check(got, ref, "bf16", masks)
