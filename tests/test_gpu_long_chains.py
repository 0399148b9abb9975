"""Chains longer than one drafting block on the matrix cores (the chunked chain
kernel): outputs and final states against the oracle for bf16 and fp32 inputs
at head sizes 64 and 128, with chain lengths and final lengths on and off the
16-token chunk boundaries, an empty chain, outputs alone and final states
alone."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import TOL, require_gpu, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

LENS = [64, 17, 5, 40, 33, 16, 0, 200]
FINAL = [64, 16, 0, 33, 32, 7, 0, 150]


def _unit(rng, *shape):
    g = rng.standard_normal(shape)
    return g / np.linalg.norm(g, axis=-1, keepdims=True)


def _case(rng, d_, dtype, hk=2, hv=4):
    cu = np.zeros(len(LENS) + 1, np.int32)
    cu[1:] = np.cumsum(LENS)
    T = int(cu[-1])
    x = {"q": _unit(rng, T, hk, d_).astype(np.float32), "k": _unit(rng, T, hk, d_).astype(np.float32),
         "v": rng.standard_normal((T, hv, d_)).astype(np.float32),
         "a": rng.uniform(0.5, 1.0, (T, hv)).astype(np.float32),
         "b": rng.uniform(0.0, 1.0, (T, hv)).astype(np.float32)}
    if dtype == "bf16":
        for key in ("q", "k", "v"):
            x[key] = W.f32_to_bf16_bits(x[key])
    S0 = (0.3 * rng.standard_normal((len(LENS), hv, d_, d_))).astype(np.float32)
    return cu, T, x, S0


@pytest.mark.parametrize("d_", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["both", "outputs", "final"])
def test_chunked_chains(d_, dtype, mode, monkeypatch):
    G = require_gpu()
    monkeypatch.delenv("GDN_KERNEL_PATH", raising=False)
    rng = np.random.default_rng(6000 + d_ + (1 if dtype == "f32" else 0))
    hk, hv = 2, 4
    cu, T, inp, S0 = _case(rng, d_, dtype, hk, hv)
    tol = TOL if dtype == "bf16" else 1e-4
    B = len(LENS)
    slots = np.arange(B, dtype=np.int32)
    dims = G.make_dims(B, T, max(LENS), hk, hv, d_, B, G.GDN_BF16 if dtype == "bf16" else G.GDN_F32)
    dev = {k: to_dev(v) for k, v in inp.items()}
    want_out, want_fin = mode in ("both", "outputs"), mode in ("both", "final")
    out = torch.full((T, hv, d_), float("nan"), device="cuda") if want_out else None
    fin = torch.full((B, hv, d_, d_), float("nan"), device="cuda") if want_fin else None
    fl = np.array(FINAL, np.int32)
    print("chunked chains d=%d %s %s" % (d_, dtype, mode), flush=True)
    ws = G.new_workspace(dims)
    G.gdn_chain_verify(dims, to_dev(cu), dev["q"] if want_out else None, dev["k"], dev["v"], dev["a"], dev["b"],
                       to_dev(S0), to_dev(slots), out, to_dev(fl) if want_fin else None, fin, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    for s, L in enumerate(LENS):
        lo, hi = int(cu[s]), int(cu[s + 1])
        sl = {k: v[lo:hi] for k, v in inp.items()}
        if want_out and L > 0:
            ref, _ = oracle.chain(sl["k"], sl["v"], sl["a"], sl["b"], S0[s], q=sl["q"])
            got = out[lo:hi].cpu().numpy()
            assert slice_rel_err(got.transpose(1, 0, 2).reshape(hv, -1), ref.transpose(1, 0, 2).reshape(hv, -1)) <= tol, s
        if want_fin:
            f = int(fl[s])
            _, ref_fin = oracle.chain(sl["k"][:f], sl["v"][:f], sl["a"][:f], sl["b"][:f], S0[s])
            g = fin[s].cpu().numpy()
            if f == 0:
                assert np.array_equal(g, S0[s]), s
            else:
                assert slice_rel_err(g.reshape(hv, -1), ref_fin.reshape(hv, -1)) <= tol, s


def test_chunked_chain_matches_recurrent_walk(monkeypatch):
    """The chunked kernel and the recurrent chain walk agree to the parity bar on a
    300-token chain at d = 128 (bf16), outputs and the state after 287 tokens."""
    G = require_gpu()
    rng = np.random.default_rng(6100)
    hk, hv, d_, n = 2, 6, 128, 300
    inp = {"q": W.f32_to_bf16_bits(_unit(rng, n, hk, d_).astype(np.float32)),
           "k": W.f32_to_bf16_bits(_unit(rng, n, hk, d_).astype(np.float32)),
           "v": W.f32_to_bf16_bits(rng.standard_normal((n, hv, d_)).astype(np.float32)),
           "a": rng.uniform(0.7, 1.0, (n, hv)).astype(np.float32), "b": rng.uniform(0.0, 1.0, (n, hv)).astype(np.float32)}
    S0 = (0.3 * rng.standard_normal((1, hv, d_, d_))).astype(np.float32)
    dims = G.make_dims(1, n, n, hk, hv, d_, 1, G.GDN_BF16)
    dev = {k: to_dev(v) for k, v in inp.items()}
    res = []
    for path in ("auto", "recurrent"):
        if path == "recurrent":
            monkeypatch.setenv("GDN_KERNEL_PATH", "recurrent")
        else:
            monkeypatch.delenv("GDN_KERNEL_PATH", raising=False)
        out = torch.full((n, hv, d_), float("nan"), device="cuda")
        fin = torch.full((1, hv, d_, d_), float("nan"), device="cuda")
        G.gdn_chain_verify(dims, to_dev(np.array([0, n], np.int32)), dev["q"], dev["k"], dev["v"], dev["a"],
                           dev["b"], to_dev(S0), to_dev(np.zeros(1, np.int32)), out,
                           to_dev(np.array([287], np.int32)), fin, G.new_workspace(dims))
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), fin.cpu().numpy()))
    (o1, f1), (o2, f2) = res
    assert slice_rel_err(o1.transpose(1, 0, 2).reshape(hv, -1), o2.transpose(1, 0, 2).reshape(hv, -1)) <= TOL
    assert slice_rel_err(f1[0].reshape(hv, -1), f2[0].reshape(hv, -1)) <= TOL
