"""Pins of the oracle's activations and gated MLP (oracle/qlora.py).

- activations: special values and limits, torch's silu and tanh-GELU, torch
  autograd derivatives and scalar central differences over [-20, 20];
- MLP backward: central finite differences of <dY, Y> for dX and all six LoRA
  factors on tiny shapes, both activations; torch autograd;
- B = 0 on every projection reduces to the plain gated MLP;
- the per-row helper equals the full computation on its rows.
"""
import numpy as np
import pytest
import torch

from oracle import qlora as Q

ACTS = ["swiglu", "geglu_tanh"]


def test_activation_special_values():
    z = np.array([0.0])
    assert Q.silu(z)[0] == 0.0 and Q.silu_grad(z)[0] == 0.5
    assert Q.gelu_tanh(z)[0] == 0.0 and Q.gelu_tanh_grad(z)[0] == 0.5
    big = np.array([40.0, -40.0])
    assert np.allclose(Q.silu_grad(big), [1.0, 0.0], atol=1e-12)
    assert np.allclose(Q.gelu_tanh_grad(big), [1.0, 0.0], atol=1e-12)
    assert np.allclose(Q.silu(big), [40.0, 0.0], atol=1e-12)
    assert np.allclose(Q.gelu_tanh(big), [40.0, 0.0], atol=1e-12)


def test_activations_match_torch():
    x = np.linspace(-20, 20, 4001)
    t = torch.tensor(x, requires_grad=True)
    ref = torch.nn.functional.silu(t)
    ref.sum().backward()
    assert np.allclose(Q.silu(x), ref.detach().numpy(), rtol=1e-14, atol=1e-15)
    assert np.allclose(Q.silu_grad(x), t.grad.numpy(), rtol=1e-13, atol=1e-13)
    t = torch.tensor(x, requires_grad=True)
    ref = torch.nn.functional.gelu(t, approximate="tanh")
    ref.sum().backward()
    assert np.allclose(Q.gelu_tanh(x), ref.detach().numpy(), rtol=1e-14, atol=1e-15)
    assert np.allclose(Q.gelu_tanh_grad(x), t.grad.numpy(), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("act", ACTS)
def test_activation_derivative_central_difference(act):
    f, fp = Q.ACTS[act]
    x = np.linspace(-20, 20, 801)
    h = 1e-5
    fd = (f(x + h) - f(x - h)) / (2 * h)
    assert np.max(np.abs(fd - fp(x))) < 1e-8


def _mlp_case(m=4, d=64, h=128, r=2, seed=0):
    g = np.random.default_rng(seed)
    X = g.standard_normal((m, d))
    W = dict(Wg=g.standard_normal((h, d)) * 0.1, Wu=g.standard_normal((h, d)) * 0.1,
             Wd=g.standard_normal((d, h)) * 0.1)
    L = dict(Ag=g.standard_normal((r, d)) * 0.2, Bg=g.standard_normal((h, r)) * 0.2,
             Au=g.standard_normal((r, d)) * 0.2, Bu=g.standard_normal((h, r)) * 0.2,
             Ad=g.standard_normal((r, h)) * 0.2, Bd=g.standard_normal((d, r)) * 0.2)
    dY = g.standard_normal((m, d))
    return X, W, L, dY


def _fwd(X, W, L, s, act):
    return Q.mlp_fwd(X, W["Wg"], W["Wu"], W["Wd"], L["Ag"], L["Bg"], L["Au"], L["Bu"],
                     L["Ad"], L["Bd"], s, act)


@pytest.mark.parametrize("act", ACTS)
def test_mlp_backward_matches_central_differences(act):
    X, W, L, dY = _mlp_case(seed=1)
    s = 1.5
    _, sv = _fwd(X, W, L, s, act)
    gr = Q.mlp_bwd(dY, X, sv, W["Wg"], W["Wu"], W["Wd"], L["Ag"], L["Bg"], L["Au"], L["Bu"],
                   L["Ad"], L["Bd"], s, act)

    def loss():
        return float(np.sum(dY * _fwd(X, W, L, s, act)[0]))

    h = 1e-4
    params = [("dX", X)] + [("d" + k, L[k]) for k in ("Ag", "Bg", "Au", "Bu", "Ad", "Bd")]
    for name, P in params:
        fd = np.zeros_like(P)
        for idx in np.ndindex(P.shape):
            old = P[idx]
            P[idx] = old + h
            lp = loss()
            P[idx] = old - h
            lm = loss()
            P[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - gr[name])) / np.max(np.abs(gr[name]))
        assert err < 1e-7, (act, name, err)


@pytest.mark.parametrize("act", ACTS)
def test_mlp_backward_matches_torch_autograd(act):
    X, W, L, dY = _mlp_case(m=6, d=32, h=48, r=3, seed=2)
    s = 0.75
    t = {k: torch.tensor(v, requires_grad=True) for k, v in L.items()}
    tX = torch.tensor(X, requires_grad=True)
    Wt = {k: torch.tensor(v) for k, v in W.items()}
    actf = (torch.nn.functional.silu if act == "swiglu"
            else (lambda z: torch.nn.functional.gelu(z, approximate="tanh")))
    g = tX @ Wt["Wg"].T + s * (tX @ t["Ag"].T) @ t["Bg"].T
    u = tX @ Wt["Wu"].T + s * (tX @ t["Au"].T) @ t["Bu"].T
    H = actf(g) * u
    Y = H @ Wt["Wd"].T + s * (H @ t["Ad"].T) @ t["Bd"].T
    (Y * torch.tensor(dY)).sum().backward()
    _, sv = _fwd(X, W, L, s, act)
    gr = Q.mlp_bwd(dY, X, sv, W["Wg"], W["Wu"], W["Wd"], L["Ag"], L["Bg"], L["Au"], L["Bu"],
                   L["Ad"], L["Bd"], s, act)
    assert np.allclose(gr["dX"], tX.grad.numpy(), rtol=1e-11, atol=1e-12)
    for k in L:
        assert np.allclose(gr["d" + k], t[k].grad.numpy(), rtol=1e-11, atol=1e-12), k


@pytest.mark.parametrize("act", ACTS)
def test_b_zero_reduces_to_plain_gated_mlp(act):
    X, W, L, _ = _mlp_case(seed=3)
    for k in ("Bg", "Bu", "Bd"):
        L[k] = np.zeros_like(L[k])
    Y, _ = _fwd(X, W, L, 2.0, act)
    tX = torch.tensor(X)
    actf = (torch.nn.functional.silu if act == "swiglu"
            else (lambda z: torch.nn.functional.gelu(z, approximate="tanh")))
    ref = (actf(tX @ torch.tensor(W["Wg"]).T) * (tX @ torch.tensor(W["Wu"]).T)) @ torch.tensor(W["Wd"]).T
    assert np.allclose(Y, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_per_row_helper_matches_full():
    X, W, L, dY = _mlp_case(m=8, seed=4)
    s, act = 1.0, "swiglu"
    Y, sv = _fwd(X, W, L, s, act)
    gr = Q.mlp_bwd(dY, X, sv, W["Wg"], W["Wu"], W["Wd"], L["Ag"], L["Bg"], L["Au"], L["Bu"],
                   L["Ad"], L["Bd"], s, act)
    rows = np.array([1, 6, 3])
    pr = Q.mlp_rows(rows, X, dY, W["Wg"], W["Wu"], W["Wd"], L["Ag"], L["Bg"], L["Au"], L["Bu"],
                    L["Ad"], L["Bd"], s, act)
    assert np.allclose(pr["Y"], Y[rows], rtol=1e-13, atol=1e-14)
    assert np.allclose(pr["dX"], gr["dX"][rows], rtol=1e-13, atol=1e-14)
    for k in ("g", "u", "Ug", "Uu", "Ud"):
        assert np.allclose(pr[k], sv[k][rows], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("act", ACTS)
def test_lora_grads_helper_matches_torch_autograd_and_adds_over_blocks(act):
    """mlp_lora_grads (the six LoRA gradients alone, for long batches in row
    blocks) against torch fp64 autograd of <dY, Y>, and the sum of its results
    over two row blocks against the whole batch."""
    X, W, L, dY = _mlp_case(m=10, d=32, h=48, r=3, seed=5)
    s = 1.25
    t = {k: torch.tensor(v, requires_grad=True) for k, v in L.items()}
    tX = torch.tensor(X)
    Wt = {k: torch.tensor(v) for k, v in W.items()}
    actf = (torch.nn.functional.silu if act == "swiglu"
            else (lambda z: torch.nn.functional.gelu(z, approximate="tanh")))
    g = tX @ Wt["Wg"].T + s * (tX @ t["Ag"].T) @ t["Bg"].T
    u = tX @ Wt["Wu"].T + s * (tX @ t["Au"].T) @ t["Bu"].T
    H = actf(g) * u
    Y = H @ Wt["Wd"].T + s * (H @ t["Ad"].T) @ t["Bd"].T
    (Y * torch.tensor(dY)).sum().backward()
    args = (W["Wg"], W["Wu"], W["Wd"], L["Ag"], L["Bg"], L["Au"], L["Bu"], L["Ad"], L["Bd"], s, act)
    full = Q.mlp_lora_grads(X, dY, *args)
    for k in L:
        assert np.allclose(full["d" + k], t[k].grad.numpy(), rtol=1e-11, atol=1e-12), k
    parts = [Q.mlp_lora_grads(X[a:b], dY[a:b], *args) for a, b in ((0, 3), (3, 10))]
    for k in full:
        assert np.allclose(parts[0][k] + parts[1][k], full[k], rtol=1e-12, atol=1e-13), k
