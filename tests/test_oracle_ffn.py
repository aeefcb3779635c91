"""Pins of the blockwise feed-forward oracle (CPU): torch autograd (library special case),
finite differences, chunk invariance and a closed form."""
import numpy as np
import pytest
import torch

import oracle


def _case(T=37, d=12, f=20, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w1, w3 = rng.standard_normal((f, d)) * 0.3, rng.standard_normal((f, d)) * 0.3
    w2 = rng.standard_normal((d, f)) * 0.3
    return x, w1, w3, w2


def _torch_ffn(x, w1, w3, w2):
    # a different formulation: torch's silu and linear layers, autograd for the gradients
    tx, t1, t3, t2 = (torch.tensor(a, requires_grad=True) for a in (x, w1, w3, w2))
    y = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(tx, t1))
                                   * torch.nn.functional.linear(tx, t3), t2)
    return y, (tx, t1, t3, t2)


@pytest.mark.parametrize("chunk", [None, 1, 5, 37, 100])
def test_forward_and_gradients_match_torch(chunk):
    x, w1, w3, w2 = _case()
    y, leaves = _torch_ffn(x, w1, w3, w2)
    np.testing.assert_allclose(oracle.ffn_forward(x, w1, w3, w2, chunk=chunk), y.detach().numpy(), atol=1e-12)
    dout = np.random.default_rng(1).standard_normal(y.shape)
    y.backward(torch.tensor(dout))
    grads = oracle.ffn_backward(x, w1, w3, w2, dout, chunk=chunk)
    for g, leaf in zip(grads, leaves):
        np.testing.assert_allclose(g, leaf.grad.numpy(), atol=1e-11)


def test_finite_differences():
    x, w1, w3, w2 = _case(T=5, d=4, f=6, seed=2)
    dout = np.random.default_rng(3).standard_normal((5, 4))
    dx, dw1, dw3, dw2 = oracle.ffn_backward(x, w1, w3, w2, dout, chunk=2)
    loss = lambda *a: float(np.sum(dout * oracle.ffn_forward(*a)))  # noqa: E731
    eps = 1e-6
    for arr_i, grad in ((0, dx), (1, dw1), (2, dw3), (3, dw2)):
        args = [x, w1, w3, w2]
        for idx in ((0, 0), (1, 2), (3, 1)):
            if idx[0] >= args[arr_i].shape[0] or idx[1] >= args[arr_i].shape[1]:
                continue
            ap, am = args[arr_i].copy(), args[arr_i].copy()
            ap[idx] += eps
            am[idx] -= eps
            pa, ma = list(args), list(args)
            pa[arr_i], ma[arr_i] = ap, am
            assert abs((loss(*pa) - loss(*ma)) / (2 * eps) - grad[idx]) < 1e-6


def test_closed_form_zero_gate():
    # W1 = 0 gives silu(0) = 0: the output is zero whatever W3, W2 and x are
    x, w1, w3, w2 = _case(seed=4)
    assert np.all(oracle.ffn_forward(x, np.zeros_like(w1), w3, w2) == 0.0)
    # one hidden unit and identity-like weights: y = silu(x0) * x0 on the first coordinate
    x = np.array([[1.5, 0.0], [-2.0, 0.0]])
    w1 = np.array([[1.0, 0.0]])
    w3 = np.array([[1.0, 0.0]])
    w2 = np.array([[1.0], [0.0]])
    y = oracle.ffn_forward(x, w1, w3, w2)
    for t, a in enumerate((1.5, -2.0)):
        assert abs(y[t, 0] - a * a / (1.0 + np.exp(-a))) < 1e-15 and y[t, 1] == 0.0


def test_empty_sequence():
    x, w1, w3, w2 = _case(T=0)
    assert oracle.ffn_forward(x, w1, w3, w2).shape == (0, 12)
    dx, dw1, dw3, dw2 = oracle.ffn_backward(x, w1, w3, w2, np.zeros((0, 12)))
    assert dx.shape == (0, 12) and not dw1.any() and not dw2.any() and not dw3.any()


# planted mistakes in the oracle's source: each must fail the torch pin
import os  # noqa: E402
import types  # noqa: E402

FFN_SRC = open(oracle.ffn.__file__).read() if hasattr(oracle, "ffn") else open(
    os.path.join(os.path.dirname(oracle.__file__), "ffn.py")).read()
FFN_MUTANTS = {
    "silu_derivative_dropped": ("dg = dh * u * s * (1.0 + g * (1.0 - s))", "dg = dh * u * s"),
    "gate_on_the_wrong_branch": ("out[i0:i1] = (g * _sigmoid(g) * u) @ w2.T", "out[i0:i1] = (u * _sigmoid(u) * g) @ w2.T"),
    "dw2_transposed_operands": ("dw2 += dc.T @ h", "dw2 += (h.T @ dc).T * 0.5 + (dc.T @ h) * 0.5 + 1e-3"),
    "dx_missing_up_branch": ("dx[i0:i1] = dg @ w1 + du @ w3", "dx[i0:i1] = dg @ w1"),
}


@pytest.mark.parametrize("name", sorted(FFN_MUTANTS))
def test_ffn_planted_mistakes_are_caught(name):
    old, new = FFN_MUTANTS[name]
    assert FFN_SRC.count(old) == 1, name
    mod = types.ModuleType("ffn_mutant_" + name)
    exec(compile(FFN_SRC.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        x, w1, w3, w2 = _case(seed=9)
        y, leaves = _torch_ffn(x, w1, w3, w2)
        np.testing.assert_allclose(mod.ffn_forward(x, w1, w3, w2, chunk=7), y.detach().numpy(), atol=1e-12)
        dout = np.random.default_rng(10).standard_normal(y.shape)
        y.backward(torch.tensor(dout))
        for g, leaf in zip(mod.ffn_backward(x, w1, w3, w2, dout, chunk=7), leaves):
            np.testing.assert_allclose(g, leaf.grad.numpy(), atol=1e-11)
