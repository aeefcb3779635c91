"""Planted mistakes: each mutant copy of the oracle must fail at least one pin.

A mutant is the oracle's own source with one plausible slip edited in (a
dropped term, a wrong sign, an off-by-one, a wrong index, a transposed
operand).  The pins below are independent of the oracle: hand-derived worked
examples, closed forms, torch's scaled_dot_product_attention with autograd,
finite differences and gradient invariants.  Everything runs on the CPU.
"""
import json
import os
import types

import numpy as np
import pytest
import torch

import oracle.attention as ATT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SRC = open(ATT.__file__).read()

MUTANTS = {
    "causal_strict": ("vis &= (j // c)[None, :] <= (q_pos // c)[:, None]", "vis &= (j // c)[None, :] < (q_pos // c)[:, None]"),
    "causal_local_index": ("vis &= (j // c)[None, :] <= (q_pos // c)[:, None]",
                           "vis &= (j // c)[None, :] <= (np.arange(len(q_pos)) // c)[:, None]"),
    "causal_block_ignored": ("vis &= (j // c)[None, :] <= (q_pos // c)[:, None]", "vis &= j[None, :] <= q_pos[:, None]"),
    "causal_block_ceil": ("vis &= (j // c)[None, :] <= (q_pos // c)[:, None]",
                          "vis &= ((j + c - 1) // c)[None, :] <= (q_pos // c)[:, None]"),
    "segment_local_index": ("vis &= seg_row[None, :] == seg_row[q_pos][:, None]",
                            "vis &= seg_row[None, :] == seg_row[np.arange(len(q_pos))][:, None]"),
    "bias_dropped": ("        s = s + bias_row[None, :]", "        s = s"),
    "bias_scaled": ("    s = scale * (qb @ kb.T)\n    if bias_row is not None:\n        s = s + bias_row[None, :]",
                    "    s = qb @ kb.T\n    if bias_row is not None:\n        s = s + bias_row[None, :]\n    s = scale * s"),
    "bias_no_modulo_wraps_wrong": ("bias[h, np.arange(kv_len) % bias.shape[1]]",
                                   "bias[h, (np.arange(kv_len) // bias.shape[1]) % bias.shape[1]]"),
    "scale_ignored": ("    s = scale * (qb @ kb.T)", "    s = (qb @ kb.T)"),
    "lse_without_max": ("m_safe + np.log(np.where(z > 0, z, 1.0))", "np.log(np.where(z > 0, z, 1.0))"),
    "softmax_unnormalised": ("    p = e / np.where(z > 0, z, 1.0)[:, None]", "    p = e"),
    "delta_dropped": ("ds = p * (dp - dl[:, None])", "ds = p * dp"),
    "delta_sign": ("ds = p * (dp - dl[:, None])", "ds = p * (dl[:, None] - dp)"),
    "dk_transposed": ("dk[b, :, h, :] += scale * (ds.T @ qb)", "dk[b, :, h, :] += scale * (ds @ qb)"),
    "dv_transposed": ("dv[b, :, h, :] += p.T @ dob", "dv[b, :, h, :] += p @ dob"),
    "dq_unscaled": ("dq[b, i0:i1, h, :] = scale * (ds @ kb)", "dq[b, i0:i1, h, :] = ds @ kb"),
    "dq_uses_values": ("dq[b, i0:i1, h, :] = scale * (ds @ kb)", "dq[b, i0:i1, h, :] = scale * (ds @ vb)"),
    "dp_uses_keys": ("dp = dob @ vb.T", "dp = dob @ kb.T"),
    "dbias_is_p": ("ds = p * (dob @ vb.T - dl[:, None])", "ds = p"),
    "dbias_wrong_index": ("np.add.at(dbias[h], np.arange(Lk) % nb, ds.sum(axis=0))",
                          "np.add.at(dbias[h], (np.arange(Lk) // nb) % nb, ds.sum(axis=0))"),
    "dbias_scaled": ("np.add.at(dbias[h], np.arange(Lk) % nb, ds.sum(axis=0))",
                     "np.add.at(dbias[h], np.arange(Lk) % nb, scale * ds.sum(axis=0))"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, name
    mod = types.ModuleType("oracle_mutant_" + name)
    exec(compile(SRC.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


# ------------------------------------------------------------------ pins, written against a module M
def pin_worked_examples(M):
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        cases = {k: v for k, v in json.load(f).items() if not k.startswith("_")}
    for ex in cases.values():
        q = np.array(ex["q"])[None, :, None, :]
        k = np.array(ex["k"])[None, :, None, :]
        v = np.array(ex["v"])[None, :, None, :]
        bias = np.array(ex["bias"])[None, :] if "bias" in ex else None
        seg = np.array(ex["segment_ids"])[None, :] if "segment_ids" in ex else None
        out, lse = M.forward(q, k, v, q_pos=np.arange(q.shape[1]), causal=ex["causal"], scale=ex["scale"],
                             bias=bias, segment_ids=seg)
        np.testing.assert_allclose(out[0, :, 0, :], ex["out"], atol=1e-12)
        np.testing.assert_allclose(lse[0, 0], ex["lse"], atol=1e-12)


def pin_zero_keys_per_rank(M):
    rng = np.random.default_rng(1)
    B, L, H, D, n, r = 1, 16, 1, 3, 4, 2
    q, v = rng.standard_normal((B, L // n, H, D)), rng.standard_normal((B, L, H, D))
    pos = M.query_positions(L // n, L, n, r)
    out, lse = M.forward(q, np.zeros((B, L, H, D)), v, q_pos=pos, causal=True)
    cum = np.cumsum(v, axis=1) / np.arange(1, L + 1)[None, :, None, None]
    np.testing.assert_allclose(out, cum[:, r * 4:(r + 1) * 4], atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(pos + 1), atol=1e-13)


def _case(seed, L=16, n=4, rank=-1, bias_len=6, seg=True):
    rng = np.random.default_rng(seed)
    B, H, D = 1, 2, 4
    Lq = L if rank < 0 else L // n
    q, k, v = rng.standard_normal((B, Lq, H, D)), rng.standard_normal((B, L, H, D)), rng.standard_normal((B, L, H, D))
    bias = rng.standard_normal((H, bias_len)) if bias_len else None
    segs = np.sort(rng.integers(0, 3, size=(B, L)), axis=1) if seg else None
    pos = (np.arange(L) if rank < 0 else rank * (L // n) + np.arange(L // n))
    return q, k, v, bias, segs, pos


def pin_sdpa(M):
    for rank in (-1, 2):
        q, k, v, bias, segs, pos = _case(3, rank=rank)
        scale = 0.6
        B, Lq, H, D = q.shape
        Lk = k.shape[1]
        tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy(), requires_grad=True) for x in (q, k, v))
        j, p = torch.arange(Lk), torch.as_tensor(pos)
        add = torch.as_tensor(bias)[:, j % bias.shape[1]][None, :, None, :].expand(B, H, Lq, Lk).clone()
        add = add.masked_fill((j[None, :] > p[:, None])[None, None], float("-inf"))
        st = torch.as_tensor(segs)
        add = add.masked_fill((st[:, None, :] != st[:, p][:, :, None])[:, None], float("-inf"))
        t_out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=add, scale=scale)
        out, _ = M.forward(q, k, v, q_pos=pos, causal=True, scale=scale, bias=bias, segment_ids=segs)
        np.testing.assert_allclose(out, t_out.detach().numpy().transpose(0, 2, 1, 3), atol=1e-12)
        dout = np.random.default_rng(4).standard_normal(out.shape)
        t_out.backward(torch.tensor(dout.transpose(0, 2, 1, 3).copy()))
        grads = M.backward(q, k, v, dout, q_pos=pos, causal=True, scale=scale, bias=bias, segment_ids=segs)[:3]
        for g, leaf in zip(grads, (tq, tk, tv)):
            np.testing.assert_allclose(g, leaf.grad.numpy().transpose(0, 2, 1, 3), atol=1e-11)


def pin_gradient_invariants(M):
    q, k, v, bias, segs, pos = _case(5)
    dout = np.random.default_rng(6).standard_normal(q.shape)
    dq, dk, dv, _ = M.backward(q, k, v, dout, q_pos=pos, causal=True, scale=0.5, bias=bias, segment_ids=segs)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=1), dout.sum(axis=1), atol=1e-12)
    np.testing.assert_allclose(np.einsum("blhd,blhd->bh", dq, q), np.einsum("blhd,blhd->bh", dk, k), atol=1e-12)


def pin_causal_blocks(M):
    # causal block size c: the rows of causal block b equal unmasked attention over the keys of
    # blocks 0..b (a formulation that never touches the causal code); c >= L is no mask at all
    rng = np.random.default_rng(8)
    L, c = 12, 4
    q, k, v = (rng.standard_normal((1, L, 2, 3)) for _ in range(3))
    out, lse = M.forward(q, k, v, q_pos=np.arange(L), causal=c, scale=0.7)
    for b in range(L // c):
        rows, keys = slice(b * c, (b + 1) * c), slice(0, (b + 1) * c)
        o_b, l_b = M.forward(q[:, rows], k[:, keys], v[:, keys], q_pos=np.arange(b * c, (b + 1) * c), causal=False,
                             scale=0.7)
        np.testing.assert_allclose(out[:, rows], o_b, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, rows], l_b, atol=1e-13)
    o_all, _ = M.forward(q, k, v, q_pos=np.arange(L), causal=False, scale=0.7)
    np.testing.assert_allclose(M.forward(q, k, v, q_pos=np.arange(L), causal=L, scale=0.7)[0], o_all, atol=1e-13)
    assert M.visible_pairs(np.arange(L), L, c) == sum((p // c + 1) * c for p in range(L))


def pin_bias_grad(M):
    # torch autograd through the bias gathered by key position (library special case), and the
    # gradient of the scores summing to zero over each query's keys
    q, k, v, bias, segs, pos = _case(9, bias_len=5)
    scale = 0.45
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    tb = torch.tensor(bias, requires_grad=True)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3).copy()) for x in (q, k, v))
    j, p = torch.arange(Lk), torch.as_tensor(pos)
    st = torch.as_tensor(segs)
    mask = (j[None, :] > p[:, None])[None, None] | (st[:, None, :] != st[:, p][:, :, None])[:, None]
    add = tb[:, j % bias.shape[1]][None, :, None, :].expand(B, H, Lq, Lk).masked_fill(mask, float("-inf"))
    t_out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=add, scale=scale)
    dout = np.random.default_rng(10).standard_normal(q.shape)
    t_out.backward(torch.tensor(dout.transpose(0, 2, 1, 3).copy()))
    g = M.bias_grad(q, k, v, dout, q_pos=pos, causal=True, scale=scale, bias=bias, segment_ids=segs)
    np.testing.assert_allclose(g, tb.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-12)


PINS = [pin_worked_examples, pin_zero_keys_per_rank, pin_sdpa, pin_gradient_invariants, pin_causal_blocks,
        pin_bias_grad]


def test_pins_pass_on_the_oracle():
    for pin in PINS:
        pin(ATT)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name):
    M = _mutant(name)
    caught = []
    for pin in PINS:
        try:
            pin(M)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
