"""Blockwise feed-forward, plain float64 definition -- test infrastructure only.

"RingAttention核心功能全解析" (section "快速上手") exports ``blockwise_feedforward``
next to ``ringattention`` and gives nothing but its name.  Its sharding example
builds the device mesh from ``LLaMAConfig`` (section "计算与通信重叠"), so the
feed-forward taken is the LLaMA one, SwiGLU:

    FFN(x) = W2 ( silu(W1 x) * (W3 x) ),   silu(a) = a / (1 + exp(-a))

applied to every token independently, with W1, W3: [d_ff, d_model] and
W2: [d_model, d_ff] (output-by-input, as a linear layer stores them).
"Blockwise" means the sequence is processed in chunks of ``chunk`` tokens, so
that the [tokens, d_ff] intermediate never exists for the whole sequence; the
result does not depend on the chunking (the FFN is per token), which the tests
pin.  x: [tokens, d_model].

Backward, given dout = dL/dFFN(x), with g = W1 x, u = W3 x, s = sigmoid(g):

    h   = silu(g) * u
    dh  = W2^T dout
    dg  = dh * u * s * (1 + g (1 - s))        (silu'(g) = s (1 + g (1 - s)))
    du  = dh * silu(g)
    dx  = W1^T dg + W3^T du
    dW1 = sum_tokens dg x^T,  dW3 = sum_tokens du x^T,  dW2 = sum_tokens dout h^T
"""
import numpy as np


def _sigmoid(a):
    return 1.0 / (1.0 + np.exp(-a))


def _chunks(n, chunk):
    chunk = max(1, int(chunk))
    for i0 in range(0, n, chunk):
        yield i0, min(n, i0 + chunk)


def ffn_forward(x, w1, w3, w2, *, chunk=None):
    """SwiGLU feed-forward of every token, float64.  x [T, d]; returns [T, d]."""
    x = np.asarray(x, dtype=np.float64)
    w1, w3, w2 = (np.asarray(w, dtype=np.float64) for w in (w1, w3, w2))
    out = np.zeros((x.shape[0], w2.shape[0]), dtype=np.float64)
    for i0, i1 in _chunks(x.shape[0], chunk or x.shape[0] or 1):
        xc = x[i0:i1]
        g, u = xc @ w1.T, xc @ w3.T
        out[i0:i1] = (g * _sigmoid(g) * u) @ w2.T
    return out


def ffn_backward(x, w1, w3, w2, dout, *, chunk=None):
    """Gradients (dx [T, d], dw1 [f, d], dw3 [f, d], dw2 [d, f]) of sum(dout * FFN(x)), float64,
    recomputing the intermediate chunk by chunk."""
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    w1, w3, w2 = (np.asarray(w, dtype=np.float64) for w in (w1, w3, w2))
    dx = np.zeros_like(x)
    dw1, dw3, dw2 = np.zeros_like(w1), np.zeros_like(w3), np.zeros_like(w2)
    for i0, i1 in _chunks(x.shape[0], chunk or x.shape[0] or 1):
        xc, dc = x[i0:i1], dout[i0:i1]
        g, u = xc @ w1.T, xc @ w3.T
        s = _sigmoid(g)
        h = g * s * u
        dh = dc @ w2
        dg = dh * u * s * (1.0 + g * (1.0 - s))
        du = dh * g * s
        dx[i0:i1] = dg @ w1 + du @ w3
        dw1 += dg.T @ xc
        dw3 += du.T @ xc
        dw2 += dc.T @ h
    return dx, dw1, dw3, dw2
