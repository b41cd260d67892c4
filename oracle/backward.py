"""Oracle: gradients of the block-sparse attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[P2] §4 (training) and [P3] ask the backward pass to reuse the forward's
block selection: the attended set A_i of every query is the same as in the
forward (`attention.allowed_mask`), and the gradients are those of

  O_i = sum_{p in A_i} softmax_p(q_i . k_p / sqrt(d)) v_p

with respect to Q, K and V.  Here they come from automatic differentiation
(torch, float64, CPU) of that plain definition: full score rows, the mask,
softmax, P V.  Autograd is a library primitive applied to the definition, so
the result is the exact gradient up to fp64 rounding; the pins compare it
with torch's own fp64 causal attention backward (every block selected) and
with central finite differences.

For a whole problem, dK and dV of a key gather the contributions of every
query (of every row and, under shared GQA routing, every query head of the
group) that attends it.
"""
from __future__ import annotations

import numpy as np
import torch

from .attention import allowed_mask


def masked_attention_grads(q_rows, q_pos, k, v, length: int, b: int, blocks, causal: bool, dout):
    """(dq [m, d], dk [length, d], dv [length, d]) of sum(O * dout) for one
    head and one set of query rows; k, v [>= length, d]; dout [m, d]."""
    mask = torch.as_tensor(allowed_mask(np.asarray(q_pos), length, b, blocks, causal))
    q = torch.tensor(np.asarray(q_rows, dtype=np.float64), requires_grad=True)
    kk = torch.tensor(np.asarray(k[:length], dtype=np.float64), requires_grad=True)
    vv = torch.tensor(np.asarray(v[:length], dtype=np.float64), requires_grad=True)
    s = (q @ kk.T) / np.sqrt(q.shape[1])
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.softmax(s, dim=1)
    o = p @ vv
    o.backward(torch.as_tensor(np.asarray(dout, dtype=np.float64)))
    return q.grad.numpy(), kk.grad.numpy(), vv.grad.numpy()
