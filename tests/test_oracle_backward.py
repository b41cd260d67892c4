"""Pins of the backward oracle (oracle/backward.py): with every causal block
selected it equals torch's fp64 causal attention backward (an independent
routine); on a sparse selection it matches central finite differences of the
forward definition; keys outside the attended set get zero gradient."""
import numpy as np
import torch

from oracle import attention, backward


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_dense_selection_equals_sdpa_backward():
    n, d, b = 40, 8, 8
    q, k, v, do = (_rand((n, d), s) for s in (1, 2, 3, 4))
    dq, dk, dv = backward.masked_attention_grads(q, np.arange(n), k, v, n, b, list(range(5)), True, do)
    qt, kt, vt = (torch.tensor(x[None, None], requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    o.backward(torch.tensor(do[None, None]))
    assert np.max(np.abs(dq - qt.grad[0, 0].numpy())) < 1e-12
    assert np.max(np.abs(dk - kt.grad[0, 0].numpy())) < 1e-12
    assert np.max(np.abs(dv - vt.grad[0, 0].numpy())) < 1e-12


def test_sparse_selection_matches_finite_differences():
    n, d, b = 24, 4, 4
    q, k, v, do = (_rand((n, d), s) for s in (5, 6, 7, 8))
    rows = np.arange(16, 24)            # query block 4
    blocks = [0, 2, 4]
    dq, dk, dv = backward.masked_attention_grads(q[rows], rows, k, v, n, b, blocks, True, do[rows])

    def loss(qq, kk, vv):
        o = attention.masked_attention(qq, rows, kk, vv, n, b, blocks, True)["o"]
        return float(np.sum(o * do[rows]))

    eps = 1e-6
    for arr, grad, name in ((q, dq, "q"), (k, dk, "k"), (v, dv, "v")):
        idx = [(i, j) for i in range(arr.shape[0]) for j in range(d)]
        rng = np.random.default_rng(9)
        for t in rng.choice(len(idx), size=12, replace=False):
            i, j = idx[t]
            if name == "q" and i not in rows:
                continue
            a1, a2 = arr.copy(), arr.copy()
            a1[i, j] += eps
            a2[i, j] -= eps
            args1 = {"q": (a1[rows], k, v), "k": (q[rows], a1, v), "v": (q[rows], k, a1)}[name]
            args2 = {"q": (a2[rows], k, v), "k": (q[rows], a2, v), "v": (q[rows], k, a2)}[name]
            fd = (loss(*args1) - loss(*args2)) / (2 * eps)
            g = grad[list(rows).index(i), j] if name == "q" else grad[i, j]
            assert abs(fd - g) < 1e-6, (name, i, j, fd, g)
    # keys of unselected blocks (1, 3, 5) get no gradient
    for blk in (1, 3, 5):
        ks = slice(blk * b, min((blk + 1) * b, n))
        assert not dk[ks].any() and not dv[ks].any()
