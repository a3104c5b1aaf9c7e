"""Pins of the oracle's backward pass (oracle.attention_grad).

The gradient of the loss sum(out * dout) through the block-sparse masks is
pinned three independent ways, on small float64 cases:
  * central finite differences of the forward oracle (which is itself pinned
    by test_oracle_attention.py), element by element on a sample of every
    input, including rows of cache slots no frame uses (gradient exactly 0);
  * torch autograd through a separate formulation (torch.softmax over
    -inf-masked logits), whole tensors;
  * the sum rules of softmax attention: the key gradients of one (batch,
    head) sum to zero over all keys, and the value gradients sum to the sum
    of the output gradients over the query rows.
A wrong sign, a dropped D term, a transposed product or a misrouted slot
breaks at least one of them.
"""
import numpy as np
import pytest
import torch

from oracle import lf_oracle as O

T, BLOCK, FC, FH, S_SLOTS, D = 10, 4, 2, 3, 7, 8   # nb = 3 (ragged last block of 2 tokens)
NB = 3
SLOTS = [4, 0, 6, 2, 5]                               # logical frame -> cache slot (slots 1, 3 unused)


def _case(seed, n_keep=2):
    rng = np.random.default_rng(seed)
    B, H = 1, 2
    Lq = FC * T
    q = rng.standard_normal((B, H, Lq, D))
    k = rng.standard_normal((B, H, S_SLOTS, T, D))
    v = rng.standard_normal((B, H, S_SLOTS, T, D))
    dout = rng.standard_normal((B, H, Lq, D))
    nqb = FC * NB
    max_sel = n_keep + 1
    sel = np.full((B, H, nqb, max_sel), -1, np.int32)
    n_sel = np.zeros((B, H, nqb), np.int32)
    for h in range(H):
        for qb in range(nqb):
            ids = np.sort(rng.choice(FH * NB, size=n_keep, replace=False))
            sel[0, h, qb, :n_keep] = ids
            n_sel[0, h, qb] = n_keep
    return q, k, v, dout, sel, n_sel


def _loss(q, k, v, dout, sel, n_sel, scale):
    out = O.attention(q, k, v, SLOTS, sel, n_sel, T, BLOCK, FC, FH, scale)["out"]
    return float(np.sum(out * dout))


def _grads(q, k, v, dout, sel, n_sel, scale):
    return O.attention_grad(q, k, v, SLOTS, sel, n_sel, dout, T, BLOCK, FC, FH, scale)


def test_finite_differences():
    q, k, v, dout, sel, n_sel = _case(3)
    scale = 0.4
    g = _grads(q, k, v, dout, sel, n_sel, scale)
    rng = np.random.default_rng(7)
    eps = 1e-6
    checked = 0
    for name, x, gx in (("q", q, g["dq"]), ("k", k, g["dk_cache"]), ("v", v, g["dv_cache"])):
        idx = [tuple(rng.integers(0, n) for n in x.shape) for _ in range(25)]
        if name != "q":  # rows of unused slots 1 and 3 must get exactly zero
            idx += [(0, 1, 1, 3, 2), (0, 0, 3, 9, 7)]
        for ix in idx:
            xp, xm = x.copy(), x.copy()
            xp[ix] += eps
            xm[ix] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], dout, sel, n_sel, scale)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], dout, sel, n_sel, scale)
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - gx[ix]) <= 1e-6 * max(1.0, abs(fd)), (name, ix, fd, gx[ix])
            checked += 1
    assert checked == 79


def test_matches_autograd_of_separate_formulation():
    q, k, v, dout, sel, n_sel = _case(5, n_keep=3)
    scale = 0.35
    g = _grads(q, k, v, dout, sel, n_sel, scale)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    loss = 0.0
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            keys = torch.cat([tk[b, h, s] for s in SLOTS], 0)
            vals = torch.cat([tv[b, h, s] for s in SLOTS], 0)
            for qb in range(FC * NB):
                fc, j = divmod(qb, NB)
                lo, hi = j * BLOCK, min((j + 1) * BLOCK, T)
                rows = slice(fc * T + lo, fc * T + hi)
                allowed = torch.zeros(len(SLOTS) * T, dtype=torch.bool)
                allowed[FH * T:] = True
                for bid in sel[b, h, qb, :n_sel[b, h, qb]]:
                    f, jj = divmod(int(bid), NB)
                    allowed[f * T + jj * BLOCK:f * T + min((jj + 1) * BLOCK, T)] = True
                logits = (tq[b, h, rows] @ keys.T) * scale
                logits = logits.masked_fill(~allowed, float("-inf"))
                out = torch.softmax(logits, dim=-1) @ vals
                loss = loss + (out * torch.tensor(dout[b, h, rows])).sum()
    loss.backward()
    np.testing.assert_allclose(g["dq"], tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dk_cache"], tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dv_cache"], tv.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_sum_rules(seed):
    q, k, v, dout, sel, n_sel = _case(seed)
    g = _grads(q, k, v, dout, sel, n_sel, 0.5)
    for h in range(q.shape[1]):
        dk = g["dk_cache"][0, h].reshape(-1, D)
        dv = g["dv_cache"][0, h].reshape(-1, D)
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
        np.testing.assert_allclose(dv.sum(axis=0), dout[0, h].sum(axis=0), rtol=1e-12, atol=1e-12)


def test_planted_sign_error_is_caught():
    """The finite-difference pin notices a flipped D term (a plausible slip)."""
    q, k, v, dout, sel, n_sel = _case(3)
    scale = 0.4
    K = O.logical_sequence(k[0, 0], SLOTS, FH + FC)
    V = O.logical_sequence(v[0, 0], SLOTS, FH + FC)
    rows = slice(FH * 0, 4)
    mask = O.visible_keys(sel[0, 0, 0, :n_sel[0, 0, 0]], T, BLOCK, FH, FC)
    o, _, p = O.masked_softmax_attention(q[0, 0, rows], K, V, mask, scale)
    dp = dout[0, 0, rows] @ V.T
    wrong = scale * ((p * (dp + np.sum(dout[0, 0, rows] * o, 1, keepdims=True))) @ K)
    right, _, _ = O.masked_softmax_attention_grad(q[0, 0, rows], K, V, mask, scale, dout[0, 0, rows])
    assert np.max(np.abs(wrong - right)) > 1e-3
