"""Pins of the language-model head oracle (final RMSNorm, untied lm_head,
cross-entropy) against facts that do not come from the oracle itself:
brute-force loops, log-sum-exp identities, a uniform-logit closed form, the
zero column sums of dW forced by softmax rows summing to one, counted-row
semantics, and central finite differences.  CPU only."""
import math

import numpy as np
import pytest

from oracle import block as ob
from oracle import lm_head as oh


def _case(rng, N=7, C=16, V=11, scale=0.5):
    x = rng.standard_normal((N, C))
    w = rng.standard_normal((V, C)) * scale
    t = rng.integers(0, V, size=N)
    return x, w, t


def test_lse_identities_and_large_logits():
    rng = np.random.default_rng(31)
    z = rng.standard_normal((5, 9)) * 3
    for c in (-7.5, 0.0, 2.25):
        assert np.allclose(oh.lse_rows(z + c), oh.lse_rows(z) + c, rtol=1e-14, atol=1e-12)
    # max <= lse <= max + log V, and no overflow for large logits
    lse = oh.lse_rows(z)
    assert np.all(lse >= z.max(axis=1)) and np.all(lse <= z.max(axis=1) + math.log(9) + 1e-12)
    big = oh.lse_rows(z + 1e4)
    assert np.all(np.isfinite(big)) and np.allclose(big - 1e4, lse, rtol=0, atol=1e-9)


def test_loss_brute_force_loops():
    rng = np.random.default_rng(32)
    N, C, V = 3, 4, 5
    x, w, t = _case(rng, N, C, V)
    loss, c = oh.head_loss(x, w, t)
    total = 0.0
    for i in range(N):
        ms = math.sqrt(sum(x[i, k] ** 2 for k in range(C)) / C + 1e-6)
        h = [x[i, k] / ms for k in range(C)]
        z = [sum(h[k] * w[v, k] for k in range(C)) for v in range(V)]
        total += -math.log(math.exp(z[t[i]]) / sum(math.exp(zz) for zz in z))
    assert math.isclose(loss, total / N, rel_tol=1e-12)


def test_uniform_logits_give_log_v():
    rng = np.random.default_rng(33)
    x, w, t = _case(rng, N=6, C=8, V=13)
    loss, c = oh.head_loss(x, np.zeros_like(w), t)
    assert math.isclose(loss, math.log(13), rel_tol=1e-15)
    g = oh.head_loss_bwd(1.0, c, np.zeros_like(w))
    assert np.array_equal(g["dx"], np.zeros_like(x))       # dh = dz W = 0


def test_dw_columns_sum_to_zero():
    # each row of softmax(z) - onehot sums to zero, so sum_v dW[v, :] = 0
    rng = np.random.default_rng(34)
    x, w, t = _case(rng, N=9, C=12, V=17)
    _, c = oh.head_loss(x, w, t)
    g = oh.head_loss_bwd(1.0, c, w)
    assert np.max(np.abs(g["dw_lm"].sum(axis=0))) < 1e-14
    assert np.max(np.abs(g["dw_lm"])) > 1e-3


def test_uncounted_rows_drop_out():
    rng = np.random.default_rng(35)
    x, w, t = _case(rng, N=8, C=12, V=10)
    t2 = t.copy()
    t2[[1, 4]] = -1
    t2[6] = 10          # = V: outside the vocabulary, not counted either
    keep = np.array([i for i in range(8) if 0 <= t2[i] < 10])
    loss2, c2 = oh.head_loss(x, w, t2)
    loss_k, ck = oh.head_loss(x[keep], w, t[keep])
    assert math.isclose(loss2, loss_k, rel_tol=1e-14)
    g2 = oh.head_loss_bwd(1.0, c2, w)
    gk = oh.head_loss_bwd(1.0, ck, w)
    assert np.allclose(g2["dw_lm"], gk["dw_lm"], rtol=1e-13, atol=1e-15)
    assert np.array_equal(g2["dx"][[1, 4, 6]], np.zeros((3, 12)))
    assert np.allclose(g2["dx"][keep], gk["dx"], rtol=1e-13, atol=1e-15)
    # nothing counted: zero loss and gradients
    l0, c0 = oh.head_loss(x, w, np.full(8, -1))
    g0 = oh.head_loss_bwd(1.0, c0, w)
    assert l0 == 0.0 and not np.any(g0["dx"]) and not np.any(g0["dw_lm"])


def test_head_bwd_central_differences():
    rng = np.random.default_rng(36)
    x, w, t = _case(rng, N=5, C=6, V=7)
    t[2] = -1
    dloss = 0.7
    _, c = oh.head_loss(x, w, t)
    g = oh.head_loss_bwd(dloss, c, w)
    h = 1e-6

    def L(xx, ww):
        return dloss * oh.head_loss(xx, ww, t)[0]

    for arr, name in ((x, "dx"), (w, "dw_lm")):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            if name == "dx":
                num[idx] = (L(a1, w) - L(a2, w)) / (2 * h)
            else:
                num[idx] = (L(x, a1) - L(x, a2)) / (2 * h)
        assert np.allclose(g[name], num, rtol=1e-6, atol=1e-8), name


def test_head_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(37)
    x, w, t = _case(rng, N=10, C=32, V=40)
    t[3] = -1
    loss, c = oh.head_loss(x, w, t)
    g = oh.head_loss_bwd(1.0, c, w)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    h = xt * torch.rsqrt((xt * xt).mean(dim=-1, keepdim=True) + 1e-6)
    lt = torch.nn.functional.cross_entropy(h @ wt.T, torch.tensor(t), ignore_index=-1)
    lt.backward()
    assert math.isclose(loss, float(lt), rel_tol=1e-12)
    assert np.allclose(g["dx"], xt.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(g["dw_lm"], wt.grad.numpy(), rtol=1e-10, atol=1e-12)
