"""Pins of the CPU float64 oracle against facts that do not come from the
oracle itself: closed forms, invariants, brute force on tiny inputs, central
finite differences, an independent autograd derivation, and the figures the
pages print.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

from blockinputs import BlockShape, DecodeShape, block_param_count, from_depth, make_block_inputs, make_decode_inputs
from oracle import block as ob

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _weights(rng, C, F, H, scale=0.3):
    return (rng.standard_normal((3 * C, C)) * scale, rng.standard_normal((C, C)) * scale,
            rng.standard_normal((F, C)) * scale, rng.standard_normal((C, F)) * scale)


# ------------------------------------------------------------ shapes (pages)
def test_depth_rule_reproduces_printed_table():
    g = json.load(open(os.path.join(GOLDEN, "depth_table.json")))
    V = g["vocab"]
    for row in g["rows"]:
        d = row["depth"]
        C, H, F = from_depth(d)
        assert (C, H) == (row["width"], row["heads"])
        scaling = d * block_param_count(C, F) + V * C          # blocks + lm_head
        n_value_emb = d // 2                                    # alternate layers
        total = scaling + V * C + n_value_emb * V * C           # + wte + value embeddings
        assert round(total / 1e6) == row["total_params_M"], (d, total)
        assert round(row["ratio"] * scaling / 1e9, 2) == row["tokens_B"]
    C, H, F = from_depth(12)
    assert round((12 * block_param_count(C, F) + V * C) / 1e6) == g["d12_scaling_params_M"]
    s = g["speedrun_oct2025"]
    C, H, F = from_depth(s["depth"])
    assert (C, H, C // H) == (s["width"], s["heads"], s["head_dim"])
    total = s["depth"] * block_param_count(C, F) + 2 * s["vocab"] * C
    assert abs(total / 1e6 - s["params_M_approx"]) < 5


def test_block_param_count_is_12_c_squared():
    for d in (6, 12, 20, 26):
        C, H, F = from_depth(d)
        assert block_param_count(C, F) == 12 * C * C


# ------------------------------------------------------------ RMSNorm
def test_rmsnorm_closed_form_constant_row():
    eps = 1e-6
    for c in (0.5, 3.0, -2.0):
        x = np.full((1, 16), c)
        h, r = ob.rmsnorm(x, eps)
        assert np.allclose(h, c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
        assert np.isclose(r[0], 1 / math.sqrt(c * c + eps), rtol=1e-15)


def test_rmsnorm_output_rms_and_scale_invariance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 64)) * 3
    eps = 1e-6
    h, _ = ob.rmsnorm(x, eps)
    m = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(h * h, axis=-1), m / (m + eps), rtol=1e-13)
    h2, _ = ob.rmsnorm(5.0 * x, 0.0)
    h3, _ = ob.rmsnorm(x, 0.0)
    assert np.allclose(h2, h3, rtol=1e-13)


def test_rmsnorm_bwd_finite_differences():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 10))
    g = rng.standard_normal((3, 10))
    h, r = ob.rmsnorm(x, 1e-3)
    dx = ob.rmsnorm_bwd(g, h, r)
    eps_fd = 1e-6
    num = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps_fd
        xm[idx] -= eps_fd
        num[idx] = (np.sum(g * ob.rmsnorm(xp, 1e-3)[0]) - np.sum(g * ob.rmsnorm(xm, 1e-3)[0])) / (2 * eps_fd)
    assert np.allclose(dx, num, rtol=1e-7, atol=1e-9)


# ------------------------------------------------------------ rotary
def test_rope_pairing_and_sign_closed_form():
    # D = 4, base 10000: pair (0, 2) turns at 1 rad per position, pair (1, 3)
    # at 10000^(-1/2) = 0.01 rad per position; counter-clockwise.
    cos, sin = ob.rope_tables(np.array([0, 1, 3]), 4, 10000.0)
    z = np.zeros((3, 4))
    z[:, 0] = 1.0
    z[:, 3] = 2.0
    out = ob.rope(z, cos, sin)
    assert np.allclose(out[0], [1, 0, 0, 2], atol=0)
    assert np.allclose(out[1], [math.cos(1), -2 * math.sin(0.01), math.sin(1), 2 * math.cos(0.01)], rtol=1e-15)
    assert np.allclose(out[2], [math.cos(3), -2 * math.sin(0.03), math.sin(3), 2 * math.cos(0.03)], rtol=1e-14)


def test_rope_norm_preservation_and_shift_invariance():
    rng = np.random.default_rng(3)
    D = 128
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    cos, sin = ob.rope_tables(np.arange(40), D, 10000.0)
    Q = ob.rope(np.tile(q, (40, 1)), cos, sin)
    K = ob.rope(np.tile(k, (40, 1)), cos, sin)
    assert np.allclose(np.linalg.norm(Q, axis=1), np.linalg.norm(q), rtol=1e-13)
    for t, tp, s in ((5, 2, 7), (30, 0, 9), (3, 3, 20)):
        assert np.isclose(Q[t] @ K[tp], Q[t + s] @ K[tp + s], rtol=1e-11, atol=1e-11)


def test_rope_bwd_is_inverse_rotation():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((2, 9, 16))
    cos, sin = ob.rope_tables(np.arange(9) * 13, 16, 10000.0)
    assert np.allclose(ob.rope_bwd(ob.rope(z, cos, sin), cos, sin), z, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------ attention
def test_attention_brute_force_loops():
    rng = np.random.default_rng(5)
    T, D = 6, 4
    q, k, v = (rng.standard_normal((T, D)) for _ in range(3))
    o, _ = ob.causal_attention(q, k, v)
    for i in range(T):
        w = [math.exp(sum(q[i, d] * k[j, d] for d in range(D)) / math.sqrt(D)) for j in range(i + 1)]
        z = sum(w)
        for d in range(D):
            assert math.isclose(o[i, d], sum(w[j] * v[j, d] for j in range(i + 1)) / z, rel_tol=1e-12, abs_tol=1e-13)


def test_attention_t1_is_v_and_q0_is_prefix_mean():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((3, 1, 8))
    o, _ = ob.causal_attention(rng.standard_normal((3, 1, 8)), rng.standard_normal((3, 1, 8)), v)
    assert np.array_equal(o, v)
    T = 11
    v = rng.standard_normal((T, 8))
    o, _ = ob.causal_attention(np.zeros((T, 8)), rng.standard_normal((T, 8)), v)
    assert np.allclose(o, np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None], rtol=1e-13, atol=1e-14)


def test_online_softmax_matches_materialised():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((2, 3, 37, 16)) * 2 for _ in range(3))
    o1, P = ob.causal_attention(q, k, v)
    o2, lse = ob.online_causal_attention(q, k, v, block=8)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-13)
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / 4.0
    T = 37
    s = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, s)
    assert np.allclose(np.exp(s - lse[..., None]), P, rtol=1e-11, atol=1e-15)


# ------------------------------------------------- sliding-window attention
def test_window_brute_force_loops():
    # query i averages v over keys max(0, i-W+1) .. i with softmax weights
    rng = np.random.default_rng(21)
    T, D, Wn = 9, 4, 3
    q, k, v = (rng.standard_normal((T, D)) for _ in range(3))
    o, _ = ob.causal_attention(q, k, v, window=Wn)
    for i in range(T):
        keys = range(max(0, i - Wn + 1), i + 1)
        w = {j: math.exp(sum(q[i, d] * k[j, d] for d in range(D)) / math.sqrt(D)) for j in keys}
        z = sum(w.values())
        for d in range(D):
            ref = sum(w[j] * v[j, d] for j in keys) / z
            assert math.isclose(o[i, d], ref, rel_tol=1e-12, abs_tol=1e-13)


def test_window_row_support_and_wide_window_is_causal():
    rng = np.random.default_rng(22)
    T, Wn = 13, 4
    q, k, v = (rng.standard_normal((2, T, 8)) for _ in range(3))
    _, P = ob.causal_attention(q, k, v, window=Wn)
    counts = np.count_nonzero(P, axis=-1)
    assert np.array_equal(counts[0], np.minimum(np.arange(T) + 1, Wn))
    o_c, P_c = ob.causal_attention(q, k, v)
    for wide in (T, T + 5):
        o_w, P_w = ob.causal_attention(q, k, v, window=wide)
        assert np.array_equal(o_w, o_c) and np.array_equal(P_w, P_c)


def test_window_one_is_value_and_stops_qk_gradients():
    # a window of one key: each query attends to itself only, so o = v and
    # the scores carry no gradient back to q and k
    rng = np.random.default_rng(23)
    q, k, v, do = (rng.standard_normal((3, 10, 16)) for _ in range(4))
    o, P = ob.causal_attention(q, k, v, window=1)
    assert np.array_equal(o, v)
    dq, dk, dv = ob.causal_attention_bwd(do, q, k, v, o, P)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    assert np.array_equal(dv, do)


@pytest.mark.parametrize("window", [None, 5, 16])
def test_online_softmax_with_window_matches_materialised(window):
    rng = np.random.default_rng(24)
    q, k, v = (rng.standard_normal((2, 3, 37, 16)) * 2 for _ in range(3))
    o1, _ = ob.causal_attention(q, k, v, window=window)
    o2, _ = ob.online_causal_attention(q, k, v, block=8, window=window)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-13)


def test_window_block_bwd_central_differences():
    # the adjoint with a window: directional derivatives of <dy, y>
    rng = np.random.default_rng(25)
    B, T, C, H, Wn = 1, 7, 256, 2, 3
    x = rng.standard_normal((B, T, C))
    W = _weights(rng, C, 4 * C, H, 0.05)
    dy = rng.standard_normal((B, T, C))
    g = ob.block_bwd(dy, ob.block_fwd(x, *W, H=H, window=Wn), *W, H=H)
    h = 1e-7
    for trial in range(3):
        dx_dir = rng.standard_normal(x.shape)
        dW_dir = [rng.standard_normal(w.shape) for w in W]
        Lp = np.sum(dy * ob.block_fwd(x + h * dx_dir, *[w + h * d for w, d in zip(W, dW_dir)], H=H, window=Wn).y)
        Lm = np.sum(dy * ob.block_fwd(x - h * dx_dir, *[w - h * d for w, d in zip(W, dW_dir)], H=H, window=Wn).y)
        num = (Lp - Lm) / (2 * h)
        ana = np.sum(g["dx"] * dx_dir) + sum(np.sum(g[n] * d) for n, d in zip(("dw_qkv", "dw_o", "dw_fc", "dw_proj"), dW_dir))
        assert math.isclose(ana, num, rel_tol=1e-7), (ana, num)


def test_window_block_locality():
    # with a window W, output row t depends on input rows t-W+1 .. t only
    rng = np.random.default_rng(26)
    B, T, C, H, Wn = 1, 10, 256, 2, 3
    x = rng.standard_normal((B, T, C))
    W = _weights(rng, C, 4 * C, H, 0.05)
    y0 = ob.block_fwd(x, *W, H=H, window=Wn).y
    x2 = x.copy()
    x2[0, 2] += 1.0
    y1 = ob.block_fwd(x2, *W, H=H, window=Wn).y
    changed = np.any(y0[0] != y1[0], axis=-1)
    assert np.array_equal(np.nonzero(changed)[0], np.arange(2, 2 + Wn))


# ------------------------------------------------- grouped-query attention
def _gqa_weights(rng, C, F, H, G, scale=0.05):
    D = C // H
    return (rng.standard_normal(((H + 2 * G) * D, C)) * scale, rng.standard_normal((C, C)) * scale,
            rng.standard_normal((F, C)) * scale, rng.standard_normal((C, F)) * scale)


def _as_mha(w_qkv, H, G, D):
    """MHA projection whose key/value heads repeat the G grouped ones: head h
    gets the rows of key/value head h // (H/G)."""
    C = H * D
    q, k, v = w_qkv[:C], w_qkv[C:C + G * D], w_qkv[C + G * D:]
    rep = lambda z: np.concatenate([z[(h // (H // G)) * D:(h // (H // G) + 1) * D] for h in range(H)])
    return np.concatenate([q, rep(k), rep(v)])


@pytest.mark.parametrize("G", [1, 2])
def test_gqa_equals_mha_with_repeated_kv_weights(G):
    rng = np.random.default_rng(41)
    B, T, C, H = 2, 6, 512, 4
    D = C // H
    W = _gqa_weights(rng, C, 4 * C, H, G)
    x = rng.standard_normal((B, T, C))
    dy = rng.standard_normal((B, T, C))
    Wm = (_as_mha(W[0], H, G, D),) + W[1:]
    cg = ob.block_fwd(x, *W, H=H, n_kv_head=G)
    cm = ob.block_fwd(x, *Wm, H=H)
    assert np.allclose(cg.y, cm.y, rtol=1e-12, atol=1e-12)
    gg = ob.block_bwd(dy, cg, *W, H=H)
    gm = ob.block_bwd(dy, cm, *Wm, H=H)
    assert np.allclose(gg["dx"], gm["dx"], rtol=1e-11, atol=1e-12)
    for k in ("dw_o", "dw_fc", "dw_proj"):
        assert np.allclose(gg[k], gm[k], rtol=1e-11, atol=1e-12), k
    # a shared parameter's gradient is the sum over its copies
    C_ = H * D
    dm = gm["dw_qkv"]
    assert np.allclose(gg["dw_qkv"][:C_], dm[:C_], rtol=1e-11, atol=1e-12)
    for part in range(2):
        blk = dm[C_ + part * C_:C_ + (part + 1) * C_].reshape(G, H // G, D, C).sum(axis=1).reshape(G * D, C)
        got = gg["dw_qkv"][C_ + part * G * D:C_ + (part + 1) * G * D]
        assert np.allclose(got, blk, rtol=1e-11, atol=1e-12)


def test_gqa_g_equals_h_is_mha():
    rng = np.random.default_rng(42)
    x = rng.standard_normal((1, 5, 256))
    W = _weights(rng, 256, 1024, 2, 0.05)
    assert np.array_equal(ob.block_fwd(x, *W, H=2, n_kv_head=2).y, ob.block_fwd(x, *W, H=2).y)


def test_gqa_block_bwd_central_differences():
    rng = np.random.default_rng(43)
    B, T, C, H, G = 1, 5, 512, 4, 2
    x = rng.standard_normal((B, T, C))
    W = _gqa_weights(rng, C, 4 * C, H, G)
    dy = rng.standard_normal((B, T, C))
    g = ob.block_bwd(dy, ob.block_fwd(x, *W, H=H, n_kv_head=G), *W, H=H)
    h = 1e-7
    for trial in range(3):
        dx_dir = rng.standard_normal(x.shape)
        dW_dir = [rng.standard_normal(w.shape) for w in W]
        Lp = np.sum(dy * ob.block_fwd(x + h * dx_dir, *[w + h * d for w, d in zip(W, dW_dir)], H=H, n_kv_head=G).y)
        Lm = np.sum(dy * ob.block_fwd(x - h * dx_dir, *[w - h * d for w, d in zip(W, dW_dir)], H=H, n_kv_head=G).y)
        num = (Lp - Lm) / (2 * h)
        ana = np.sum(g["dx"] * dx_dir) + sum(np.sum(g[n] * d) for n, d in zip(("dw_qkv", "dw_o", "dw_fc", "dw_proj"), dW_dir))
        assert math.isclose(ana, num, rel_tol=1e-7), (ana, num)


def test_gqa_decode_equals_prefill_row():
    rng = np.random.default_rng(44)
    B, C, H, G, S = 2, 512, 4, 1, 12
    D = C // H
    W = _gqa_weights(rng, C, 4 * C, H, G)
    lens = np.array([4, 9])
    xs = rng.standard_normal((B, S, C))
    kc = rng.standard_normal((B, G, S, D))
    vc = rng.standard_normal((B, G, S, D))
    for b in range(B):
        L = int(lens[b])
        c = ob.block_fwd(xs[b:b + 1, :L + 1], *W, H=H, n_kv_head=G)
        kc[b, :, :L] = c.kn[0, :, :L]
        vc[b, :, :L] = c.v[0, :, :L]
    xnew = np.stack([xs[b, lens[b]] for b in range(B)])
    y, kc2, _ = ob.decode_step(xnew, *W, kc, vc, lens, H=H, n_kv_head=G)
    for b in range(B):
        L = int(lens[b])
        ref = ob.block_fwd(xs[b:b + 1, :L + 1], *W, H=H, n_kv_head=G)
        assert np.allclose(y[b], ref.y[0, L], rtol=1e-11, atol=1e-11)
        assert np.allclose(kc2[b, :, L], ref.kn[0, :, L], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ block
def _loss_grads(shape_kw, seed=0, wscale=0.3):
    rng = np.random.default_rng(seed)
    B, T, C, H = shape_kw["B"], shape_kw["T"], shape_kw["C"], shape_kw["H"]
    F = 4 * C
    x = rng.standard_normal((B, T, C))
    W = _weights(rng, C, F, H, wscale)
    dy = rng.standard_normal((B, T, C))
    return x, W, dy


@pytest.mark.parametrize("B,T,C,H,eps", [(2, 5, 8, 2, 1e-6), (1, 4, 12, 3, 1e-2)])
def test_block_bwd_central_differences_every_coordinate(B, T, C, H, eps):
    x, W, dy = _loss_grads(dict(B=B, T=T, C=C, H=H))
    base = 10.0

    def L(x_, W_):
        return float(np.sum(dy * ob.block_fwd(x_, *W_, H=H, eps=eps, rope_base=base).y))

    cache = ob.block_fwd(x, *W, H=H, eps=eps, rope_base=base)
    g = ob.block_bwd(dy, cache, *W, H=H)
    h = 1e-6

    def fd(arr_get, shape):
        out = np.zeros(shape)
        for idx in np.ndindex(shape):
            vals = []
            for sgn in (1, -1):
                xx, WW = arr_get(idx, sgn * h)
                vals.append(L(xx, WW))
            out[idx] = (vals[0] - vals[1]) / (2 * h)
        return out

    def bump_x(idx, d):
        xx = x.copy(); xx[idx] += d
        return xx, W

    num = fd(bump_x, x.shape)
    assert np.allclose(g["dx"], num, rtol=1e-6, atol=1e-7)
    for wi, name in enumerate(("dw_qkv", "dw_o", "dw_fc", "dw_proj")):
        def bump_w(idx, d, wi=wi):
            WW = [w.copy() for w in W]; WW[wi][idx] += d
            return x, WW
        num = fd(bump_w, W[wi].shape)
        assert np.allclose(g[name], num, rtol=1e-6, atol=1e-7), name


def test_block_bwd_directional_derivative_head_dim_128():
    # the specified head size: D = 128, C = 256, T = 6; a few random directions
    rng = np.random.default_rng(11)
    B, T, C, H = 1, 6, 256, 2
    x = rng.standard_normal((B, T, C))
    W = _weights(rng, C, 4 * C, H, 0.05)
    dy = rng.standard_normal((B, T, C))
    cache = ob.block_fwd(x, *W, H=H)
    g = ob.block_bwd(dy, cache, *W, H=H)
    # small step: larger ones let some MLP pre-activations cross the ReLU^2
    # kink at 0, where the second derivative jumps and central differences
    # lose their h^2 accuracy
    h = 1e-7
    for trial in range(3):
        dx_dir = rng.standard_normal(x.shape)
        dW_dir = [rng.standard_normal(w.shape) for w in W]
        Lp = np.sum(dy * ob.block_fwd(x + h * dx_dir, *[w + h * d for w, d in zip(W, dW_dir)], H=H).y)
        Lm = np.sum(dy * ob.block_fwd(x - h * dx_dir, *[w - h * d for w, d in zip(W, dW_dir)], H=H).y)
        num = (Lp - Lm) / (2 * h)
        ana = np.sum(g["dx"] * dx_dir) + sum(np.sum(g[n] * d) for n, d in zip(("dw_qkv", "dw_o", "dw_fc", "dw_proj"), dW_dir))
        assert math.isclose(ana, num, rel_tol=1e-7), (ana, num)


def test_block_bwd_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    x, W, dy = _loss_grads(dict(B=2, T=9, C=256, H=2), seed=3, wscale=0.05)
    H, eps, base = 2, 1e-6, 10000.0
    cache = ob.block_fwd(x, *W, H=H, eps=eps, rope_base=base)
    g = ob.block_bwd(dy, cache, *W, H=H)

    # the same forward written with torch ops; gradients by torch autograd
    tx = torch.tensor(x, requires_grad=True)
    tW = [torch.tensor(w, requires_grad=True) for w in W]
    B, T, C = x.shape
    D = C // H

    def norm(z):
        return z * torch.rsqrt(z.pow(2).mean(-1, keepdim=True) + eps)

    h1 = norm(tx)
    q, k, v = (h1 @ tW[0].T).split(C, dim=-1)
    q, k, v = (t.view(B, T, H, D).transpose(1, 2) for t in (q, k, v))
    inv = base ** (-torch.arange(0, D // 2, dtype=torch.float64) * 2 / D)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None]
    c, s = ang.cos(), ang.sin()

    def rot(z):
        z1, z2 = z[..., :D // 2], z[..., D // 2:]
        return torch.cat([z1 * c - z2 * s, z1 * s + z2 * c], -1)

    q, k = norm(rot(q)), norm(rot(k))
    sc = (q @ k.transpose(-1, -2)) / math.sqrt(D)
    sc = sc.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    o = (sc.softmax(-1) @ v).transpose(1, 2).reshape(B, T, C)
    y1 = tx + o @ tW[1].T
    y = y1 + torch.relu(norm(y1) @ tW[2].T).square() @ tW[3].T
    (y * torch.tensor(dy)).sum().backward()
    assert np.allclose(y.detach().numpy(), cache.y, rtol=1e-12, atol=1e-12)
    assert np.allclose(tx.grad.numpy(), g["dx"], rtol=1e-10, atol=1e-12)
    for t, n in zip(tW, ("dw_qkv", "dw_o", "dw_fc", "dw_proj")):
        assert np.allclose(t.grad.numpy(), g[n], rtol=1e-10, atol=1e-12), n


def test_block_causality_forward_and_anticausal_backward():
    x, W, dy = _loss_grads(dict(B=1, T=12, C=16, H=2), seed=5)
    H = 2
    t = 6
    c0 = ob.block_fwd(x, *W, H=H)
    x2 = x.copy()
    x2[:, t + 1:] = np.random.default_rng(99).standard_normal(x2[:, t + 1:].shape)
    c1 = ob.block_fwd(x2, *W, H=H)
    assert np.allclose(c0.y[:, :t + 1], c1.y[:, :t + 1], rtol=1e-14, atol=1e-14)
    assert not np.allclose(c0.y[:, t + 1:], c1.y[:, t + 1:])
    # upstream gradient at positions < s cannot reach inputs at positions >= s
    s = 5
    dy2 = dy.copy()
    dy2[:, :s] = 0
    g0 = ob.block_bwd(dy, c0, *W, H=H)
    g1 = ob.block_bwd(dy2, c0, *W, H=H)
    assert np.allclose(g0["dx"][:, s:], g1["dx"][:, s:], rtol=1e-12, atol=1e-13)


def test_block_t1_is_value_path():
    rng = np.random.default_rng(8)
    B, C, H = 3, 16, 2
    x = rng.standard_normal((B, 1, C))
    W = _weights(rng, C, 4 * C, H)
    c = ob.block_fwd(x, *W, H=H)
    h1, _ = ob.rmsnorm(x, 1e-6)
    vpath = h1 @ W[0][2 * C:].T
    y1 = x + vpath @ W[1].T
    y = y1 + ob.relu2(ob.rmsnorm(y1, 1e-6)[0] @ W[2].T) @ W[3].T
    assert np.allclose(c.y, y, rtol=1e-13, atol=1e-13)
    g = ob.block_bwd(rng.standard_normal((B, 1, C)), c, *W, H=H)
    # the q and k rows receive no gradient (zero up to the rounding of
    # do.v - rowsum(do*o), two orders of the same sum)
    assert np.max(np.abs(g["dw_qkv"][:2 * C])) < 1e-12 * np.max(np.abs(g["dw_qkv"][2 * C:]))


def test_block_batch_additivity_of_weight_gradients():
    x, W, dy = _loss_grads(dict(B=3, T=7, C=16, H=2), seed=9)
    H = 2
    full = ob.block_bwd(dy, ob.block_fwd(x, *W, H=H), *W, H=H)
    parts = [ob.block_bwd(dy[b:b + 1], ob.block_fwd(x[b:b + 1], *W, H=H), *W, H=H) for b in range(3)]
    for n in ("dw_qkv", "dw_o", "dw_fc", "dw_proj"):
        assert np.allclose(full[n], sum(p[n] for p in parts), rtol=1e-12, atol=1e-12)
    assert np.allclose(full["dx"], np.concatenate([p["dx"] for p in parts]), rtol=1e-13, atol=1e-14)


def test_block_adjoint_identity_full_d6_shape():
    # <dy, J dx_dir> = <J^T dy, dx_dir> at the full d6 fp32 workload shape
    sh = BlockShape(B=1, T=512, C=384, H=3, F=1536, dtype="f32")
    inp = make_block_inputs(sh, seed=0)
    W = (inp["w_qkv"], inp["w_o"], inp["w_fc"], inp["w_proj"])
    c = ob.block_fwd(inp["x"], *W, H=sh.H)
    g = ob.block_bwd(inp["dy"], c, *W, H=sh.H)
    rng = np.random.default_rng(12)
    d = rng.standard_normal(inp["x"].shape)
    h = 1e-5
    yp = ob.block_fwd(inp["x"] + h * d, *W, H=sh.H).y
    ym = ob.block_fwd(inp["x"] - h * d, *W, H=sh.H).y
    lhs = np.sum(inp["dy"] * (yp - ym)) / (2 * h)
    rhs = np.sum(g["dx"] * d)
    assert math.isclose(lhs, rhs, rel_tol=1e-7)


# ------------------------------------------------------------ decode
@pytest.mark.parametrize("ragged,window", [(False, None), (True, None), (True, 6)])
def test_decode_equals_prefill_row(ragged, window):
    rng = np.random.default_rng(13)
    B, C, H, S = 3, 256, 2, 20
    F = 4 * C
    W = _weights(rng, C, F, H, 0.05)
    lens = np.array([5, 11, 19]) if ragged else np.array([12, 12, 12])
    xs = rng.standard_normal((B, S, C))
    kc = rng.standard_normal((B, H, S, 128))
    vc = rng.standard_normal((B, H, S, 128))
    for b in range(B):
        L = int(lens[b])
        c = ob.block_fwd(xs[b:b + 1, :L + 1], *W, H=H, window=window)
        kc[b, :, :L] = c.kn[0, :, :L]
        vc[b, :, :L] = c.v[0, :, :L]
    xnew = np.stack([xs[b, lens[b]] for b in range(B)])
    y, kc2, vc2 = ob.decode_step(xnew, *W, kc, vc, lens, H=H, window=window)
    for b in range(B):
        L = int(lens[b])
        ref = ob.block_fwd(xs[b:b + 1, :L + 1], *W, H=H, window=window)
        assert np.allclose(y[b], ref.y[0, L], rtol=1e-11, atol=1e-11)
        assert np.allclose(kc2[b, :, L], ref.kn[0, :, L], rtol=1e-12, atol=1e-12)
        assert np.array_equal(kc2[b, :, L + 1:], kc[b, :, L + 1:])


def test_decode_ignores_slots_beyond_length():
    sh = DecodeShape(B=2, C=256, H=2, F=1024, S_max=40)
    inp = make_decode_inputs(sh, seed=1, ragged=True, ragged_lo=3, ragged_hi=30)
    W = (inp["w_qkv"], inp["w_o"], inp["w_fc"], inp["w_proj"])
    y0, _, _ = ob.decode_step(inp["x"], *W, inp["k_cache"], inp["v_cache"], inp["cache_len"], H=2)
    kc = inp["k_cache"].copy()
    for b in range(2):
        kc[b, :, inp["cache_len"][b]:] = 1e3
    y1, _, _ = ob.decode_step(inp["x"], *W, kc, inp["v_cache"], inp["cache_len"], H=2)
    assert np.array_equal(y0, y1)
