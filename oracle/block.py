"""CPU float64 oracle for one training step of the dense GPT decoder block.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library: plain numpy, float64 throughout, every
step written as its textbook definition (no blocking, fusion or reordering).

Sources (titles of the pages the method is described on; sections named):
  [RU]  "nanochat: свой ChatGPT от токенизатора до чата" (ai.flicky.cc course
        page), section "Модель: что изменилось со времён GPT-2" -- rotary
        position embeddings, QK-norm before attention, ReLU^2 MLP
        activation, parameter-free RMSNorm, no biases in linear layers; and
        its glossary entry for RMSNorm (x / sqrt(mean(x^2) + eps)).
  [CN]  "4小时100美元！Andrej Karpathy新开源项目nanochat，人人都能拥有专属
        ChatGPT" (CSDN article), section 一, item 1 -- dense Llama-like
        transformer, rotary embeddings, QK norm.
  [ES]  "Andrej Karpathy lanza nanochat ..." (7minutos.es), section
        "Modelo, escalado y objetivo de 'speedrun'" -- d20 is 1280 channels,
        10 heads of 128 dimensions.
  [ZH]  "karpathy/nanochat" README mirror (pigsec.cn), section "精度 / dtype"
        -- bf16 compute with fp32 master weights cast inside the linear layer.

Readings where the pages are silent (each is listed with its reason in the
design notes): pre-norm order norm->attention->residual, norm->MLP->residual;
eps = 1e-6 for the two block norms and QK-norm; rotary base 10000 with
half-split pairing (i, i + D/2), counter-clockwise rotation by t*base^(-2i/D),
positions counted from 0 per sequence; softmax scale 1/sqrt(D); causal mask
key <= query; fused QKV output split as [q | k | v] with heads contiguous in
each; weights stored [out, in] and applied as y = x W^T.

Grouped-query attention (optional, G key/value heads for H query heads, G
dividing H): [RU], same section, lists GQA support -- the query heads form
G groups and each group shares one K/V pair; G = H is multi-head attention.
The fused projection then has (H + 2G) heads of output, [q | k | v] with q
in H heads and k, v in G heads each; query head h uses key/value head
h // (H / G).

Sliding-window attention (optional window W): [RU], same section, names an
alternation of attention windows, three layers of four with a short window
of a quarter of the context and one with the full context (the last layer
always full).  The pages do not fix the window's boundary; read here as:
query i sees the W keys i - W < j <= i, itself included.  W >= T is the
causal mask.  Which layer gets which window is the caller's choice.

Backward: the adjoints of the forward steps, derived by hand; pinned in the
tests by central finite differences, an autograd cross-check and invariants.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "rmsnorm", "rmsnorm_bwd", "rope_tables", "rope", "rope_bwd",
    "visible", "causal_attention", "causal_attention_bwd", "online_causal_attention",
    "BlockCache", "block_fwd", "block_bwd", "decode_step", "relu2", "relu2_bwd",
]


# ---------------------------------------------------------------- RMSNorm
def rmsnorm(x: np.ndarray, eps: float):
    """Parameter-free RMSNorm over the last axis ([RU] glossary, without the
    gain g since the block's norms have no learnable parameters).
    Returns (h, r) with r = (mean(x^2) + eps)^(-1/2) and h = r * x."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r, r[..., 0]


def rmsnorm_bwd(dh: np.ndarray, h: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Adjoint of h = r(x) x:  dx = r * (dh - h * mean(dh * h))."""
    return r[..., None] * (dh - h * np.mean(dh * h, axis=-1, keepdims=True))


# ---------------------------------------------------------------- rotary
def rope_tables(positions: np.ndarray, D: int, base: float):
    """cos/sin of phi[t, i] = pos[t] * base^(-2i/D), i in [0, D/2)."""
    i = np.arange(D // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / D)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(phi), np.sin(phi)


def rope(z: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate each pair (z[i], z[i + D/2]) by phi ([RU], [CN]: rotary position
    embedding).  z: [..., T, D]; cos/sin: [T, D/2]."""
    d = z.shape[-1] // 2
    z1, z2 = z[..., :d], z[..., d:]
    return np.concatenate([z1 * cos - z2 * sin, z1 * sin + z2 * cos], axis=-1)


def rope_bwd(dz: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Adjoint of :func:`rope`: the transpose rotation, by -phi."""
    d = dz.shape[-1] // 2
    g1, g2 = dz[..., :d], dz[..., d:]
    return np.concatenate([g1 * cos + g2 * sin, -g1 * sin + g2 * cos], axis=-1)


# ---------------------------------------------------------------- attention
def visible(T: int, window=None) -> np.ndarray:
    """[T, T] boolean: query i sees key j when j <= i and, with a window W,
    j > i - W."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    vis = j <= i
    if window is not None:
        vis &= j > i - int(window)
    return vis


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, window=None):
    """softmax(q k^T / sqrt(D)) v over the keys :func:`visible` to each query
    (j <= i, and j > i - W with a window).  Materialises the full score
    matrix.  q, k, v: [..., T, D].  Returns (o, P)."""
    D = q.shape[-1]
    T = q.shape[-2]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / np.sqrt(D)
    s = np.where(visible(T, window), s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    P = e / np.sum(e, axis=-1, keepdims=True)
    return np.matmul(P, v), P


def causal_attention_bwd(do, q, k, v, o, P):
    """Adjoint of :func:`causal_attention` given the probabilities P.
    dv = P^T do;  dP = do v^T;  dS = P * (dP - rowsum(do * o));
    dq = dS k / sqrt(D);  dk = dS^T q / sqrt(D)."""
    D = q.shape[-1]
    dv = np.matmul(np.swapaxes(P, -1, -2), do)
    dP = np.matmul(do, np.swapaxes(v, -1, -2))
    delta = np.sum(do * o, axis=-1, keepdims=True)
    dS = P * (dP - delta)
    dq = np.matmul(dS, k) / np.sqrt(D)
    dk = np.matmul(np.swapaxes(dS, -1, -2), q) / np.sqrt(D)
    return dq, dk, dv


def online_causal_attention(q, k, v, block: int = 16, window=None):
    """Same result as :func:`causal_attention`, computed key block by key
    block with a running maximum and running denominator (the online softmax
    of flash-style attention).  Used only to cross-check the materialised
    form; returns (o, lse) with lse the natural log of the softmax
    denominator including the maximum."""
    D = q.shape[-1]
    T = q.shape[-2]
    lead = q.shape[:-2]
    m = np.full(lead + (T,), -np.inf)
    l = np.zeros(lead + (T,))
    acc = np.zeros(lead + (T, D))
    qi = np.arange(T)[:, None]
    for j0 in range(0, T, block):
        j1 = min(T, j0 + block)
        s = np.matmul(q, np.swapaxes(k[..., j0:j1, :], -1, -2)) / np.sqrt(D)
        kj = np.arange(j0, j1)[None, :]
        hidden = kj > qi
        if window is not None:
            hidden = hidden | (kj <= qi - int(window))
        s = np.where(hidden, -np.inf, s)
        m_new = np.maximum(m, np.max(s, axis=-1))
        alpha = np.where(np.isfinite(m_new), np.exp(m - m_new), 0.0)
        p = np.where(np.isfinite(m_new)[..., None], np.exp(s - m_new[..., None]), 0.0)
        l = alpha * l + np.sum(p, axis=-1)
        acc = alpha[..., None] * acc + np.matmul(p, v[..., j0:j1, :])
        m = m_new
    return acc / l[..., None], m + np.log(l)


# ---------------------------------------------------------------- MLP
def relu2(u):
    """ReLU^2, relu(u).square() ([RU] section on the model: the MLP
    activation replacing GELU)."""
    return np.square(np.maximum(u, 0.0))


def relu2_bwd(da, u):
    return da * 2.0 * np.maximum(u, 0.0)


# ---------------------------------------------------------------- block
@dataclasses.dataclass
class BlockCache:
    x: np.ndarray
    r1: np.ndarray
    h1: np.ndarray
    cos: np.ndarray
    sin: np.ndarray
    qr: np.ndarray      # after rotary, before QK-norm  [B,H,T,D]
    kr: np.ndarray
    rho_q: np.ndarray   # QK-norm factors               [B,H,T]
    rho_k: np.ndarray
    qn: np.ndarray      # after QK-norm                  [B,H,T,D]
    kn: np.ndarray      # [B,G,T,D] (G key/value heads; G = H without grouping)
    v: np.ndarray       # [B,G,T,D]
    P: np.ndarray       # attention probabilities       [B,H,T,T]
    o_heads: np.ndarray  # [B,H,T,D]
    o: np.ndarray       # heads concatenated            [B,T,C]
    y1: np.ndarray
    r2: np.ndarray
    h2: np.ndarray
    u: np.ndarray
    a: np.ndarray
    y: np.ndarray


def _heads(z, H):
    B, T, C = z.shape
    return z.reshape(B, T, H, C // H).transpose(0, 2, 1, 3)


def _merge(z):
    B, H, T, D = z.shape
    return z.transpose(0, 2, 1, 3).reshape(B, T, H * D)


def repeat_kv(z, H: int):
    """[B,G,T,D] -> [B,H,T,D]: key/value head g serves query heads
    g*(H/G) .. g*(H/G) + H/G - 1."""
    return np.repeat(z, H // z.shape[1], axis=1)


def sum_groups(dz, G: int):
    """Adjoint of :func:`repeat_kv`: [B,H,T,D] -> [B,G,T,D], summing each
    group's query heads."""
    B, H, T, D = dz.shape
    return dz.reshape(B, G, H // G, T, D).sum(axis=2)


def split_qkv(qkv, H: int, G: int, D: int):
    """Split the fused projection [B,T,(H+2G)D] into q [B,H,T,D] and
    k, v [B,G,T,D]."""
    C = H * D
    return (_heads(qkv[..., :C], H), _heads(qkv[..., C:C + G * D], G), _heads(qkv[..., C + G * D:], G))


def block_fwd(x, w_qkv, w_o, w_fc, w_proj, H: int, eps: float = 1e-6,
              rope_base: float = 10000.0, positions=None, window=None, n_kv_head=None) -> BlockCache:
    """Forward of the decoder block on x [B,T,C] (float64).

    1 RMSNorm; 2 fused QKV projection (no bias); 3 rotary on q, k;
    4 QK-norm; 5 causal multi-head attention (optionally sliding-window, and
    with G = n_kv_head key/value heads shared by groups of query heads);
    6 output projection plus residual; 7 RMSNorm; 8 MLP up-projection with
    ReLU^2; 9 down-projection plus residual.  [RU], [CN], [ES].
    w_qkv is [(H + 2G) D, C]."""
    x = np.asarray(x, dtype=np.float64)
    B, T, C = x.shape
    D = C // H
    G = H if n_kv_head is None else int(n_kv_head)
    h1, r1 = rmsnorm(x, eps)
    qkv = h1 @ w_qkv.T
    q, k, v = split_qkv(qkv, H, G, D)
    pos = np.arange(T) if positions is None else np.asarray(positions)
    cos, sin = rope_tables(pos, D, rope_base)
    qr, kr = rope(q, cos, sin), rope(k, cos, sin)
    qn, rho_q = rmsnorm(qr, eps)
    kn, rho_k = rmsnorm(kr, eps)
    o_heads, P = causal_attention(qn, repeat_kv(kn, H), repeat_kv(v, H), window)
    o = _merge(o_heads)
    y1 = x + o @ w_o.T
    h2, r2 = rmsnorm(y1, eps)
    u = h2 @ w_fc.T
    a = relu2(u)
    y = y1 + a @ w_proj.T
    return BlockCache(x=x, r1=r1, h1=h1, cos=cos, sin=sin, qr=qr, kr=kr,
                      rho_q=rho_q, rho_k=rho_k, qn=qn, kn=kn, v=v, P=P,
                      o_heads=o_heads, o=o, y1=y1, r2=r2, h2=h2, u=u, a=a, y=y)


def _flat(z):
    return z.reshape(-1, z.shape[-1])


def block_bwd(dy, cache: BlockCache, w_qkv, w_o, w_fc, w_proj, H: int):
    """Gradients of <dy, y> with respect to x and the four weights.
    Returns dict dx [B,T,C], dw_qkv, dw_o, dw_fc, dw_proj (float64)."""
    c = cache
    dy = np.asarray(dy, dtype=np.float64)
    # 9: y = y1 + a W_proj^T
    dw_proj = _flat(dy).T @ _flat(c.a)
    da = dy @ w_proj
    # 8: a = relu(u)^2, u = h2 W_fc^T
    du = relu2_bwd(da, c.u)
    dw_fc = _flat(du).T @ _flat(c.h2)
    dh2 = du @ w_fc
    # 7: h2 = rmsnorm(y1); y1 also feeds y directly
    dy1 = dy + rmsnorm_bwd(dh2, c.h2, c.r2)
    # 6: y1 = x + o W_o^T
    dw_o = _flat(dy1).T @ _flat(c.o)
    do = _heads(dy1 @ w_o, H)
    # 5: attention (over the key/value heads repeated to the query heads)
    G = c.kn.shape[1]
    dqn, dkn_r, dv_r = causal_attention_bwd(do, c.qn, repeat_kv(c.kn, H), repeat_kv(c.v, H), c.o_heads, c.P)
    dkn, dv = sum_groups(dkn_r, G), sum_groups(dv_r, G)
    # 4: QK-norm
    dqr = rmsnorm_bwd(dqn, c.qn, c.rho_q)
    dkr = rmsnorm_bwd(dkn, c.kn, c.rho_k)
    # 3: rotary
    dq = rope_bwd(dqr, c.cos, c.sin)
    dk = rope_bwd(dkr, c.cos, c.sin)
    # 2: fused QKV projection
    dqkv = np.concatenate([_merge(dq), _merge(dk), _merge(dv)], axis=-1)
    dw_qkv = _flat(dqkv).T @ _flat(c.h1)
    dh1 = dqkv @ w_qkv
    # 1: h1 = rmsnorm(x); x also feeds y1 directly
    dx = dy1 + rmsnorm_bwd(dh1, c.h1, c.r1)
    return {"dx": dx, "dw_qkv": dw_qkv, "dw_o": dw_o, "dw_fc": dw_fc, "dw_proj": dw_proj}


def decode_step(x, w_qkv, w_o, w_fc, w_proj, k_cache, v_cache, cache_len,
                H: int, eps: float = 1e-6, rope_base: float = 10000.0, window=None, n_kv_head=None):
    """One new token per sequence at position p = cache_len[b]: forward steps
    1-4 on that row, its k (after rotary and QK-norm) and v written at slot
    p, attention over slots 0..p (p-W+1..p with a window W), then steps 6-9.
    Inference with a KV
    cache and prefill/decode is named on the 7minutos.es page (section on
    midtraining, SFT and tool use) and in the launch thread.

    x [B,C]; caches [B,G,S,D] (post-rotary/QK-norm keys, values of the G
    key/value heads); returns (y [B,C], k_cache', v_cache') with the new
    slots written."""
    x = np.asarray(x, dtype=np.float64)
    B, C = x.shape
    D = C // H
    G = H if n_kv_head is None else int(n_kv_head)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    y = np.zeros_like(x)
    for b in range(B):
        p = int(cache_len[b])
        xb = x[b:b + 1]
        h1, _ = rmsnorm(xb, eps)
        qkv = h1 @ w_qkv.T
        q = qkv[0, :C].reshape(H, 1, D)
        k = qkv[0, C:C + G * D].reshape(G, 1, D)
        v = qkv[0, C + G * D:].reshape(G, 1, D)
        cos, sin = rope_tables(np.array([p]), D, rope_base)
        qn, _ = rmsnorm(rope(q, cos, sin), eps)
        kn, _ = rmsnorm(rope(k, cos, sin), eps)
        kc[b, :, p, :] = kn[:, 0, :]
        vc[b, :, p, :] = v[:, 0, :]
        j0 = 0 if window is None else max(0, p - int(window) + 1)
        keys = np.repeat(kc[b, :, j0:p + 1, :], H // G, axis=0)   # [H, p+1-j0, D]
        vals = np.repeat(vc[b, :, j0:p + 1, :], H // G, axis=0)
        s = np.matmul(qn, np.swapaxes(keys, -1, -2)) / np.sqrt(D)   # [H,1,p+1]
        e = np.exp(s - np.max(s, axis=-1, keepdims=True))
        Pb = e / np.sum(e, axis=-1, keepdims=True)
        o = np.matmul(Pb, vals).reshape(1, C)   # heads concatenated in order
        y1 = xb + o @ w_o.T
        h2, _ = rmsnorm(y1, eps)
        a = relu2(h2 @ w_fc.T)
        y[b] = (y1 + a @ w_proj.T)[0]
    return y, kc, vc
