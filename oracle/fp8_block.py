"""CPU float64 oracle of the decoder block with fp8 (E4M3) linear layers.

TEST INFRASTRUCTURE ONLY (see oracle/block.py).

The fp8 mode computes the same block as oracle/block.py, except that every
GEMM of the four linear layers takes its two operands rounded to E4M3 with
per-tensor current scaling (oracle/fp8.py) and accumulates exactly; the
attention, the norms, rotary and the residual adds are unquantised.  This
oracle is that definition written out in float64, so the GPU's fp8 path is
checked against it; its distance from the unquantised block is the recipe's
own error, reported beside the gate.

The fp8 mode runs on a bf16 pipeline, and a code choice is a floating-point
decision: it is taken on the tensor as that pipeline holds it.  So the
oracle rounds to bf16 each intermediate the pipeline stores in bf16 (the
`store` rounding: h1, the rotated and normalised q and k and v, o, y1, h2,
a; du, dh2, dy1, dO, dqkv, dh1), takes the ReLU^2 derivative 2 max(u, 0) as
2 sqrt(a) from the stored a, and quantises the bf16 values (quant_bf16).
Every E4M3 code is a discontinuous function of its input, so a difference
of one bf16 rounding upstream moves a share of the codes downstream to the
neighbouring code, and that share grows along the chain of quantisations;
taking the same roundings keeps the code decisions of the oracle and the
kernels apart only by float32-versus-float64 arithmetic and the attention
kernels' own roundings.  Everything else (the GEMM sums, attention, norms,
rotary) is exact float64.

Quantised operands (each tensor once, with its own scale):
  forward   h1 x W_qkv, o x W_o, h2 x W_fc, a x W_proj
  backward  dy x W_proj, dy^T x a, du x W_fc, du^T x h2, dy1 x W_o,
            dy1^T x o, dqkv x W_qkv, dqkv^T x h1
(FP8 training of the linear layers: flicky.cc nanochat page, repository map
row for nanochat/fp8.py; the README mirror's leaderboard row "+fp8".)

Per-tensor scales belong to whole tensors.  To check a few sequences of a
large batch, `batch` selects them: the forward scales (h1, o, h2, a) are then
taken over the whole batch by a forward pass, and the upstream gradient must
be zero outside the selected sequences, which makes every backward tensor
zero there too, so its scale over the selection is its scale over the batch.
"""
from __future__ import annotations

import numpy as np

from . import block as ob
from .fp8 import fake_quant, round_bf16


def quant_bf16(t, amax=None):
    """The block's operand rounding: the tensor as bf16 storage holds it,
    then the E4M3 round trip with its per-tensor scale."""
    return fake_quant(round_bf16(t), amax)


def _heads(z, H):
    B, T, C = z.shape
    return z.reshape(B, T, H, C // H).transpose(0, 2, 1, 3)


def _merge(z):
    B, H, T, D = z.shape
    return z.transpose(0, 2, 1, 3).reshape(B, T, H * D)


def _amax(z) -> float:
    return float(np.max(np.abs(round_bf16(z)))) if z.size else 0.0


def _attention_out(h1q, Wq, H, eps, rope_base, window=None, G=None, store=round_bf16):
    """Rotary, QK-norm and causal (optionally sliding-window, optionally
    grouped: G key/value heads) attention of one chunk of sequences from the
    quantised h1 and W_qkv; the normalised q, k and v as stored (`store`);
    returns o (B,T,C) before its own storage rounding, and what the backward
    needs."""
    B, T, C = h1q.shape
    G = H if G is None else G
    qkv = h1q @ Wq.T
    q, k, v = ob.split_qkv(qkv, H, G, C // H)
    cos, sin = ob.rope_tables(np.arange(T), C // H, rope_base)
    qn, rho_q = ob.rmsnorm(ob.rope(q, cos, sin), eps)
    kn, rho_k = ob.rmsnorm(ob.rope(k, cos, sin), eps)
    qn, kn, v = store(qn), store(kn), store(v)
    oh, P = ob.causal_attention(qn, ob.repeat_kv(kn, H), ob.repeat_kv(v, H), window)
    return _merge(oh), (cos, sin, qn, rho_q, kn, rho_k, v, P)


def forward_amax(x, w_qkv, w_o, w_fc, H: int, eps: float = 1e-6, rope_base: float = 10000.0, quant=quant_bf16,
                 log=None, window=None, n_kv_head=None, store=round_bf16):
    """Absolute maxima of the four quantised forward activations h1, o, h2, a
    over the whole batch, computed one sequence at a time (`log(msg)` is
    called after each pass, for long runs)."""
    log = log or (lambda msg: None)
    x = np.asarray(x, dtype=np.float64)
    Wq, Wo, Wf = (quant(w) for w in (w_qkv, w_o, w_fc))
    h1 = store(ob.rmsnorm(x, eps)[0])
    m_h1 = _amax(h1)
    o = store(np.concatenate([_attention_out(quant(h1[b:b + 1], m_h1), Wq, H, eps, rope_base, window, n_kv_head,
                                             store)[0] for b in range(x.shape[0])]))
    m_o = _amax(o)
    log("fp8 oracle: attention pass done")
    h2 = store(ob.rmsnorm(store(x + quant(o, m_o) @ Wo.T), eps)[0])
    m_h2 = _amax(h2)
    m_a = max(_amax(ob.relu2(quant(h2[b:b + 1], m_h2) @ Wf.T)) for b in range(x.shape[0]))
    log("fp8 oracle: forward scales done")
    return {"h1": m_h1, "o": m_o, "h2": m_h2, "a": m_a}


def block_fwd_bwd(x, w_qkv, w_o, w_fc, w_proj, dy, H: int, eps: float = 1e-6, rope_base: float = 10000.0,
                  batch=None, quant=quant_bf16, log=None, window=None, n_kv_head=None, store=round_bf16):
    """Returns dict y, dx, dw_qkv, dw_o, dw_fc, dw_proj (float64); with
    `batch` (a list of sequence indices) y and dx cover those sequences only.
    `quant(t, amax=None)` is the operand rounding (E4M3 round trip), `store(t)`
    the rounding of a stored intermediate (bf16; the identity gives the block
    with only its GEMM operands rounded)."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(dy, dtype=np.float64)
    fa = None
    if batch is not None:
        rest = np.ones(x.shape[0], dtype=bool)
        rest[list(batch)] = False
        if np.any(g[rest] != 0):
            raise ValueError("the upstream gradient must be zero outside the selected sequences")
        fa = forward_amax(x, w_qkv, w_o, w_fc, H, eps, rope_base, quant, log, window, n_kv_head, store)
        x, g = x[list(batch)], g[list(batch)]
    amax = (lambda k: None) if fa is None else fa.get
    Wq, Wo, Wf, Wp = (quant(w) for w in (w_qkv, w_o, w_fc, w_proj))

    h1, r1 = ob.rmsnorm(x, eps)
    h1 = store(h1)
    h1q = quant(h1, amax("h1"))
    o, (cos, sin, qn, rho_q, kn, rho_k, v, P) = _attention_out(h1q, Wq, H, eps, rope_base, window, n_kv_head,
                                                               store)
    o = store(o)
    oq = quant(o, amax("o"))
    y1 = store(x + oq @ Wo.T)
    h2, r2 = ob.rmsnorm(y1, eps)
    h2 = store(h2)
    h2q = quant(h2, amax("h2"))
    u = h2q @ Wf.T
    a = store(ob.relu2(u))
    aq = quant(a, amax("a"))
    y = y1 + aq @ Wp.T

    flat = lambda z: z.reshape(-1, z.shape[-1])
    gq = quant(g)
    # the ReLU^2 derivative 2 max(u, 0), as 2 sqrt(a) from the stored a
    du = store((gq @ Wp) * 2.0 * np.sqrt(a))
    dw_proj = flat(gq).T @ flat(aq)
    duq = quant(du)
    dh2 = store(duq @ Wf)
    dw_fc = flat(duq).T @ flat(h2q)
    dy1 = store(g + ob.rmsnorm_bwd(dh2, h2, r2))
    dy1q = quant(dy1)
    do = _heads(store(dy1q @ Wo), H)
    dw_o = flat(dy1q).T @ flat(oq)
    dqn, dkn_r, dv_r = ob.causal_attention_bwd(do, qn, ob.repeat_kv(kn, H), ob.repeat_kv(v, H), _heads(o, H), P)
    dkn, dv = ob.sum_groups(dkn_r, kn.shape[1]), ob.sum_groups(dv_r, kn.shape[1])
    dq = ob.rope_bwd(ob.rmsnorm_bwd(dqn, qn, rho_q), cos, sin)
    dk = ob.rope_bwd(ob.rmsnorm_bwd(dkn, kn, rho_k), cos, sin)
    dqkv = store(np.concatenate([_merge(dq), _merge(dk), _merge(dv)], axis=-1))
    dqkvq = quant(dqkv)
    dh1 = store(dqkvq @ Wq)
    dw_qkv = flat(dqkvq).T @ flat(h1q)
    dx = dy1 + ob.rmsnorm_bwd(dh1, h1, r1)
    return {"y": y, "dx": dx, "dw_qkv": dw_qkv, "dw_o": dw_o, "dw_fc": dw_fc, "dw_proj": dw_proj}
