"""CPU float64 oracle of the language-model head and its loss: final RMSNorm,
untied lm_head, cross-entropy over the vocabulary.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library: plain numpy, float64 throughout, every
step written as its textbook definition.

Sources (titles of the pages the method is described on; sections named):
  [RU]  "nanochat: свой ChatGPT от токенизатора до чата" (ai.flicky.cc course
        page), section "Модель: что изменилось со времён GPT-2" -- the
        embedding and lm_head weights are not tied, norms carry no
        parameters, linear layers no bias; section "Метрики: bits per byte
        и CORE" -- the training loss is the (natural-log) cross-entropy,
        reported per byte of text.
  [CN]  "4小时100美元！Andrej Karpathy新开源项目nanochat ..." (CSDN article),
        section 一, item 1 -- a Llama-like dense transformer with untied
        embedding and unembedding.

Readings where the pages are silent (each is listed with its reason in the
design notes): a parameter-free RMSNorm (eps 1e-6) on the final residual
rows before the head, as in Llama-like stacks; logits z = h W^T with W
[V, C], no bias and no logit cap; loss = mean over the counted rows of
lse(z_i) - z_i[t_i]; rows whose target lies outside [0, V) are not counted;
with no counted row the loss and every gradient are zero.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from . import block

__all__ = ["lse_rows", "HeadCache", "head_loss", "head_loss_bwd"]


def lse_rows(z: np.ndarray) -> np.ndarray:
    """log sum_j exp(z[i, j]) per row, with the row maximum taken out first
    so that large logits do not overflow."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1)
    return m + np.log(np.sum(np.exp(z - m[..., None]), axis=-1))


@dataclasses.dataclass
class HeadCache:
    h: np.ndarray        # [N, C] normalised rows
    r: np.ndarray        # [N] 1/rms
    z: np.ndarray        # [N, V] logits
    lse: np.ndarray      # [N]
    targets: np.ndarray  # [N]
    count: int           # rows with a target in [0, V)


def head_loss(x, w_lm, targets, eps: float = 1e-6):
    """Mean cross-entropy of the final rows x [N, C] under the untied head
    w_lm [V, C] for integer targets [N] (outside [0, V): not counted).
    Returns (loss, cache)."""
    x = np.asarray(x, dtype=np.float64)
    w_lm = np.asarray(w_lm, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    h, r = block.rmsnorm(x, eps)
    z = h @ w_lm.T
    lse = lse_rows(z)
    counted = (t >= 0) & (t < w_lm.shape[0])
    n = int(np.count_nonzero(counted))
    rows = np.nonzero(counted)[0]
    nll = lse[rows] - z[rows, t[rows]]
    loss = float(np.sum(nll)) / n if n > 0 else 0.0
    return loss, HeadCache(h=h, r=r, z=z, lse=lse, targets=t, count=n)


def head_loss_bwd(dloss: float, cache: HeadCache, w_lm):
    """Gradients of dloss * loss: dz = dloss/n * (softmax(z) - onehot(t)) on
    counted rows (zero elsewhere); dh = dz W; dW = dz^T h; dx through the
    RMSNorm.  Returns dict dx [N, C], dw_lm [V, C]."""
    c = cache
    w_lm = np.asarray(w_lm, dtype=np.float64)
    N, V = c.z.shape
    if c.count == 0:
        return {"dx": np.zeros_like(c.h), "dw_lm": np.zeros_like(w_lm)}
    p = np.exp(c.z - c.lse[:, None])
    counted = (c.targets >= 0) & (c.targets < V)
    rows = np.nonzero(counted)[0]
    p[rows, c.targets[rows]] -= 1.0
    p[~counted] = 0.0
    dz = p * (float(dloss) / c.count)
    dh = dz @ w_lm
    dw = dz.T @ c.h
    dx = block.rmsnorm_bwd(dh, c.h, c.r)
    return {"dx": dx, "dw_lm": dw}
