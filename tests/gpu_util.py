"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
block through the C ABI, compare against the oracle.

Every output buffer (and the saved and scratch stores) is filled with NaN
bits before each call, so an element that no kernel writes fails the
comparison instead of passing on a previous call's value.  Each output
tensor is gated three ways: relative Frobenius error, max|err| / max|ref|,
and (for the row outputs y, dx) the relative error of every single row."""
from __future__ import annotations

import sys

import numpy as np

from blockinputs import BlockShape, to_storage

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
# a single row of y or dx may be at most this many times the tensor's
# tolerance away from the oracle (relative to that row's norm)
ROW_FACTOR = 5.0


def poison_(t):
    """Fill a device buffer with NaN: float tensors with NaN, byte and integer
    buffers with all-ones bytes (a NaN in bf16 and in float32)."""
    import torch
    if t is None:
        return t
    if t.dtype.is_floating_point:
        t.fill_(float("nan"))
    elif t.dtype == torch.uint8:
        t.fill_(0xFF)
    else:
        t.fill_(-1)
    return t


def note(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def to_dev(a: np.ndarray, dtype: str):
    import torch
    st = to_storage(a, dtype)
    if dtype == "bf16":
        t = torch.from_numpy(st.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(st.copy())
    return t.to("cuda:0")


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def cfg_of(sh: BlockShape):
    import backward_gpt_block_amd as bl
    return bl.BlockConfig(B=sh.B, T=sh.T, C=sh.C, H=sh.H, F=sh.F, eps=sh.eps, rope_base=sh.rope_base,
                          dtype=bl.BLK_BF16 if sh.dtype == "bf16" else bl.BLK_F32,
                          gemm=bl.BLK_GEMM_FP8_E4M3 if sh.gemm == "fp8" else bl.BLK_GEMM_NATIVE, window=sh.window,
                          n_kv_head=sh.n_kv_head)


class GpuBlock:
    """Device buffers for one shape; fwd/bwd through the C ABI."""

    def __init__(self, sh: BlockShape, inp: dict):
        import torch
        import backward_gpt_block_amd as bl
        self.sh = sh
        self.cfg = cfg_of(sh)
        dt = sh.dtype
        self.x = to_dev(inp["x"], dt)
        self.w = [to_dev(inp[k], dt) for k in ("w_qkv", "w_o", "w_fc", "w_proj")]
        self.dy = to_dev(inp["dy"], dt)
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        self.dw = [torch.empty(w.shape, dtype=torch.float32, device="cuda:0") for w in self.w]
        self.saved = torch.empty(bl.block_saved_bytes(self.cfg), dtype=torch.uint8, device="cuda:0")
        self.scratch = torch.empty(bl.block_scratch_bytes(self.cfg), dtype=torch.uint8, device="cuda:0")

    def fwd(self, x=None):
        import backward_gpt_block_amd as bl
        for t in (self.y, self.saved, self.scratch):
            poison_(t)
        bl.block_fwd(self.cfg, self.x if x is None else x, *self.w, self.y, self.saved, self.scratch)

    def bwd(self, dy=None, accumulate=0):
        import backward_gpt_block_amd as bl
        poison_(self.dx)
        poison_(self.scratch)
        if not accumulate:
            for t in self.dw:
                poison_(t)
        bl.block_bwd(self.cfg, self.dy if dy is None else dy, self.x, *self.w, self.saved, self.dx, *self.dw,
                     accumulate, self.scratch)

    def results(self):
        import torch
        torch.cuda.synchronize()
        out = {"y": to_np(self.y), "dx": to_np(self.dx)}
        for k, t in zip(("dw_qkv", "dw_o", "dw_fc", "dw_proj"), self.dw):
            out[k] = to_np(t)
        return out


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Relative Frobenius error ||gpu - ref|| / ||ref||."""
    den = float(np.linalg.norm(ref.ravel()))
    return float(np.linalg.norm((gpu - ref).ravel())) / (den if den > 0 else 1.0)


def oracle_step(sh: BlockShape, inp: dict, batch=None):
    from oracle import block as ob
    sl = slice(None) if batch is None else batch
    x = inp["x"][sl]
    dy = inp["dy"][sl]
    W = (inp["w_qkv"], inp["w_o"], inp["w_fc"], inp["w_proj"])
    c = ob.block_fwd(x, *W, H=sh.H, eps=sh.eps, rope_base=sh.rope_base, window=sh.window or None,
                     n_kv_head=sh.n_kv_head or None)
    g = ob.block_bwd(dy, c, *W, H=sh.H)
    g["y"] = c.y
    return g


def max_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / max |ref| over the whole tensor."""
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(gpu - ref))) / (den if den > 0 else 1.0) if ref.size else 0.0


def row_errs(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative error of every row (last axis) against that row's norm; a row
    whose reference norm is below 1e-3 of the median row norm is measured
    against that floor."""
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    den = np.linalg.norm(r, axis=1)
    floor = 1e-3 * float(np.median(den)) if den.size else 0.0
    den = np.maximum(den, floor if floor > 0 else 1.0)
    return np.linalg.norm(g - r, axis=1) / den


ROW_KEYS = ("y", "dx")


def compare(gpu: dict, ref: dict, tol: float, keys=("y", "dx", "dw_qkv", "dw_o", "dw_fc", "dw_proj"),
            row_keys=ROW_KEYS, max_tol=None):
    """Gate every tensor in `keys`: all elements finite, relative Frobenius
    error <= tol, max|err|/max|ref| <= tol (or max_tol[key]); rows of the
    `row_keys` tensors each <= ROW_FACTOR * tol.  Returns the Frobenius
    errors."""
    max_tol = max_tol or {}
    for k in keys:
        bad = int(np.count_nonzero(~np.isfinite(gpu[k])))
        assert bad == 0, f"{k}: {bad} elements not finite (unwritten or NaN)"
    errs = {k: rel_err(gpu[k], ref[k]) for k in keys}
    mx = {k: max_err(gpu[k], ref[k]) for k in keys}
    rows = {k: float(np.max(row_errs(gpu[k], ref[k]))) for k in keys if k in row_keys and gpu[k].size}
    print("  rel errs (Frobenius / max|err|/max|ref|): "
          + ", ".join(f"{k}={errs[k]:.2e}/{mx[k]:.2e}" for k in keys), flush=True)
    if rows:
        print("  worst row: " + ", ".join(f"{k}={v:.2e}" for k, v in rows.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"relative Frobenius error above {tol}: {bad}"
    bad = {k: v for k, v in mx.items() if not (v <= max_tol.get(k, tol))}
    assert not bad, f"max|err|/max|ref| above {tol} ({max_tol}): {bad}"
    bad = {k: v for k, v in rows.items() if not (v <= ROW_FACTOR * tol)}
    assert not bad, f"a row's relative error above {ROW_FACTOR * tol}: {bad}"
    return errs


def check_forward_rows(y_gpu: np.ndarray, sh: BlockShape, inp: dict, seqs, tol: float):
    """Compare y of the sequences `seqs` with the oracle's forward, one
    sequence at a time (forward only: the check of sequences whose upstream
    gradient a sampled test leaves at zero)."""
    from oracle import block as ob
    W = (inp["w_qkv"], inp["w_o"], inp["w_fc"], inp["w_proj"])
    worst = (0.0, 0.0, 0.0)
    for b in seqs:
        c = ob.block_fwd(inp["x"][b:b + 1], *W, H=sh.H, eps=sh.eps, rope_base=sh.rope_base,
                         window=sh.window or None, n_kv_head=sh.n_kv_head or None)
        got = y_gpu[b:b + 1]
        assert np.all(np.isfinite(got)), f"y of sequence {b} not finite"
        e = (rel_err(got, c.y), max_err(got, c.y), float(np.max(row_errs(got, c.y))))
        worst = tuple(max(a, x) for a, x in zip(worst, e))
        assert e[0] <= tol and e[1] <= tol and e[2] <= ROW_FACTOR * tol, (b, e)
    print(f"  forward of {len(list(seqs))} further sequences: worst Frobenius {worst[0]:.2e}, "
          f"max-ratio {worst[1]:.2e}, row {worst[2]:.2e}", flush=True)
    return worst
