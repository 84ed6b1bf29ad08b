"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
block through the C ABI, compare against the oracle."""
from __future__ import annotations

import sys

import numpy as np

from blockinputs import BlockShape, to_storage

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


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
        bl.block_fwd(self.cfg, self.x if x is None else x, *self.w, self.y, self.saved, self.scratch)

    def bwd(self, dy=None, accumulate=0):
        import backward_gpt_block_amd as bl
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


def compare(gpu: dict, ref: dict, tol: float, keys=("y", "dx", "dw_qkv", "dw_o", "dw_fc", "dw_proj")):
    errs = {k: rel_err(gpu[k], ref[k]) for k in keys}
    print("  rel errs: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    assert not bad, f"relative Frobenius error above {tol}: {bad}"
    for k in keys:
        assert np.all(np.isfinite(gpu[k])), k
    return errs
