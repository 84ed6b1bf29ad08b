"""decode_step_noalloc (the decode step with its temporaries in the library's
static per-device workspace) against decode_step with a caller-supplied
scratch buffer: same inputs, bitwise the same outputs (y and both caches),
on two calls in a row, the second with a smaller configuration; and a
configuration whose workspace exceeds the static one is refused."""
import numpy as np
import pytest

from blockinputs import DECODE_WORKLOADS, DecodeShape, make_decode_inputs

from gpu_util import note, poison_, to_dev

pytestmark = pytest.mark.gpu

WNAMES = ("w_qkv", "w_o", "w_fc", "w_proj")


def _pair(sh: DecodeShape, seed: int, **kw):
    import torch
    import backward_gpt_block_amd as bl
    note(f"no-alloc decode B={sh.B} C={sh.C} S_max={sh.S_max} G={sh.n_kv_head} {kw}")
    inp = make_decode_inputs(sh, seed=seed, **kw)
    cfg = bl.DecodeConfig(B=sh.B, C=sh.C, H=sh.H, F=sh.F, S_max=sh.S_max, window=sh.window, n_kv_head=sh.n_kv_head)
    assert bl.decode_scratch_bytes(cfg) <= bl.binding.BLK_NOALLOC_SCRATCH_BYTES
    W = [to_dev(inp[k], "bf16") for k in WNAMES]
    x = to_dev(inp["x"], "bf16")
    lens = torch.from_numpy(inp["cache_len"].astype(np.int32)).to("cuda:0")
    out = []
    for noalloc in (False, True):
        kc, vc = to_dev(inp["k_cache"], "bf16"), to_dev(inp["v_cache"], "bf16")
        y = poison_(torch.empty_like(x))
        if noalloc:
            bl.decode_step_noalloc(cfg, x, *W, kc, vc, lens, y)
        else:
            scratch = poison_(torch.empty(bl.decode_scratch_bytes(cfg), dtype=torch.uint8, device="cuda:0"))
            bl.decode_step(cfg, x, *W, kc, vc, lens, y, scratch)
        torch.cuda.synchronize()
        out.append([t.view(torch.int16).cpu().numpy() for t in (y, kc, vc)])
    for name, a, b in zip(("y", "k_cache", "v_cache"), *out):
        assert np.array_equal(a, b), f"{name}: {np.count_nonzero(a != b)} elements differ"
    yf = out[1][0].view(np.uint16).astype(np.uint32) << 16
    assert np.all(np.isfinite(yf.view(np.float32)))


def test_noalloc_decode_matches_decode_step_twice():
    # the full d20 decode workload, then a smaller configuration on the same
    # (shared, reused) static workspace
    _pair(DECODE_WORKLOADS["d20_decode"], seed=0, ragged=True, ragged_lo=128, ragged_hi=2048)
    _pair(DecodeShape(B=5, C=384, H=3, F=1536, S_max=300, window=100, n_kv_head=1), seed=3, ragged=True,
          ragged_lo=0)


def test_noalloc_decode_refuses_oversize_workspace():
    import backward_gpt_block_amd as bl
    cfg = bl.DecodeConfig(B=1024, C=2048, H=16, F=8192, S_max=4096)
    assert bl.decode_scratch_bytes(cfg) > bl.binding.BLK_NOALLOC_SCRATCH_BYTES
    code = bl.decode_step_noalloc(cfg, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x20000, 0x30000, 0x10000,
                                  0x10000, raise_on_error=False)
    assert code == bl.binding.BLK_ELIMIT
