"""GPU parity of decode_step against the float64 oracle (bf16 bar: 2e-2
relative Frobenius error and max|err|/max|ref|, every row of y within 5x;
y and the scratch start as NaN):

- y for every row;
- the new cache slot p = cache_len[b] of every (sequence, head), keys after
  rotary and QK-norm and values;
- every other cache slot bit for bit unchanged (the step writes one slot);

on ragged lengths (0, S_max-1, several 256-key splits, a ragged tail), more
rows than one 64-row tile, two chained steps, y written over x, and the full
d20 decode workload (64 sequences, caches of 2049 slots) with uniform and
ragged 128..2048 lengths."""
import numpy as np
import pytest

from blockinputs import DECODE_WORKLOADS, DecodeShape, make_decode_inputs

from gpu_util import ROW_FACTOR, TOL, max_err, note, poison_, rel_err, row_errs, to_dev, to_np

pytestmark = pytest.mark.gpu

WNAMES = ("w_qkv", "w_o", "w_fc", "w_proj")


class GpuDecode:
    def __init__(self, sh: DecodeShape, inp: dict):
        import torch
        import backward_gpt_block_amd as bl
        self.sh = sh
        self.cfg = bl.DecodeConfig(B=sh.B, C=sh.C, H=sh.H, F=sh.F, S_max=sh.S_max, eps=sh.eps,
                                   rope_base=sh.rope_base, window=sh.window, n_kv_head=sh.n_kv_head)
        self.w = [to_dev(inp[k], "bf16") for k in WNAMES]
        self.kc = to_dev(inp["k_cache"], "bf16")
        self.vc = to_dev(inp["v_cache"], "bf16")
        self.scratch = torch.empty(bl.decode_scratch_bytes(self.cfg), dtype=torch.uint8, device="cuda:0")

    def step(self, x_np, lens_np, in_place=False):
        import torch
        import backward_gpt_block_amd as bl
        x = to_dev(x_np, "bf16")
        lens = torch.from_numpy(np.asarray(lens_np, dtype=np.int32)).to("cuda:0")
        y = x if in_place else poison_(torch.empty_like(x))
        poison_(self.scratch)
        bl.decode_step(self.cfg, x, *self.w, self.kc, self.vc, lens, y, self.scratch)
        torch.cuda.synchronize()
        return to_np(y)

    def caches_bits(self):
        import torch
        return [t.view(torch.int16).cpu().numpy() for t in (self.kc, self.vc)]


def _bits(a: np.ndarray) -> np.ndarray:
    from blockinputs import to_storage
    return to_storage(a, "bf16").view(np.int16)


def _check_step(sh, inp, g: GpuDecode, x, lens, before_bits, in_place=False):
    from oracle import block as ob
    y = g.step(x, lens, in_place=in_place)
    W = [inp[k] for k in WNAMES]
    y_ref, kc_ref, vc_ref = ob.decode_step(x, *W, inp["k_cache"], inp["v_cache"], lens, H=sh.H, eps=sh.eps,
                                           rope_base=sh.rope_base, window=sh.window or None,
                                           n_kv_head=sh.n_kv_head or None)
    assert np.all(np.isfinite(y)), "y not finite (unwritten or NaN)"
    e = rel_err(y, y_ref)
    em = max_err(y, y_ref)
    er = float(np.max(row_errs(y, y_ref)))
    kb, vb = g.caches_bits()
    bidx = np.arange(sh.B)
    from blockinputs import from_storage
    k_new = from_storage(kb[bidx, :, lens, :].view(np.uint16), "bf16")
    v_new = from_storage(vb[bidx, :, lens, :].view(np.uint16), "bf16")
    ek = rel_err(k_new, kc_ref[bidx, :, lens, :])
    ev = rel_err(v_new, vc_ref[bidx, :, lens, :])
    ekm, evm = max_err(k_new, kc_ref[bidx, :, lens, :]), max_err(v_new, vc_ref[bidx, :, lens, :])
    print(f"  y={e:.2e} (max-ratio {em:.2e}, worst row {er:.2e}) k_slot={ek:.2e}/{ekm:.2e} "
          f"v_slot={ev:.2e}/{evm:.2e}", flush=True)
    tol = TOL["bf16"]
    assert e <= tol and ek <= tol and ev <= tol, (e, ek, ev)
    assert em <= tol and ekm <= tol and evm <= tol, (em, ekm, evm)
    assert er <= ROW_FACTOR * tol, er
    mask = np.ones(kb.shape[:3], dtype=bool)
    mask[bidx, :, lens] = False
    for got, want in zip((kb, vb), before_bits):
        assert np.array_equal(got[mask], want[mask]), "a slot other than cache_len[b] changed"
    # the oracle's caches become the next step's input
    inp["k_cache"], inp["v_cache"] = kc_ref, vc_ref
    return y, (kb, vb)


def _decode_case(sh: DecodeShape, lens=None, seed=0, steps=1, in_place=False, **kw):
    note(f"decode B={sh.B} C={sh.C} S_max={sh.S_max} lens={'given' if lens is not None else kw} steps={steps}")
    inp = make_decode_inputs(sh, seed=seed, **kw)
    if lens is not None:
        inp["cache_len"] = np.asarray(lens, dtype=np.int32)
    g = GpuDecode(sh, inp)
    bits = [_bits(inp["k_cache"]), _bits(inp["v_cache"])]
    lens = inp["cache_len"].copy()
    rng = np.random.default_rng(seed + 100)
    x = inp["x"]
    for t in range(steps):
        _, bits = _check_step(sh, inp, g, x, lens, bits, in_place=in_place)
        lens = np.minimum(lens + 1, sh.S_max - 1)
        from blockinputs import round_to
        x = round_to(rng.standard_normal(x.shape), "bf16")


def test_decode_ragged_edges():
    # position 0 (attends only to itself), S_max - 1, a split boundary (256)
    sh = DecodeShape(B=4, C=256, H=2, F=1024, S_max=300)
    _decode_case(sh, lens=[0, 150, 299, 256])


def test_decode_ragged_random_three_splits():
    _decode_case(DecodeShape(B=5, C=384, H=3, F=1536, S_max=777), ragged=True, ragged_lo=0)


def test_decode_more_rows_than_a_tile():
    _decode_case(DecodeShape(B=70, C=256, H=2, F=1024, S_max=40), ragged=True, ragged_lo=0)


def test_decode_two_chained_steps():
    _decode_case(DecodeShape(B=3, C=256, H=2, F=1024, S_max=520), lens=[5, 255, 400], steps=2)


def test_decode_in_place():
    _decode_case(DecodeShape(B=2, C=256, H=2, F=1024, S_max=64), lens=[10, 63], in_place=True)


def test_decode_d20_uniform_2048():
    _decode_case(DECODE_WORKLOADS["d20_decode"], cache_len=2048)


def test_decode_d20_ragged_128_2048():
    _decode_case(DECODE_WORKLOADS["d20_decode"], ragged=True, ragged_lo=128, ragged_hi=2048)


def test_decode_window_edges():
    # window W = 100: lengths below, at and past W, and windows that start
    # inside a later 256-key split
    sh = DecodeShape(B=6, C=256, H=2, F=1024, S_max=600, window=100)
    _decode_case(sh, lens=[0, 50, 99, 100, 299, 599])


def test_decode_window_two_chained_steps():
    _decode_case(DecodeShape(B=3, C=256, H=2, F=1024, S_max=520, window=257), lens=[5, 256, 400], steps=2)


def test_decode_d20_window_512_ragged():
    sh = DECODE_WORKLOADS["d20_decode"]
    sh = DecodeShape(B=sh.B, C=sh.C, H=sh.H, F=sh.F, S_max=sh.S_max, window=512)
    _decode_case(sh, ragged=True, ragged_lo=128, ragged_hi=2048)


def test_decode_gqa_ragged():
    # four query heads on one key/value head; then two groups of two
    _decode_case(DecodeShape(B=5, C=512, H=4, F=2048, S_max=600, n_kv_head=1), lens=[0, 1, 255, 256, 599])
    _decode_case(DecodeShape(B=4, C=512, H=4, F=2048, S_max=520, n_kv_head=2), ragged=True, ragged_lo=0)


def test_decode_gqa_window_two_chained_steps():
    _decode_case(DecodeShape(B=3, C=768, H=6, F=3072, S_max=520, window=200, n_kv_head=3), lens=[5, 256, 400],
                 steps=2)


def test_decode_d20_gqa_ragged_128_2048():
    _decode_case(DECODE_WORKLOADS["d20_decode_gqa"], ragged=True, ragged_lo=128, ragged_hi=2048)


def test_decode_out_of_range_lengths_reported():
    # lengths outside [0, S_max - 1] are errors of their sequences: no cache
    # write, a NaN row of y, counted in the status word; the other sequences
    # are computed as usual
    import torch
    import backward_gpt_block_amd as bl
    from oracle import block as ob
    sh = DecodeShape(B=4, C=256, H=2, F=1024, S_max=64)
    note("decode out-of-range lengths")
    inp = make_decode_inputs(sh, seed=12)
    lens = np.array([5, -1, 64, 63], dtype=np.int32)
    g = GpuDecode(sh, inp)
    before = [t.clone() for t in (g.kc, g.vc)]
    x = to_dev(inp["x"], "bf16")
    y = poison_(torch.empty_like(x))
    status = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
    bl.decode_step(g.cfg, x, *g.w, g.kc, g.vc, torch.from_numpy(lens).to("cuda:0"), y, g.scratch, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 2
    yn = to_np(y)
    assert np.all(np.isnan(yn[[1, 2]]))
    for t, t0 in zip((g.kc, g.vc), before):
        assert torch.equal(t[[1, 2]], t0[[1, 2]]), "a sequence with an invalid length changed its cache"
    ok = [0, 3]
    W = [inp[k] for k in WNAMES]
    y_ref, _, _ = ob.decode_step(inp["x"][ok], *W, inp["k_cache"][ok], inp["v_cache"][ok], lens[ok], H=sh.H,
                                 eps=sh.eps, rope_base=sh.rope_base)
    assert rel_err(yn[ok], y_ref) <= TOL["bf16"]
    # a valid step afterwards resets the word
    bl.decode_step(g.cfg, x, *g.w, g.kc, g.vc, torch.from_numpy(np.array([1, 2, 3, 4], dtype=np.int32)).to("cuda:0"),
                   y, g.scratch, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
