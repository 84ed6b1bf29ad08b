"""GPU parity of block_fwd + block_bwd (through the C ABI) against the CPU
float64 oracle, on seeded inputs, plus invariants the method fixes
(causality, T = 1, determinism, accumulation).

Gate per output tensor (y, dx, dW_qkv, dW_o, dW_fc, dW_proj): relative
Frobenius error and max|err|/max|ref| <= 1e-4 for float32 and <= 2e-2 for
bfloat16 operands, and every row of y and dx within 5x that of its own norm;
every output buffer starts as NaN, so an unwritten element fails."""
import numpy as np
import pytest

from blockinputs import WORKLOADS, BlockShape, make_block_inputs

from gpu_util import TOL, GpuBlock, check_forward_rows, compare, note, oracle_step, to_dev

pytestmark = pytest.mark.gpu


def _run(sh: BlockShape, seed=0):
    inp = make_block_inputs(sh, seed=seed)
    g = GpuBlock(sh, inp)
    g.fwd()
    g.bwd()
    return g, inp


def _parity(sh: BlockShape, seed=0):
    note(f"parity B={sh.B} T={sh.T} C={sh.C} H={sh.H} dtype={sh.dtype} seed={seed}")
    g, inp = _run(sh, seed)
    return compare(g.results(), oracle_step(sh, inp), TOL[sh.dtype])


def test_d6_f32_full_workload():
    _parity(WORKLOADS["d6_f32"])


@pytest.mark.parametrize("B,T,C", [
    (2, 300, 256),    # two query tiles of 128 and a ragged tail of 44
    (1, 77, 384),     # one partial tile
    (3, 1, 256),      # T = 1
    (1, 520, 768),    # d12 width, ragged
    (2, 192, 384),    # token count a multiple of 64 (weight gradients on the eight-wave body), ragged width
    (1, 4096, 256),   # the longest sequence whose dS the dK/dV pass stores for the dQ pass
    (1, 4160, 256),   # past it: the dQ pass recomputes dS (causal), ragged last tiles
])
def test_bf16_ragged(B, T, C):
    _parity(BlockShape(B=B, T=T, C=C, H=C // 128, F=4 * C, dtype="bf16"))


@pytest.mark.parametrize("T", [1, 45, 130])
def test_f32_ragged(T):
    _parity(BlockShape(B=2, T=T, C=256, H=2, F=1024, dtype="f32"), seed=3)


def _sampled_full(name, keep, fwd_seqs=None):
    """Full-size workload; the upstream gradient is zero outside the sampled
    sequences, so every gradient (dx and dW) comes from them alone and the
    oracle only needs those sequences.  The forward output y of the other
    sequences (all of them, or `fwd_seqs`) is compared with the oracle's
    forward, one sequence at a time."""
    sh = WORKLOADS[name]
    note(f"sampled full-size {name} keep={keep}")
    inp = make_block_inputs(sh, seed=0)
    mask = np.zeros(sh.B, dtype=bool)
    mask[list(keep)] = True
    inp["dy"] = np.where(mask[:, None, None], inp["dy"], 0.0)
    g = GpuBlock(sh, inp)
    g.fwd()
    g.bwd()
    res = g.results()
    ref = oracle_step(sh, inp, batch=list(keep))
    others = [b for b in range(sh.B) if b not in keep] if fwd_seqs is None else list(fwd_seqs)
    check_forward_rows(res["y"], sh, inp, others, TOL[sh.dtype])
    res["y"] = res["y"][list(keep)]
    res["dx"] = res["dx"][list(keep)]
    return compare(res, ref, TOL[sh.dtype])


def test_d12_full_size_sampled():
    _sampled_full("d12_bf16", (0, 7))


def test_d20_full_size_sampled():
    _sampled_full("d20_bf16", (0, 31))


@pytest.mark.parametrize("B,T,C,W", [
    (2, 300, 256, 1),       # each token attends to itself only
    (2, 300, 256, 64),      # window of one key tile
    (2, 300, 256, 100),     # window edge inside tiles, ragged tail
    (1, 520, 384, 130),     # window crossing query-tile and workgroup boundaries
    (1, 700, 256, 257),     # just over a 256-query workgroup
    (2, 192, 256, 300),     # window >= T: the causal path
])
def test_bf16_window(B, T, C, W):
    _parity(BlockShape(B=B, T=T, C=C, H=C // 128, F=4 * C, dtype="bf16", window=W), seed=4)


@pytest.mark.parametrize("T,W", [(130, 45), (200, 1), (97, 64)])
def test_f32_window(T, W):
    _parity(BlockShape(B=2, T=T, C=256, H=2, F=1024, dtype="f32", window=W), seed=6)


def test_d20_window_full_size_sampled():
    _sampled_full("d20_bf16_swa", (0, 31), fwd_seqs=(1, 9, 17, 30))


def test_window_locality_bitwise():
    # with a window W, changing input row t changes output rows t .. t+W-1
    # only; every other row is bitwise the same
    W = 70
    sh = BlockShape(B=1, T=400, C=256, H=2, F=1024, dtype="bf16", window=W)
    note("window locality")
    inp = make_block_inputs(sh, seed=8)
    g = GpuBlock(sh, inp)
    g.fwd()
    y0 = g.results()["y"].copy()
    t = 150
    x2 = inp["x"].copy()
    x2[:, t] = np.random.default_rng(9).standard_normal(x2[:, t].shape)
    g.fwd(x=to_dev(x2, "bf16"))
    y1 = g.results()["y"]
    changed = np.nonzero(np.any(y0[0] != y1[0], axis=-1))[0]
    assert changed.min() == t and changed.max() <= t + W - 1, changed
    assert np.array_equal(y0[:, :t], y1[:, :t]) and np.array_equal(y0[:, t + W:], y1[:, t + W:])


def test_causality_bitwise():
    sh = BlockShape(B=2, T=200, C=256, H=2, F=1024, dtype="bf16")
    note("causality")
    inp = make_block_inputs(sh, seed=5)
    g = GpuBlock(sh, inp)
    g.fwd()
    y0 = g.results()["y"].copy()
    t = 97
    x2 = inp["x"].copy()
    x2[:, t + 1:] = np.random.default_rng(7).standard_normal(x2[:, t + 1:].shape)
    g.fwd(x=to_dev(x2, "bf16"))
    y1 = g.results()["y"]
    assert np.array_equal(y0[:, :t + 1], y1[:, :t + 1])
    assert not np.array_equal(y0[:, t + 1:], y1[:, t + 1:])


def test_determinism_and_accumulate():
    sh = BlockShape(B=2, T=160, C=256, H=2, F=1024, dtype="bf16")
    note("determinism / accumulate")
    g, inp = _run(sh, seed=2)
    r1 = g.results()
    g.fwd()
    g.bwd()
    r2 = g.results()
    for k in r1:
        assert np.array_equal(r1[k], r2[k]), k
    g.bwd(accumulate=1)
    r3 = g.results()
    for k in ("dw_qkv", "dw_o", "dw_fc", "dw_proj"):
        assert np.allclose(r3[k], 2 * r1[k], rtol=1e-6, atol=1e-6), k


def test_t1_value_path_gradients_vanish_for_q_k():
    sh = BlockShape(B=4, T=1, C=256, H=2, F=1024, dtype="f32")
    note("T=1 value path")
    g, inp = _run(sh, seed=4)
    r = g.results()
    C = sh.C
    assert np.max(np.abs(r["dw_qkv"][:2 * C])) <= 1e-5 * np.max(np.abs(r["dw_qkv"][2 * C:]))


@pytest.mark.parametrize("B,T,C,G,dtype,W", [
    (2, 300, 512, 1, "bf16", 0),     # one key/value head shared by four query heads
    (1, 257, 512, 2, "bf16", 0),     # two groups of two, ragged tail of one
    (2, 130, 768, 3, "bf16", 0),     # six heads in three groups
    (1, 300, 512, 2, "bf16", 100),   # grouped heads under a sliding window
    (2, 97, 512, 2, "f32", 0),
    (2, 130, 512, 1, "f32", 45),
])
def test_gqa(B, T, C, G, dtype, W):
    _parity(BlockShape(B=B, T=T, C=C, H=C // 128, F=4 * C, dtype=dtype, window=W, n_kv_head=G), seed=8)


@pytest.mark.parametrize("B,T,C,G,W", [
    # dK/dV 2 x 160 x 2 = 640 units, dQ 640, forward 320: workgroups walk
    # several units; the second key tile of each sequence holds 2 keys, so
    # three of its four waves have no rows at all
    (160, 130, 256, 0, 0),
    # grouped heads under a window: 384 dK/dV units of 2 query heads each,
    # 768 dQ units
    (96, 200, 512, 2, 100),
])
def test_attention_units_beyond_one_per_cu(B, T, C, G, W):
    # the backward attention grids hold one workgroup per CU (256 on MI355X);
    # these shapes need more units than that, at sizes compared in full
    _parity(BlockShape(B=B, T=T, C=C, H=C // 128, F=4 * C, dtype="bf16", window=W, n_kv_head=G), seed=11)


def test_gqa_g_equals_h_matches_mha_bitwise():
    # n_kv_head = H takes the same kernels over the same layout as MHA
    sh = BlockShape(B=2, T=200, C=256, H=2, F=1024, dtype="bf16")
    inp = make_block_inputs(sh, seed=9)
    outs = []
    for G in (0, 2):
        s2 = BlockShape(B=2, T=200, C=256, H=2, F=1024, dtype="bf16", n_kv_head=G)
        g = GpuBlock(s2, inp)
        g.fwd()
        g.bwd()
        outs.append(g.results())
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_d20_gqa_full_size_sampled():
    _sampled_full("d20_bf16_gqa", (0, 31), fwd_seqs=(2, 13, 22, 29))
