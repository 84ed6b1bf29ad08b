"""Pins of the oracle's E4M3 quantiser: the code table against the format's
defining constants, round-to-nearest-even on midpoints, saturation, and a
cross-check of in-range rounding against torch's float8_e4m3fn cast.  CPU."""
import numpy as np
import pytest

from oracle import fp8


def test_code_table_landmarks():
    t = fp8.e4m3_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0 ** -9                             # smallest subnormal
    assert t[0x08] == 2.0 ** -6                             # smallest normal
    assert t[0x07] == 7 * 2.0 ** -9                          # largest subnormal
    assert t[0x38] == 1.0                                   # exponent field 7 = bias
    fin = t[:0x7F]
    assert np.all(np.diff(fin) > 0)                         # codes 0..126 increase
    assert np.array_equal(t[0x80:0xFF], -fin)


def test_encode_roundtrip_all_finite_codes():
    t = fp8.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])])
    assert np.array_equal(fp8.e4m3_encode(t[codes]), codes.astype(np.uint8))


def test_midpoints_round_to_even_code_and_saturate():
    t = fp8.e4m3_table()
    for c in range(0, 0x7E):
        mid = 0.5 * (t[c] + t[c + 1])
        want = c if c % 2 == 0 else c + 1
        assert fp8.e4m3_encode(np.array([mid]))[0] == want, c
        assert fp8.e4m3_encode(np.array([-mid]))[0] == (want | 0x80), c
    assert fp8.e4m3_encode(np.array([1e6, -500.0]))[0] == 0x7E
    assert fp8.e4m3_encode(np.array([-1e6]))[0] == 0xFE


def test_in_range_rounding_matches_torch_cast():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 120.0)])
    x = x[np.abs(x) <= 440].astype(np.float32)
    ours = fp8.e4m3_encode(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_round_bf16_ties_and_torch_cast():
    torch = pytest.importorskip("torch")
    # ties go to the even 8-bit significand; the sign and zero are kept
    assert fp8.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert fp8.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert fp8.round_bf16(np.array([-(1 + 2.0 ** -8 + 2.0 ** -20)]))[0] == -(1 + 2.0 ** -7)
    assert np.signbit(fp8.round_bf16(np.array([-0.0]))[0])
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(fp8.round_bf16(x), want)


def test_quantize_tensor_scale_and_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(4096) * 3
    codes, s = fp8.quantize_tensor(x)
    assert s == np.float32(np.max(np.abs(x.astype(np.float32)))) / np.float32(448)
    deq = fp8.e4m3_values(codes) * np.float64(s)
    # relative error of a 3-bit-mantissa rounding is at most 2^-4 for normals
    big = np.abs(x) > 2.0 ** -6 * s * 2
    assert np.all(np.abs(deq[big] - x[big]) <= np.abs(x[big]) * 2.0 ** -4 + 1e-12)
    z, s0 = fp8.quantize_tensor(np.array([0.0, -0.0, 0.0]))
    assert s0 == 1.0 and list(z) == [0x00, 0x80, 0x00]
    # a given amax overrides the slice's own maximum
    c2, s2 = fp8.quantize_tensor(np.array([1.0, -2.0]), amax=448.0)
    assert s2 == 1.0 and list(fp8.e4m3_values(c2)) == [1.0, -2.0]


def _small_block(seed, B=2, T=9, C=256):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, C))
    W = [rng.standard_normal(s) * 0.05 for s in ((3 * C, C), (C, C), (4 * C, C), (C, 4 * C))]
    dy = rng.standard_normal((B, T, C))
    return x, W, dy


def _exact(x, W, dy, H):
    from oracle import block as ob
    c = ob.block_fwd(x, *W, H=H)
    ref = ob.block_bwd(dy, c, *W, H=H)
    ref["y"] = c.y
    return ref


def test_fp8_block_without_rounding_is_the_exact_block():
    # with the operand rounding replaced by the identity, the fp8 oracle must
    # be the unquantised block (pinned by finite differences and autograd)
    from oracle import fp8_block
    x, W, dy = _small_block(3)
    ident = lambda t, amax=None: np.asarray(t, dtype=np.float64)
    got = fp8_block.block_fwd_bwd(x, *W, dy, H=2, quant=ident, store=ident)
    ref = _exact(x, W, dy, 2)
    for k in ref:
        assert np.allclose(got[k], ref[k], rtol=1e-12, atol=1e-12), k


def test_fp8_block_rounds_every_gemm_operand():
    # counts the roundings: 4 weights, 4 forward activations, 4 backward
    # gradients; each a distinct tensor of the expected shape
    from oracle import fp8_block
    x, W, dy = _small_block(4, B=1, T=5)
    seen = []

    def rec(t, amax=None):
        seen.append(np.shape(t))
        return np.asarray(t, dtype=np.float64)

    fp8_block.block_fwd_bwd(x, *W, dy, H=2, quant=rec)
    C = x.shape[-1]
    act = (1, 5, C)
    assert sorted(seen) == sorted([(3 * C, C), (C, C), (4 * C, C), (C, 4 * C),
                                   act, act, act, (1, 5, 4 * C),            # h1, o, h2, a
                                   act, (1, 5, 4 * C), act, (1, 5, 3 * C)])  # dy, du, dy1, dqkv


def test_fp8_block_rounds_every_stored_intermediate():
    # the bf16 pipeline's stored intermediates, each rounded once: h1, q, k,
    # v (per head), o, y1, h2, a; du, dh2, dy1, dO, dqkv, dh1
    from oracle import fp8_block
    x, W, dy = _small_block(6, B=1, T=5)
    seen = []

    def rec(t):
        seen.append(np.shape(t))
        return np.asarray(t, dtype=np.float64)

    fp8_block.block_fwd_bwd(x, *W, dy, H=2, store=rec)
    C = x.shape[-1]
    act, head = (1, 5, C), (1, 2, 5, C // 2)
    assert sorted(seen) == sorted([act, head, head, head, act, act, act, (1, 5, 4 * C),     # h1 q k v o y1 h2 a
                                   (1, 5, 4 * C), act, act, act, (1, 5, 3 * C), act])      # du dh2 dy1 dO dqkv dh1


def test_fp8_block_stored_rounding_moves_codes_downstream():
    # one bf16 rounding of a stored intermediate moves E4M3 codes downstream:
    # with and without the store rounding the weight gradients differ by far
    # more than a bf16 rounding (2^-9), and y by a few percent at most
    from oracle import fp8_block
    x, W, dy = _small_block(7, B=2, T=64)
    ident = lambda t: np.asarray(t, dtype=np.float64)
    a = fp8_block.block_fwd_bwd(x, *W, dy, H=2)
    b = fp8_block.block_fwd_bwd(x, *W, dy, H=2, store=ident)
    rel = {k: np.linalg.norm(a[k] - b[k]) / np.linalg.norm(b[k]) for k in a}
    assert rel["y"] < 5e-2, rel
    assert min(rel[k] for k in ("dw_qkv", "dw_o", "dw_fc", "dw_proj")) > 4 * 2.0 ** -9, rel


def test_fp8_emulating_block_tracks_exact_block():
    # quantising the GEMM operands perturbs each output by a few percent at
    # most (3-bit mantissas, per-tensor scales), and by a visible amount
    from oracle import fp8_block
    x, W, dy = _small_block(3)
    emu = fp8_block.block_fwd_bwd(x, *W, dy, H=2)
    ref = _exact(x, W, dy, 2)
    for k in emu:
        err = np.linalg.norm(emu[k] - ref[k]) / np.linalg.norm(ref[k])
        assert 1e-4 < err < 0.1, (k, err)


def test_fp8_block_selected_sequences_match_whole_batch():
    # with dy zero outside the selection, the selection's outputs and the
    # weight gradients equal those of the whole batch: the forward scales come
    # from the whole batch, the backward tensors vanish outside the selection
    from oracle import fp8_block
    x, W, dy = _small_block(5, B=3, T=7)
    dy[1] = 0.0
    whole = fp8_block.block_fwd_bwd(x, *W, dy, H=2)
    sub = fp8_block.block_fwd_bwd(x, *W, dy, H=2, batch=[0, 2])
    for k in ("y", "dx"):
        assert np.allclose(sub[k], whole[k][[0, 2]], rtol=0, atol=1e-12), k
    for k in ("dw_qkv", "dw_o", "dw_fc", "dw_proj"):
        assert np.allclose(sub[k], whole[k], rtol=1e-12, atol=1e-12), k
    with pytest.raises(ValueError):
        fp8_block.block_fwd_bwd(x, *W, dy, H=2, batch=[0])
