"""GPU checks of the fp8 (E4M3) mode of the linear layers.

- the quantiser (block_fp8_quantize) matches the oracle's codes bit for bit
  and its amax exactly (byte results: bit-exact bar);
- the block with fp8 GEMMs matches the float64 oracle of the fp8 block (the
  same GEMM operands rounded to E4M3, code choices taken on bf16 values as
  the kernels take them, everything else exact) within 6e-2 relative
  Frobenius error per output, on ragged and full-size shapes;
- the GPU's distance from the UNQUANTISED block is no larger than the fp8
  oracle's own (the recipe's rounding error, 0.05-0.10 for the weight
  gradients here), within 15%: the kernels add no error of their own.

The gates of gpu_util.compare apply to every output: Frobenius error <= 6e-2
against the fp8 oracle, max|err|/max|ref| <= 6e-2 for y and dx, each row of
y and dx within 5x; the weight gradients' max|err|/max|ref| <= 6e-2 at the
d26 workload and <= 0.12 at the small shapes.  A weight-gradient element
is a sum over the tokens of products of E4M3 codes, and the attention
kernels' own bf16 roundings (of P and dS, which the oracle does not take)
move a share of the downstream codes to a neighbouring code: at a few dozen
tokens the largest element error sits at about twice the Frobenius error.  Against
the unquantised block the recipe itself (per-tensor E4M3 on all three GEMMs
of every linear layer) does not reach 6e-2 for the deepest weight gradients
at the d26 width; those distances are printed, and held to the fp8 oracle's
own distance by the ratio check."""
import numpy as np
import pytest

from blockinputs import WORKLOADS, BlockShape, make_block_inputs, round_to

from gpu_util import TOL, GpuBlock, compare, max_err, note, oracle_step, poison_, rel_err, to_dev

pytestmark = pytest.mark.gpu


def test_quantizer_bit_exact():
    import torch
    import backward_gpt_block_amd as bl
    from oracle import fp8
    rng = np.random.default_rng(21)
    for scale, n in ((1.0, 1 << 20), (1e-3, 4096), (300.0, 65536), (0.0, 1024)):
        note(f"fp8 quantizer scale={scale} n={n}")
        x = round_to(rng.standard_normal(n) * scale, "bf16")
        if scale == 1.0:
            x[:8] = [0.0, -0.0, 1e-30, -1e-30, 2.0 ** -20, 448.0, -448.0, 3.0]
            x = round_to(x, "bf16")
        xd = to_dev(x, "bf16")
        codes = poison_(torch.empty(n, dtype=torch.uint8, device="cuda:0"))
        amax = poison_(torch.empty(1, dtype=torch.int32, device="cuda:0"))
        bl.block_fp8_quantize(xd, n, codes, amax)
        torch.cuda.synchronize()
        want, s = fp8.quantize_tensor(x)
        got = codes.cpu().numpy()
        amax_got = np.array([amax.cpu().item()], dtype=np.int32).view(np.float32)[0]
        assert amax_got == np.float32(np.max(np.abs(x))), (amax_got, np.max(np.abs(x)))
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{bad.size} codes differ, e.g. x={x[bad[:5]]} got={got[bad[:5]]} want={want[bad[:5]]}"


ACCURACY_RATIO = 1.15


def _fp8_parity(sh: BlockShape, seed=0, keep=None, dw_max_factor=2.0):
    from oracle import fp8_block
    note(f"fp8 block B={sh.B} T={sh.T} C={sh.C} keep={keep} seed={seed}")
    inp = make_block_inputs(sh, seed=seed)
    if keep is not None:
        mask = np.zeros(sh.B, dtype=bool)
        mask[list(keep)] = True
        inp["dy"] = np.where(mask[:, None, None], inp["dy"], 0.0)
    g = GpuBlock(sh, inp)
    g.fwd()
    g.bwd()
    res = g.results()
    del g
    if keep is not None:
        res["y"], res["dx"] = res["y"][list(keep)], res["dx"][list(keep)]
    emu = fp8_block.block_fwd_bwd(inp["x"], inp["w_qkv"], inp["w_o"], inp["w_fc"], inp["w_proj"], inp["dy"],
                                  H=sh.H, eps=sh.eps, rope_base=sh.rope_base,
                                  batch=None if keep is None else list(keep), log=note, window=sh.window or None,
                                  n_kv_head=sh.n_kv_head or None)
    errs = compare(res, emu, TOL["fp8"], keys=list(emu),
                   max_tol={k: dw_max_factor * TOL["fp8"] for k in ("dw_qkv", "dw_o", "dw_fc", "dw_proj")})
    ref = oracle_step(sh, inp, batch=None if keep is None else list(keep))
    gpu_acc = {k: rel_err(res[k], ref[k]) for k in ref}
    emu_acc = {k: rel_err(emu[k], ref[k]) for k in ref}
    print("  distance from the unquantised block, GPU / fp8 oracle: "
          + ", ".join(f"{k}={gpu_acc[k]:.2e}/{emu_acc[k]:.2e}" for k in ref), flush=True)
    print("  max|err|/max|ref| from the unquantised block, GPU: "
          + ", ".join(f"{k}={max_err(res[k], ref[k]):.2e}" for k in ref), flush=True)
    for k in ref:
        assert gpu_acc[k] <= ACCURACY_RATIO * emu_acc[k] + 1e-3, (k, gpu_acc[k], emu_acc[k])
    return errs


@pytest.mark.parametrize("B,T,C", [(2, 256, 256), (1, 77, 384), (3, 130, 256)])
def test_fp8_block_ragged(B, T, C):
    _fp8_parity(BlockShape(B=B, T=T, C=C, H=C // 128, F=4 * C, dtype="bf16", gemm="fp8"))


def test_fp8_block_window():
    _fp8_parity(BlockShape(B=2, T=300, C=256, H=2, F=1024, dtype="bf16", gemm="fp8", window=100))


@pytest.mark.timeout(900)
def test_d26_fp8_full_size_sampled():
    # the oracle's forward pass over all 16 sequences (for the per-tensor
    # scales) takes a minute or two of host time; at this size every gate is
    # the stated 6e-2, the weight gradients' max ratio included
    _fp8_parity(WORKLOADS["d26_fp8"], keep=(0, 15), dw_max_factor=1.0)


def test_fp8_block_gqa():
    _fp8_parity(BlockShape(B=2, T=300, C=512, H=4, F=2048, dtype="bf16", gemm="fp8", n_kv_head=1))


@pytest.mark.parametrize("rows,cols,ldt", [
    (77, 256, 128),      # ragged rows, padding columns 77..127 of the transposed copy
    (300, 384, 320),     # a partial last 128-row tile (its second half past ldt is not written)
    (1000, 1664, 1024),  # d26 width
    (130, 192, 192),     # width not a multiple of 128: the 64 x 64 kernel
])
def test_quantizer_2d_transposed_bit_exact(rows, cols, ldt):
    # row-major and transposed codes of a matrix, as the weight-gradient
    # GEMMs of the fp8 mode read them, against the oracle's quantiser
    import torch
    import backward_gpt_block_amd as bl
    from oracle import fp8
    note(f"fp8 2-D quantizer rows={rows} cols={cols} ldt={ldt}")
    rng = np.random.default_rng(rows + cols)
    x = round_to(rng.standard_normal((rows, cols)) * 3.0, "bf16")
    x[0, :4] = [0.0, -0.0, 448.0, -1e-30]
    x = round_to(x, "bf16")
    xd = to_dev(x, "bf16")
    codes = torch.full((rows, cols), 0x55, dtype=torch.uint8, device="cuda:0")
    codes_t = torch.full((cols, ldt), 0x55, dtype=torch.uint8, device="cuda:0")
    amax = poison_(torch.empty(1, dtype=torch.int32, device="cuda:0"))
    bl.block_fp8_quantize_2d(xd, rows, cols, codes, codes_t, ldt, amax)
    torch.cuda.synchronize()
    want, _ = fp8.quantize_tensor(x)
    want = want.reshape(rows, cols)
    got, got_t = codes.cpu().numpy(), codes_t.cpu().numpy()
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} row-major codes differ"
    assert np.array_equal(got_t[:, :rows], want.T), f"{np.count_nonzero(got_t[:, :rows] != want.T)} transposed codes differ"
    assert not np.any(got_t[:, rows:]), "padding columns of the transposed copy are not zero"
    amax_got = np.array([amax.cpu().item()], dtype=np.int32).view(np.float32)[0]
    assert amax_got == np.float32(np.max(np.abs(x)))
