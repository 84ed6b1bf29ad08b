"""Host-side checks of the C ABI (no GPU needed): the built library loads and
exports every function include/blk.h declares; size queries; every argument
error is reported before any HIP call (fake, never-dereferenced addresses)."""
import os
import re

import pytest

import backward_gpt_block_amd as bl
from blockinputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bl.library_path()):
        from backward_gpt_block_amd.build import build
        build()
    return bl.library()


def _header_functions():
    text = open(os.path.join(ROOT, "include", "blk.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(lib):
    names = _header_functions()
    assert {"block_fwd", "block_bwd", "decode_step", "block_saved_bytes", "block_scratch_bytes",
            "decode_scratch_bytes", "block_strerror", "head_loss_fwd", "head_loss_bwd",
            "head_scratch_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def _cfg(**kw):
    sh = WORKLOADS["d20_bf16"]
    d = dict(B=sh.B, T=sh.T, C=sh.C, H=sh.H, F=sh.F)
    d.update(kw)
    return bl.BlockConfig(**d)


def test_size_queries(lib):
    c = _cfg()
    saved = bl.block_saved_bytes(c)
    N, C, F = 32 * 2048, 1280, 5120
    # saved activations: h1, o, h2 (N*C), qkv (3NC), a (N*F) in bf16, plus small fp32 vectors
    assert saved >= 2 * (6 * N * C + N * F)
    assert saved < 2 * (6 * N * C + N * F) * 1.05
    assert bl.block_scratch_bytes(c) >= saved
    f32 = _cfg(dtype=bl.BLK_F32)
    assert bl.block_saved_bytes(f32) > 1.9 * saved
    for bad in (_cfg(D=64), _cfg(C=1000), _cfg(F=4000), _cfg(B=0), _cfg(T=0), _cfg(dtype=7),
                _cfg(n_kv_head=-2), _cfg(n_kv_head=4)):
        assert bl.block_saved_bytes(bad) == 0
        assert bl.block_scratch_bytes(bad) == 0
    # grouped-query attention: the saved qkv rows narrow from 3C to C + 2*G*128
    g2 = _cfg(n_kv_head=2)
    assert saved - bl.block_saved_bytes(g2) >= 2 * N * 2 * (10 - 2) * 128
    assert bl.block_saved_bytes(_cfg(n_kv_head=10)) == saved


A = 0x10000     # aligned fake addresses: the calls below must fail before any use
MIS = 0x10008


def _fwd(cfg, **kw):
    args = dict(x=A, w_qkv=A + 0x100, w_o=A + 0x200, w_fc=A + 0x300, w_proj=A + 0x400, y=A + 0x500,
                saved=A + 0x600, scratch=A + 0x700, saved_bytes=1 << 40, scratch_bytes=1 << 40)
    args.update(kw)
    return bl.block_fwd(cfg, args.pop("x"), args.pop("w_qkv"), args.pop("w_o"), args.pop("w_fc"),
                        args.pop("w_proj"), args.pop("y"), args.pop("saved"), args.pop("scratch"),
                        raise_on_error=False, stream=0, **args)


def _bwd(cfg, **kw):
    args = dict(dy=A, x=A, w_qkv=A, w_o=A, w_fc=A, w_proj=A, saved=A, dx=A + 0x800, dw_qkv=A, dw_o=A, dw_fc=A,
                dw_proj=A, accumulate=0, scratch=A, saved_bytes=1 << 40, scratch_bytes=1 << 40)
    args.update(kw)
    pos = [args.pop(k) for k in ("dy", "x", "w_qkv", "w_o", "w_fc", "w_proj", "saved", "dx", "dw_qkv", "dw_o",
                                 "dw_fc", "dw_proj", "accumulate", "scratch")]
    return bl.block_bwd(cfg, *pos, raise_on_error=False, stream=0, **args)


def test_fwd_argument_errors(lib):
    c = _cfg()
    assert _fwd(_cfg(D=64)) == bl.binding.BLK_EINVAL
    assert _fwd(_cfg(C=1000)) == bl.binding.BLK_EINVAL
    assert _fwd(c, x=None) == bl.binding.BLK_EINVAL
    assert _fwd(c, w_proj=None) == bl.binding.BLK_EINVAL
    assert _fwd(c, y=A) == bl.binding.BLK_EINVAL          # y aliases x
    assert _fwd(c, w_o=MIS) == bl.binding.BLK_EALIGN
    assert _fwd(c, saved_bytes=10) == bl.binding.BLK_ENOSPC
    assert _fwd(c, saved=None, scratch_bytes=10) == bl.binding.BLK_ENOSPC
    assert _fwd(c, saved=None, scratch=None) == bl.binding.BLK_EINVAL
    assert _fwd(_cfg(gemm=bl.BLK_GEMM_FP8_E4M3, dtype=bl.BLK_F32)) == bl.binding.BLK_EUNSUPPORTED
    assert _fwd(_cfg(gemm=5)) == bl.binding.BLK_EINVAL
    assert _fwd(_cfg(eps=float("nan"))) == bl.binding.BLK_EINVAL
    assert _fwd(_cfg(window=-1)) == bl.binding.BLK_EINVAL
    assert _fwd(_cfg(n_kv_head=-1)) == bl.binding.BLK_EINVAL
    assert _fwd(_cfg(n_kv_head=3)) == bl.binding.BLK_EINVAL     # 10 query heads are not split in groups of 3


def test_four_wave_weight_gradient_operand_limit(lib):
    # weight gradients that run on the four-wave GEMM body (float32; bf16
    # token counts not a multiple of 64; E4M3 token counts not a multiple of
    # 128) address operands with 32-bit byte offsets: a [N, F] operand (or
    # the fp8 mode's transposed [F, N rounded up to 64] codes) of 4 GiB or
    # more is refused before any launch; the eight-wave body has no limit
    E = bl.binding
    f32 = lambda T: _cfg(B=1, T=T, dtype=bl.BLK_F32)
    assert bl.block_saved_bytes(f32(209715)) > 0                 # 209715 * 5120 * 4 < 2^32
    assert bl.block_saved_bytes(f32(209716)) == 0
    assert _fwd(f32(209716)) == E.BLK_EUNSUPPORTED
    assert _bwd(f32(209716)) == E.BLK_EUNSUPPORTED
    bf = lambda T: _cfg(B=1, T=T)
    assert bl.block_saved_bytes(bf(419430)) > 0                  # ragged, 419430 * 5120 * 2 < 2^32
    assert bl.block_saved_bytes(bf(419431)) == 0
    assert _fwd(bf(419431)) == E.BLK_EUNSUPPORTED
    assert bl.block_saved_bytes(bf(419456)) > 0                  # a multiple of 64: eight-wave body
    f8 = lambda T: _cfg(B=1, T=T, gemm=bl.BLK_GEMM_FP8_E4M3, n_kv_head=1)
    assert bl.block_saved_bytes(f8(838848)) > 0                  # 838848 * 5120 < 2^32
    assert bl.block_saved_bytes(f8(838850)) == 0                 # padded to 838912 tokens
    assert _bwd(f8(838850)) == E.BLK_EUNSUPPORTED
    assert bl.block_saved_bytes(f8(838912)) > 0                  # a multiple of 128: eight-wave body


def test_bwd_argument_errors(lib):
    c = _cfg()
    assert _bwd(c, saved=None) == bl.binding.BLK_EINVAL
    assert _bwd(c, dw_fc=None) == bl.binding.BLK_EINVAL
    assert _bwd(c, scratch=None) == bl.binding.BLK_EINVAL
    assert _bwd(c, accumulate=2) == bl.binding.BLK_EINVAL
    assert _bwd(c, dx=MIS) == bl.binding.BLK_EALIGN
    assert _bwd(c, scratch_bytes=100) == bl.binding.BLK_ENOSPC
    assert _bwd(c, saved_bytes=100) == bl.binding.BLK_ENOSPC
    assert _bwd(_cfg(H=0, C=0, F=0)) == bl.binding.BLK_EINVAL


def _dcfg(**kw):
    d = dict(B=64, C=1280, H=10, F=5120, S_max=2049)
    d.update(kw)
    return bl.DecodeConfig(**d)


def _dec(cfg, **kw):
    args = dict(x=A, w_qkv=A + 0x100, w_o=A + 0x200, w_fc=A + 0x300, w_proj=A + 0x400, k_cache=A + 0x500,
                v_cache=A + 0x600, cache_len=A + 0x700, y=A + 0x800, scratch=A + 0x900, scratch_bytes=1 << 40)
    args.update(kw)
    pos = [args.pop(k) for k in ("x", "w_qkv", "w_o", "w_fc", "w_proj", "k_cache", "v_cache", "cache_len", "y",
                                 "scratch")]
    return bl.decode_step(cfg, *pos, raise_on_error=False, stream=0, **args)


def test_decode_sizes_and_argument_errors(lib):
    c = _dcfg()
    need = bl.decode_scratch_bytes(c)
    # at least the activations h1, o, h2 (bf16), y1, q (fp32), a (bf16) and the split partials
    assert need >= 64 * (1280 * (2 * 3 + 4) + 1280 * 4 + 5120 * 2)
    assert need < 64 << 20
    for bad in (_dcfg(D=64), _dcfg(C=1000), _dcfg(F=100), _dcfg(B=0), _dcfg(S_max=0), _dcfg(dtype=7),
                _dcfg(window=-3), _dcfg(n_kv_head=-1), _dcfg(n_kv_head=4)):
        assert bl.decode_scratch_bytes(bad) == 0
        assert _dec(bad) == bl.binding.BLK_EINVAL
    assert _dec(_dcfg(dtype=bl.BLK_F32)) == bl.binding.BLK_EUNSUPPORTED
    assert _dec(_dcfg(C=4096, H=32, F=16384)) == bl.binding.BLK_EUNSUPPORTED
    assert _dec(c, x=None) == bl.binding.BLK_EINVAL
    assert _dec(c, cache_len=None) == bl.binding.BLK_EINVAL
    assert _dec(c, v_cache=A + 0x500) == bl.binding.BLK_EINVAL      # v_cache aliases k_cache
    assert _dec(c, w_fc=MIS) == bl.binding.BLK_EALIGN
    assert _dec(c, cache_len=A + 0x702) == bl.binding.BLK_EALIGN
    assert _dec(c, status=A + 0x906) == bl.binding.BLK_EALIGN
    assert _dec(c, scratch_bytes=need - 1) == bl.binding.BLK_ENOSPC


def test_fp8_quantize_2d_argument_errors(lib):
    q = bl.block_fp8_quantize_2d
    E = bl.binding
    args = dict(x=A, rows=300, cols=384, codes=A + 0x100, codes_t=A + 0x200, ldt=320, amax=A + 0x300)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return q(a["x"], a["rows"], a["cols"], a["codes"], a["codes_t"], a["ldt"], a["amax"], raise_on_error=False,
                 stream=0)

    for bad in (dict(x=None), dict(codes_t=None), dict(amax=None), dict(rows=0), dict(cols=100), dict(cols=0),
                dict(ldt=299), dict(ldt=330), dict(rows=1 << 31)):
        assert call(**bad) == E.BLK_EINVAL, bad
    assert call(x=MIS) == E.BLK_EALIGN
    assert call(codes=MIS) == E.BLK_EALIGN
    assert call(amax=A + 0x302) == E.BLK_EALIGN


def test_decode_noalloc_workspace_limit(lib):
    # the static workspace holds the d20 decode workload; a configuration that
    # needs more is refused before any launch, argument errors as decode_step
    E = bl.binding
    assert bl.decode_scratch_bytes(_dcfg()) <= E.BLK_NOALLOC_SCRATCH_BYTES
    big = _dcfg(B=1024, S_max=8192)
    assert bl.decode_scratch_bytes(big) > E.BLK_NOALLOC_SCRATCH_BYTES
    call = lambda cfg, **kw: bl.decode_step_noalloc(cfg, kw.get("x", A), A, A, A, A, A + 0x100, kw.get("v", A + 0x200),
                                                    A + 0x300, A + 0x400, stream=0, raise_on_error=False)
    assert call(big) == E.BLK_ELIMIT
    assert call(_dcfg(), x=None) == E.BLK_EINVAL
    assert call(_dcfg(), v=A + 0x100) == E.BLK_EINVAL
    assert call(_dcfg(dtype=bl.BLK_F32)) == E.BLK_EUNSUPPORTED


def test_strerror(lib):
    for code in range(7):
        assert isinstance(bl.block_strerror(code), str) and bl.block_strerror(code)
    assert "unknown" in bl.block_strerror(99)


def test_layer_window_pattern():
    # S layers: a window of a quarter of the context; L layers and the last
    # layer: the whole context (0)
    T = 2048
    assert [bl.layer_window(i, 8, T) for i in range(8)] == [512, 512, 512, 0, 512, 512, 512, 0]
    assert [bl.layer_window(i, 6, T) for i in range(6)] == [512, 512, 512, 0, 512, 0]
    assert [bl.layer_window(i, 4, T, "L") for i in range(4)] == [0, 0, 0, 0]
    assert [bl.layer_window(i, 5, 512, "SL") for i in range(5)] == [128, 0, 128, 0, 0]
    for bad in ("", "SX"):
        with pytest.raises(ValueError):
            bl.layer_window(0, 4, T, bad)
    with pytest.raises(ValueError):
        bl.layer_window(4, 4, T)


def _hcfg(**kw):
    d = dict(N=32 * 2048, C=1280, V=65536)
    d.update(kw)
    return bl.HeadConfig(**d)


def test_head_sizes_and_argument_errors(lib):
    c = _hcfg()
    need = bl.head_scratch_bytes(c)
    N, C, V = 32 * 2048, 1280, 65536
    # the backward holds the softmax gradient [N, V] in bf16, W^T and dh
    assert need >= 2 * N * V + 2 * C * V + 2 * N * C
    assert need < 2 * N * V * 1.1
    for bad in (_hcfg(V=1000), _hcfg(V=0), _hcfg(C=1000), _hcfg(N=0), _hcfg(dtype=7), _hcfg(eps=float("nan"))):
        assert bl.head_scratch_bytes(bad) == 0
    assert bl.head_scratch_bytes(_hcfg(dtype=bl.BLK_F32)) == 0
    E = bl.binding
    fwd = lambda cfg, **kw: bl.head_loss_fwd(cfg, kw.get("x", A), kw.get("w", A + 0x100), kw.get("t", A + 0x200),
                                             kw.get("loss", A + 0x300), kw.get("lse", A + 0x400),
                                             kw.get("scr", A + 0x500), scratch_bytes=kw.get("nb", 1 << 40),
                                             stream=0, raise_on_error=False)
    bwd = lambda cfg, **kw: bl.head_loss_bwd(cfg, kw.get("x", A), kw.get("w", A + 0x100), kw.get("t", A + 0x200),
                                             kw.get("lse", A + 0x400), 1.0, kw.get("dx", A + 0x600),
                                             kw.get("dw", A + 0x700), kw.get("acc", 0), kw.get("scr", A + 0x500),
                                             scratch_bytes=kw.get("nb", 1 << 40), stream=0, raise_on_error=False)
    assert fwd(_hcfg(V=1000)) == E.BLK_EINVAL
    assert fwd(_hcfg(dtype=bl.BLK_F32)) == E.BLK_EUNSUPPORTED
    assert fwd(c, t=None) == E.BLK_EINVAL
    assert fwd(c, loss=None) == E.BLK_EINVAL
    assert fwd(c, x=MIS) == E.BLK_EALIGN
    assert fwd(c, t=A + 0x202) == E.BLK_EALIGN
    assert fwd(c, nb=4096) == E.BLK_ENOSPC
    assert bwd(c, lse=None) == E.BLK_EINVAL
    assert bwd(c, acc=2) == E.BLK_EINVAL
    assert bwd(c, dx=A) == E.BLK_EINVAL           # dx aliases x
    assert bwd(c, dw=MIS) == E.BLK_EALIGN
    assert bwd(c, nb=4096) == E.BLK_ENOSPC
    # ragged token counts with a weight gradient past 32-bit offsets
    assert bl.head_scratch_bytes(_hcfg(N=65537)) == 0


def test_binding_rejects_bad_tensors(lib):
    # the binding checks each tensor's element type, density, size and
    # device before calling the library (one host tensor per call, the other
    # arguments raw addresses; every check runs before the device check,
    # which refuses a host tensor last)
    import torch
    E = bl.binding
    c = bl.BlockConfig(B=1, T=8, C=128, H=1, F=512)
    bf = lambda n: torch.zeros(n, dtype=torch.bfloat16)

    def fwd_err(**kw):
        a = dict(x=A, w_qkv=A, w_o=A, w_fc=A, w_proj=A, y=A + 0x100)
        a.update(kw)
        with pytest.raises(E.BlkError) as e:
            bl.block_fwd(c, a["x"], a["w_qkv"], a["w_o"], a["w_fc"], a["w_proj"], a["y"], None, A)
        assert e.value.code == E.BLK_EINVAL
        return str(e.value)

    assert "dtype" in fwd_err(x=torch.zeros(8 * 128, dtype=torch.float32))
    assert "elements" in fwd_err(y=bf(8 * 128 - 1))
    assert "contiguous" in fwd_err(x=bf(8 * 256)[::2])
    assert "w_fc" in fwd_err(w_fc=bf(512 * 128 - 8))
    assert "GPU" in fwd_err(w_qkv=bf(384 * 128))      # right type and size, but host memory
    with pytest.raises(E.BlkError, match="dw_proj"):
        bl.block_bwd(c, A, A, A, A, A, A, A, A, A, A, A, bf(128 * 512), 0, A)   # weight gradients are float32
    d = bl.DecodeConfig(B=2, C=128, H=1, F=512, S_max=16)
    with pytest.raises(E.BlkError, match="cache_len"):
        bl.decode_step(d, A, A, A, A, A, A, A + 0x100, torch.zeros(2, dtype=torch.int64), A, A, scratch_bytes=1 << 30)
    with pytest.raises(E.BlkError, match="amax"):
        bl.block_fp8_quantize(A, 64, A, torch.zeros(1, dtype=torch.uint8))


def test_mfma_probe_argument_errors(lib):
    E = bl.binding
    probe = lambda kind, wg, it, sink: bl.block_mfma_probe(kind, wg, it, sink, stream=0, raise_on_error=False)
    assert probe(2, 4, 10, A) == E.BLK_EINVAL
    assert probe(0, 0, 10, A) == E.BLK_EINVAL
    assert probe(1, 4, 0, A) == E.BLK_EINVAL
    assert probe(0, 4, 10, None) == E.BLK_EINVAL
    assert probe(0, 4, 10, A + 2) == E.BLK_EALIGN
