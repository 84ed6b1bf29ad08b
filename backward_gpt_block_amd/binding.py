"""ctypes binding of include/blk.h (same names as the C entry points).

Arguments may be torch tensors (their device pointer is passed) or plain
integers (raw device addresses).  ``stream`` defaults to torch's current HIP
stream when torch has a GPU, else NULL (the default stream).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

HERE = os.path.dirname(os.path.abspath(__file__))

BLK_OK, BLK_EINVAL, BLK_EALIGN, BLK_ENOSPC, BLK_EUNSUPPORTED, BLK_ELAUNCH, BLK_ELIMIT = range(7)
BLK_NOALLOC_SCRATCH_BYTES = 32 << 20
BLK_F32, BLK_BF16 = 0, 1
BLK_GEMM_NATIVE, BLK_GEMM_FP8_E4M3 = 0, 1


class BlkError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: status {code} ({block_strerror(code)})")


class _Cfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("C", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("F", ctypes.c_int32), ("eps", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32), ("gemm", ctypes.c_int32),
                ("window", ctypes.c_int32), ("n_kv_head", ctypes.c_int32)]


class _DCfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("C", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("F", ctypes.c_int32), ("S_max", ctypes.c_int32), ("eps", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32), ("window", ctypes.c_int32),
                ("n_kv_head", ctypes.c_int32)]


class _HCfg(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("C", ctypes.c_int32), ("V", ctypes.c_int32), ("eps", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


@dataclasses.dataclass(frozen=True)
class BlockConfig:
    B: int
    T: int
    C: int
    H: int
    F: int
    D: int = 128
    eps: float = 1e-6
    rope_base: float = 10000.0
    dtype: int = BLK_BF16
    gemm: int = BLK_GEMM_NATIVE
    window: int = 0          # attention window (0: causal over the whole sequence)
    n_kv_head: int = 0       # key/value heads (0: as many as query heads)

    def c(self) -> _Cfg:
        return _Cfg(self.B, self.T, self.C, self.H, self.D, self.F, self.eps, self.rope_base, self.dtype, self.gemm,
                    self.window, self.n_kv_head)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    B: int
    C: int
    H: int
    F: int
    S_max: int
    D: int = 128
    eps: float = 1e-6
    rope_base: float = 10000.0
    dtype: int = BLK_BF16
    window: int = 0
    n_kv_head: int = 0

    def c(self) -> _DCfg:
        return _DCfg(self.B, self.C, self.H, self.D, self.F, self.S_max, self.eps, self.rope_base, self.dtype,
                     self.window, self.n_kv_head)


@dataclasses.dataclass(frozen=True)
class HeadConfig:
    N: int
    C: int
    V: int
    eps: float = 1e-6
    dtype: int = BLK_BF16

    def c(self) -> _HCfg:
        return _HCfg(self.N, self.C, self.V, self.eps, self.dtype)


def layer_window(layer: int, n_layer: int, T: int, pattern: str = "SSSL") -> int:
    """Attention window (BlockConfig.window) of layer `layer` of `n_layer`
    under a window pattern: the pattern repeats over the layers, an "S"
    layer attends within a short window of T // 4 tokens, an "L" layer over
    the whole context (0), and the last layer is always full.  The
    flicky.cc course page, section on what changed since GPT-2, gives SSSL
    as the default alternation."""
    if not pattern or any(ch not in "SL" for ch in pattern.upper()):
        raise ValueError(f"window pattern must be a string of S and L, got {pattern!r}")
    if not 0 <= layer < n_layer:
        raise ValueError(f"layer {layer} outside 0..{n_layer - 1}")
    if layer == n_layer - 1 or pattern.upper()[layer % len(pattern)] == "L":
        return 0
    return max(1, T // 4)


_LIB = None


def library_path() -> str:
    return os.path.join(HERE, "libblk.so")


def library() -> ctypes.CDLL:
    """Load libblk.so (built in-tree); raises if it is missing."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m backward_gpt_block_amd.build` "
                               "or __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        pc, pd = ctypes.POINTER(_Cfg), ctypes.POINTER(_DCfg)
        lib.block_saved_bytes.argtypes = [pc]
        lib.block_saved_bytes.restype = sz
        lib.block_scratch_bytes.argtypes = [pc]
        lib.block_scratch_bytes.restype = sz
        lib.block_fwd.argtypes = [pc, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
        lib.block_fwd.restype = i32
        lib.block_bwd.argtypes = [pc, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, i32, vp, sz, vp]
        lib.block_bwd.restype = i32
        lib.decode_scratch_bytes.argtypes = [pd]
        lib.decode_scratch_bytes.restype = sz
        lib.decode_step.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.decode_step.restype = i32
        lib.decode_step_noalloc.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.decode_step_noalloc.restype = i32
        ph = ctypes.POINTER(_HCfg)
        lib.head_scratch_bytes.argtypes = [ph]
        lib.head_scratch_bytes.restype = sz
        lib.head_loss_fwd.argtypes = [ph, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.head_loss_fwd.restype = i32
        lib.head_loss_bwd.argtypes = [ph, vp, vp, vp, vp, ctypes.c_float, vp, vp, i32, vp, sz, vp]
        lib.head_loss_bwd.restype = i32
        lib.block_fp8_quantize.argtypes = [vp, sz, vp, vp, vp]
        lib.block_fp8_quantize.restype = i32
        lib.block_fp8_quantize_2d.argtypes = [vp, ctypes.c_int64, ctypes.c_int64, vp, vp, ctypes.c_int64, vp, vp]
        lib.block_fp8_quantize_2d.restype = i32
        lib.block_mfma_probe.argtypes = [i32, i32, i32, vp, vp]
        lib.block_mfma_probe.restype = i32
        lib.block_timing_enable.argtypes = [i32]
        lib.block_timing_enable.restype = None
        lib.block_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int)]
        lib.block_timing_read.restype = i32
        lib.block_strerror.argtypes = [i32]
        lib.block_strerror.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_DT = {"bf16": "torch.bfloat16", "f32": "torch.float32", "i32": "torch.int32"}


def _arg(t, name: str, where: str, kind=None, numel: int = 0, nbytes: int = 0):
    """Device pointer of argument `name`.  A torch tensor must be dense
    (contiguous), of element type `kind` ('bf16', 'f32', 'i32', or None for a
    byte buffer of any type), hold at least `numel` elements (or `nbytes`
    bytes) and live on the GPU; otherwise BlkError(BLK_EINVAL) is raised
    before the library is called.  Plain integers (raw device addresses) and
    None pass through unchecked."""
    if t is None or isinstance(t, int):
        return t
    bad = None
    if kind is not None and str(t.dtype) != _DT[kind]:
        bad = f"dtype {t.dtype}, expected {_DT[kind]}"
    elif not t.is_contiguous():
        bad = "not contiguous"
    elif t.numel() < numel:
        bad = f"{t.numel()} elements, expected at least {numel}"
    elif t.numel() * t.element_size() < nbytes:
        bad = f"{t.numel() * t.element_size()} bytes, expected at least {nbytes}"
    elif t.device.type != "cuda":
        bad = f"on {t.device}, expected a GPU tensor"
    if bad:
        raise BlkError(BLK_EINVAL, f"{where}: argument {name}: {bad}")
    return t.data_ptr()


def _kind(dtype: int):
    return "bf16" if dtype == BLK_BF16 else ("f32" if dtype == BLK_F32 else None)


def _qkv_width(C: int, H: int, n_kv_head: int) -> int:
    return C + 2 * 128 * (n_kv_head or H)


def _weights(cfg, where, w_qkv, w_o, w_fc, w_proj, kind, prefix=""):
    C, F = cfg.C, cfg.F
    return (_arg(w_qkv, prefix + "w_qkv", where, kind, _qkv_width(C, cfg.H, cfg.n_kv_head) * C),
            _arg(w_o, prefix + "w_o", where, kind, C * C), _arg(w_fc, prefix + "w_fc", where, kind, F * C),
            _arg(w_proj, prefix + "w_proj", where, kind, C * F))


def _nbytes(t, given):
    if given is not None:
        return given
    if t is None or isinstance(t, int):
        return 0
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
    except ImportError:
        pass
    return None


def block_strerror(code: int) -> str:
    return library().block_strerror(code).decode()


def block_saved_bytes(cfg: BlockConfig) -> int:
    return library().block_saved_bytes(ctypes.byref(cfg.c()))


def block_scratch_bytes(cfg: BlockConfig) -> int:
    return library().block_scratch_bytes(ctypes.byref(cfg.c()))


def decode_scratch_bytes(cfg: DecodeConfig) -> int:
    return library().decode_scratch_bytes(ctypes.byref(cfg.c()))


def _check(code, where, raise_on_error):
    if code != BLK_OK and raise_on_error:
        raise BlkError(code, where)
    return code


def block_fwd(cfg: BlockConfig, x, w_qkv, w_o, w_fc, w_proj, y, saved=None, scratch=None, *,
              saved_bytes=None, scratch_bytes=None, stream=None, raise_on_error=True) -> int:
    w, k, n = "block_fwd", _kind(cfg.dtype), cfg.B * cfg.T * cfg.C
    px, py = _arg(x, "x", w, k, n), _arg(y, "y", w, k, n)
    W = _weights(cfg, w, w_qkv, w_o, w_fc, w_proj, k)
    code = library().block_fwd(ctypes.byref(cfg.c()), px, *W, py, _arg(saved, "saved", w), _nbytes(saved, saved_bytes),
                               _arg(scratch, "scratch", w), _nbytes(scratch, scratch_bytes), _stream(stream))
    return _check(code, w, raise_on_error)


def block_bwd(cfg: BlockConfig, dy, x, w_qkv, w_o, w_fc, w_proj, saved, dx, dw_qkv, dw_o, dw_fc, dw_proj,
              accumulate=0, scratch=None, *, saved_bytes=None, scratch_bytes=None, stream=None,
              raise_on_error=True) -> int:
    w, k, n = "block_bwd", _kind(cfg.dtype), cfg.B * cfg.T * cfg.C
    pdy, px, pdx = _arg(dy, "dy", w, k, n), _arg(x, "x", w, k, n), _arg(dx, "dx", w, k, n)
    W = _weights(cfg, w, w_qkv, w_o, w_fc, w_proj, k)
    dW = _weights(cfg, w, dw_qkv, dw_o, dw_fc, dw_proj, "f32", prefix="d")
    code = library().block_bwd(ctypes.byref(cfg.c()), pdy, px, *W, _arg(saved, "saved", w),
                               _nbytes(saved, saved_bytes), pdx, *dW, int(accumulate), _arg(scratch, "scratch", w),
                               _nbytes(scratch, scratch_bytes), _stream(stream))
    return _check(code, w, raise_on_error)


def decode_step(cfg: DecodeConfig, x, w_qkv, w_o, w_fc, w_proj, k_cache, v_cache, cache_len, y, scratch=None, *,
                status=None, scratch_bytes=None, stream=None, raise_on_error=True) -> int:
    """status: optional int32 device word, set to the number of sequences
    whose cache_len is out of range (their y rows are NaN)."""
    w, k = "decode_step", _kind(cfg.dtype)
    ncache = cfg.B * (cfg.n_kv_head or cfg.H) * cfg.S_max * 128
    args = (_arg(x, "x", w, k, cfg.B * cfg.C), *_weights(cfg, w, w_qkv, w_o, w_fc, w_proj, k),
            _arg(k_cache, "k_cache", w, k, ncache), _arg(v_cache, "v_cache", w, k, ncache),
            _arg(cache_len, "cache_len", w, "i32", cfg.B), _arg(status, "status", w, "i32", 1),
            _arg(y, "y", w, k, cfg.B * cfg.C))
    code = library().decode_step(ctypes.byref(cfg.c()), *args, _arg(scratch, "scratch", w),
                                 _nbytes(scratch, scratch_bytes), _stream(stream))
    return _check(code, w, raise_on_error)


def decode_step_noalloc(cfg: DecodeConfig, x, w_qkv, w_o, w_fc, w_proj, k_cache, v_cache, cache_len, y, *,
                        status=None, stream=None, raise_on_error=True) -> int:
    """decode_step with its temporaries in the library's static per-device
    workspace (no scratch argument; nothing allocated)."""
    w, k = "decode_step_noalloc", _kind(cfg.dtype)
    ncache = cfg.B * (cfg.n_kv_head or cfg.H) * cfg.S_max * 128
    args = (_arg(x, "x", w, k, cfg.B * cfg.C), *_weights(cfg, w, w_qkv, w_o, w_fc, w_proj, k),
            _arg(k_cache, "k_cache", w, k, ncache), _arg(v_cache, "v_cache", w, k, ncache),
            _arg(cache_len, "cache_len", w, "i32", cfg.B), _arg(status, "status", w, "i32", 1),
            _arg(y, "y", w, k, cfg.B * cfg.C))
    code = library().decode_step_noalloc(ctypes.byref(cfg.c()), *args, _stream(stream))
    return _check(code, w, raise_on_error)


def head_scratch_bytes(cfg: HeadConfig) -> int:
    return library().head_scratch_bytes(ctypes.byref(cfg.c()))


def head_loss_fwd(cfg: HeadConfig, x, w_lm, targets, loss, lse, scratch=None, *, scratch_bytes=None, stream=None,
                  raise_on_error=True) -> int:
    w, k = "head_loss_fwd", _kind(cfg.dtype)
    args = (_arg(x, "x", w, k, cfg.N * cfg.C), _arg(w_lm, "w_lm", w, k, cfg.V * cfg.C),
            _arg(targets, "targets", w, "i32", cfg.N), _arg(loss, "loss", w, "f32", 1), _arg(lse, "lse", w, "f32", cfg.N))
    code = library().head_loss_fwd(ctypes.byref(cfg.c()), *args, _arg(scratch, "scratch", w),
                                   _nbytes(scratch, scratch_bytes), _stream(stream))
    return _check(code, w, raise_on_error)


def head_loss_bwd(cfg: HeadConfig, x, w_lm, targets, lse, dloss: float, dx, dw_lm, accumulate=0, scratch=None, *,
                  scratch_bytes=None, stream=None, raise_on_error=True) -> int:
    w, k = "head_loss_bwd", _kind(cfg.dtype)
    args = (_arg(x, "x", w, k, cfg.N * cfg.C), _arg(w_lm, "w_lm", w, k, cfg.V * cfg.C),
            _arg(targets, "targets", w, "i32", cfg.N), _arg(lse, "lse", w, "f32", cfg.N))
    code = library().head_loss_bwd(ctypes.byref(cfg.c()), *args, ctypes.c_float(dloss),
                                   _arg(dx, "dx", w, k, cfg.N * cfg.C), _arg(dw_lm, "dw_lm", w, "f32", cfg.V * cfg.C),
                                   int(accumulate), _arg(scratch, "scratch", w), _nbytes(scratch, scratch_bytes),
                                   _stream(stream))
    return _check(code, w, raise_on_error)


def block_fp8_quantize(x, n: int, codes, amax, *, stream=None, raise_on_error=True) -> int:
    w = "block_fp8_quantize"
    code = library().block_fp8_quantize(_arg(x, "x", w, "bf16", int(n)), int(n), _arg(codes, "codes", w, nbytes=int(n)),
                                        _arg(amax, "amax", w, nbytes=4), _stream(stream))
    return _check(code, w, raise_on_error)


def block_fp8_quantize_2d(x, rows: int, cols: int, codes, codes_t, ldt: int, amax, *, stream=None,
                          raise_on_error=True) -> int:
    w = "block_fp8_quantize_2d"
    code = library().block_fp8_quantize_2d(_arg(x, "x", w, "bf16", rows * cols), int(rows), int(cols),
                                           _arg(codes, "codes", w, nbytes=rows * cols),
                                           _arg(codes_t, "codes_t", w, nbytes=cols * ldt), int(ldt),
                                           _arg(amax, "amax", w, nbytes=4), _stream(stream))
    return _check(code, w, raise_on_error)


def block_mfma_probe(kind: int, workgroups: int, iters: int, sink, *, stream=None, raise_on_error=True) -> int:
    """Register-only MFMA loop (kind 0 bf16, 1 E4M3) for measuring the
    matrix cores' achievable rate; sink holds workgroups * 256 floats."""
    w = "block_mfma_probe"
    code = library().block_mfma_probe(int(kind), int(workgroups), int(iters),
                                      _arg(sink, "sink", w, "f32", int(workgroups) * 256), _stream(stream))
    return _check(code, w, raise_on_error)


def block_timing_enable(on: bool) -> None:
    library().block_timing_enable(1 if on else 0)


def block_timing_read(max_entries: int = 64) -> dict:
    """{launch site: (total_ms, launches)} recorded since enabling."""
    names = (ctypes.c_char_p * max_entries)()
    tot = (ctypes.c_double * max_entries)()
    cnt = (ctypes.c_int * max_entries)()
    n = library().block_timing_read(max_entries, names, tot, cnt)
    if n < 0:
        raise RuntimeError("block_timing_read: HIP error")
    return {names[i].decode(): (tot[i], cnt[i]) for i in range(n)}
