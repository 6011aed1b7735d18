"""ctypes binding of librotattn (the C ABI in include/rotattn.h).

Argument marshalling only: every step of the hot path runs in the library's HIP
kernels.  torch provides device memory and the current stream.  There is no CPU
fallback: if the library is not built, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librotattn.so")

ROT_NONE, ROT_INTERLEAVED, ROT_HALF, ROT_FULL = 0, 1, 2, 3
F32, F16, BF16 = 0, 1, 2
_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
ROT_BY_NAME = {"none": ROT_NONE, "interleaved": ROT_INTERLEAVED, "half": ROT_HALF, "full": ROT_FULL}


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "H", "F", "Hs", "Ws", "D", "Df", "Dh", "Dw", "qk_blk", "kv_blk")]

    @classmethod
    def of(cls, cfg) -> "Shape":
        return cls(*[int(cfg[n]) for n, _ in cls._fields_])

    @property
    def N(self) -> int:
        return self.F * self.Hs * self.Ws


class Debug(ctypes.Structure):
    _fields_ = [("bh", ctypes.c_int32), ("row0", ctypes.c_int32), ("n_rows", ctypes.c_int32),
                ("a_qk", ctypes.c_void_p), ("p_codes", ctypes.c_void_p), ("a_pv", ctypes.c_void_p),
                ("m", ctypes.c_void_p), ("l", ctypes.c_void_p)]


class QuantizeOpts(ctypes.Structure):
    _fields_ = [("smooth_k", ctypes.c_int32), ("smooth_q", ctypes.c_int32), ("k_bias", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p)]


class AttentionOpts(ctypes.Structure):
    _fields_ = [("p_max", ctypes.c_int32), ("causal_block", ctypes.c_int32), ("k_bias", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("skip_stats", ctypes.c_void_p)]


class FallbackOpts(ctypes.Structure):
    _fields_ = [("causal_block", ctypes.c_int32), ("seq_lens", ctypes.c_void_p)]


class RotattnError(RuntimeError):
    pass


_lib = None
_VP, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "rotattn_check_shape": (_I32, [_VP]),
    "rotattn_padded_tokens": (ctypes.c_int64, [_VP]),
    "rotattn_rope_table_floats": (_SZ, [_VP]),
    "rotattn_build_rope_table": (_I32, [_VP, _I32, ctypes.c_double, _VP]),
    "rotattn_quantize_qk_workspace": (_SZ, [_VP]),
    "rotattn_quantize_qk": (_I32, [_VP, _I32, _I32, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP,
                                   _VP, _VP, _VP, _SZ, _VP]),
    "rotattn_int4_attention_workspace": (_SZ, [_VP]),
    "rotattn_int4_attention": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _VP, _VP, _VP, _SZ,
                                      _VP]),
    "rotattn_int4_attention_symmetric_p": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _VP, _VP, _VP,
                                                  _SZ, _VP]),
    "rotattn_quantize_qk_ex": (_I32, [_VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                      _VP, _VP, _VP, _SZ, _VP]),
    "rotattn_int4_attention_ex": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _I32, _VP, _VP,
                                         _VP, _SZ, _VP]),
    "rotattn_fp16_fallback_workspace": (_SZ, [_VP]),
    "rotattn_fp16_fallback": (_I32, [_VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _VP, _VP, _SZ, _VP]),
    "rotattn_fp16_fallback_ex": (_I32, [_VP, _I32, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _I32, _VP, _VP, _SZ,
                                        _VP]),
    "rotattn_p_level_probe": (_I32, [ctypes.c_uint32, ctypes.c_int64, _VP, _VP]),
    "rotattn_quantize_qk_noalloc_max_scratch": (_SZ, []),
    "rotattn_quantize_qk_noalloc_scratch": (_SZ, [_VP]),
    "rotattn_quantize_qk_noalloc": (_I32, [_VP, _I32, _I32, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _VP, _VP, _VP,
                                           _VP, _VP, _VP]),
    "rotattn_status_str": (ctypes.c_char_p, [_I32]),
}


def lib():
    """Load librotattn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RotattnError("librotattn.so is not built (run __graft_entry__.build() or "
                               "python -m int4_quantized_attention_amd.build_lib)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(st: int, what: str):
    if st != 0:
        raise RotattnError("%s: %s (status %d)" % (what, lib().rotattn_status_str(st).decode(), st))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise RotattnError("expected a contiguous device tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _lens(seq_lens: Optional[Sequence[int]]):
    """Host int32 array of per-element lengths (kept alive by the caller's frame)."""
    if seq_lens is None:
        return None
    return (ctypes.c_int32 * len(seq_lens))(*[int(n) for n in seq_lens])


def _heads(heads: Optional[Sequence[int]]):
    if heads is None:
        return None, 0
    arr = (ctypes.c_int32 * len(heads))(*[int(h) for h in heads])
    return arr, len(heads)


# ---- thin wrappers with the C names ---------------------------------------------

def rotattn_check_shape(shape: Shape) -> int:
    return lib().rotattn_check_shape(ctypes.byref(shape))


def rotattn_padded_tokens(shape: Shape) -> int:
    return int(lib().rotattn_padded_tokens(ctypes.byref(shape)))


def rotattn_build_rope_table(shape: Shape, rot: int, base: float = 10000.0) -> torch.Tensor:
    """Host RoPE table (float32 CPU tensor); copy it to the device for the calls."""
    n = lib().rotattn_rope_table_floats(ctypes.byref(shape))
    out = torch.empty(n, dtype=torch.float32)
    _check(lib().rotattn_build_rope_table(ctypes.byref(shape), rot, base, ctypes.c_void_p(out.data_ptr())),
           "rotattn_build_rope_table")
    return out


def rotattn_quantize_qk_workspace(shape: Shape) -> int:
    return int(lib().rotattn_quantize_qk_workspace(ctypes.byref(shape)))


def rotattn_int4_attention_workspace(shape: Shape) -> int:
    return int(lib().rotattn_int4_attention_workspace(ctypes.byref(shape)))


def rotattn_fp16_fallback_workspace(shape: Shape) -> int:
    return int(lib().rotattn_fp16_fallback_workspace(ctypes.byref(shape)))


def alloc_codes(shape: Shape, device="cuda", colsum: bool = True, smooth_q: bool = False) -> dict:
    """Output buffers of rotattn_quantize_qk (torch device tensors); smooth_q adds
    k_bias [B,H,Np] f32 for Q smoothing (rotattn_quantize_qk_ex with smooth_q set)."""
    Np = rotattn_padded_tokens(shape)
    B, H, D = shape.B, shape.H, shape.D
    nkb = -(-shape.N // shape.kv_blk)
    u8, f32 = torch.uint8, torch.float32
    z = dict(q_codes=torch.empty((B, H, Np, D // 2), dtype=u8, device=device),
             q_scale=torch.empty((B, H, Np // shape.qk_blk), dtype=f32, device=device),
             k_codes=torch.empty((B, H, Np, D // 2), dtype=u8, device=device),
             k_scale=torch.empty((B, H, Np // shape.qk_blk), dtype=f32, device=device),
             v_codes=torch.empty((B, H, D, Np // 2), dtype=u8, device=device),
             v_scale=torch.empty((B, H, D), dtype=f32, device=device),
             v_colsum=torch.empty((B, H, nkb, D), dtype=torch.int32, device=device) if colsum else None)
    if smooth_q:
        z["k_bias"] = torch.empty((B, H, Np), dtype=f32, device=device)
    z["workspace"] = torch.empty(rotattn_quantize_qk_workspace(shape), dtype=torch.uint8, device=device)
    z["attn_workspace"] = torch.empty(rotattn_int4_attention_workspace(shape), dtype=torch.uint8, device=device)
    return z


def rotattn_quantize_qk(shape: Shape, rot: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        rope_table: torch.Tensor, smooth_k: bool, z: dict, smooth_q: bool = False,
                        seq_lens: Optional[Sequence[int]] = None) -> dict:
    """z: buffers from alloc_codes (filled in place, returned).  smooth_q: Q smoothing,
    which fills z["k_bias"] (alloc_codes with smooth_q=True); seq_lens: B lengths of
    a variable-length batch.  Either goes through rotattn_quantize_qk_ex, and
    rotattn_int4_attention then takes both from z."""
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise RotattnError("q, k, v must share one of float32 / float16 / bfloat16")
    ws = z["workspace"]
    head = (ctypes.byref(shape), rot, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(rope_table))
    codes = (_ptr(z["q_codes"]), _ptr(z["q_scale"]), _ptr(z["k_codes"]), _ptr(z["k_scale"]),
             _ptr(z["v_codes"]), _ptr(z["v_scale"]), _ptr(z.get("v_colsum")))
    tail = (_ptr(ws), ws.numel(), _stream())
    if smooth_q and z.get("k_bias") is None:
        raise RotattnError("Q smoothing needs z['k_bias'] (alloc_codes(..., smooth_q=True))")
    if smooth_q or seq_lens is not None:
        lens = _lens(seq_lens)
        opts = QuantizeOpts(1 if smooth_k else 0, 1 if smooth_q else 0, _ptr(z["k_bias"]) if smooth_q else None,
                            ctypes.cast(lens, ctypes.c_void_p) if lens is not None else None)
        _check(lib().rotattn_quantize_qk_ex(*head, ctypes.byref(opts), *codes, *tail), "rotattn_quantize_qk_ex")
    else:
        _check(lib().rotattn_quantize_qk(*head, 1 if smooth_k else 0, *codes, *tail), "rotattn_quantize_qk")
    z["smooth_q"] = bool(smooth_q)
    z["seq_lens"] = None if seq_lens is None else [int(n) for n in seq_lens]
    return z


def rotattn_int4_attention(shape: Shape, z: dict, out: torch.Tensor, heads: Optional[Sequence[int]] = None,
                           debug: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
                           symmetric_p: bool = False, causal_block: int = 0,
                           skip_stats: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out: device [B,H,N,D] float32, float16 or bfloat16.  debug: dict(bh, row0, n_rows) ->
    filled with device tensors a_qk, p_codes, a_pv, m, l.  workspace: device uint8
    tensor of rotattn_int4_attention_workspace(shape) bytes (default z["attn_workspace"]).
    symmetric_p: the ablation baseline rotattn_int4_attention_symmetric_p (P codes
    round(7P) in [0, 7]) instead of the method's range-rectified codes.
    causal_block: 0 bidirectional; c > 0 block-causal (query i sees key j iff
    j // c <= i // c).  When z was filled with Q smoothing or a variable-length
    batch, its k_bias and seq_lens are passed on (rows past a sequence's length are
    left untouched).  skip_stats: device int64 tensor of 5 counters that the run adds
    its counts of the exact skips to (see rotattn_attention_opts in the header).
    Options other than the defaults go through rotattn_int4_attention_ex."""
    if out.dtype not in _DT:
        raise RotattnError("out must be float32, float16 or bfloat16")
    harr, nh = _heads(heads)
    ws = workspace if workspace is not None else z["attn_workspace"]
    dbg = None
    if debug is not None:
        n, N = int(debug["n_rows"]), shape.N
        S = -(-N // shape.kv_blk)
        dev = out.device
        debug.update(a_qk=torch.zeros((n, N), dtype=torch.int32, device=dev),
                     p_codes=torch.zeros((n, N), dtype=torch.int8, device=dev),
                     a_pv=torch.zeros((n, S, shape.D), dtype=torch.int32, device=dev),
                     m=torch.zeros(n, dtype=torch.float32, device=dev),
                     l=torch.zeros(n, dtype=torch.float32, device=dev))
        dbg = Debug(int(debug["bh"]), int(debug["row0"]), n, debug["a_qk"].data_ptr(),
                    debug["p_codes"].data_ptr(), debug["a_pv"].data_ptr(), debug["m"].data_ptr(),
                    debug["l"].data_ptr())
    codes = (_ptr(z["q_codes"]), _ptr(z["q_scale"]), _ptr(z["k_codes"]), _ptr(z["k_scale"]),
             _ptr(z["v_codes"]), _ptr(z["v_scale"]), harr, nh)
    tail = (_DT[out.dtype], _ptr(out), ctypes.byref(dbg) if dbg is not None else None, _ptr(ws), ws.numel(),
            _stream())
    kb = z.get("k_bias") if z.get("smooth_q") else None
    lens = _lens(z.get("seq_lens"))
    if skip_stats is not None and (skip_stats.dtype != torch.int64 or skip_stats.numel() != 5):
        raise RotattnError("skip_stats must be a device int64 tensor of 5 counters")
    if causal_block or kb is not None or lens is not None or skip_stats is not None:
        opts = AttentionOpts(7 if symmetric_p else 15, int(causal_block), _ptr(kb),
                             ctypes.cast(lens, ctypes.c_void_p) if lens is not None else None,
                             _ptr(skip_stats))
        _check(lib().rotattn_int4_attention_ex(ctypes.byref(shape), *codes, ctypes.byref(opts), *tail),
               "rotattn_int4_attention_ex")
    else:
        fn = lib().rotattn_int4_attention_symmetric_p if symmetric_p else lib().rotattn_int4_attention
        _check(fn(ctypes.byref(shape), *codes, *tail), "rotattn_int4_attention")
    return out


def rotattn_fp16_fallback(shape: Shape, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          rope_table: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                          heads: Optional[Sequence[int]] = None, causal_block: int = 0,
                          seq_lens: Optional[Sequence[int]] = None) -> torch.Tensor:
    """q, k, v: device [B,H,N,D] of one of float32 / float16 / bfloat16 (rounded to
    binary16 after RoPE); out: float32, float16 or bfloat16.  causal_block as for
    rotattn_int4_attention, seq_lens a variable-length batch (both through
    rotattn_fp16_fallback_ex)."""
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise RotattnError("q, k, v must share one of float32 / float16 / bfloat16")
    if out.dtype not in _DT:
        raise RotattnError("out must be float32, float16 or bfloat16")
    harr, nh = _heads(heads)
    head = (ctypes.byref(shape), _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(rope_table), harr, nh)
    tail = (_DT[out.dtype], _ptr(out), _ptr(workspace), workspace.numel(), _stream())
    if causal_block or seq_lens is not None:
        lens = _lens(seq_lens)
        opts = FallbackOpts(int(causal_block), ctypes.cast(lens, ctypes.c_void_p) if lens is not None else None)
        _check(lib().rotattn_fp16_fallback_ex(*head, ctypes.byref(opts), *tail), "rotattn_fp16_fallback_ex")
    else:
        _check(lib().rotattn_fp16_fallback(*head, *tail), "rotattn_fp16_fallback")
    return out


def rotattn_p_level_probe(first_bits: int, n: int, out: torch.Tensor) -> torch.Tensor:
    """out: device uint8 tensor of at least n elements; out[i] = the attention's P
    level decision for the binary32 exponent with bit pattern first_bits + i (low
    nibble) and the exact threshold fix alone (high nibble)."""
    if out.dtype != torch.uint8 or out.numel() < n:
        raise RotattnError("out must be a device uint8 tensor of at least n elements")
    _check(lib().rotattn_p_level_probe(ctypes.c_uint32(first_bits), ctypes.c_int64(n), _ptr(out), _stream()),
           "rotattn_p_level_probe")
    return out


def rotattn_quantize_qk_noalloc(shape: Shape, rot: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                rope_table: torch.Tensor, smooth_k: bool, z: dict) -> dict:
    """rotattn_quantize_qk without a workspace: the library's fixed per-device scratch
    (calls on one device must not overlap).  z: code buffers as from alloc_codes
    (its workspaces are not used)."""
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise RotattnError("q, k, v must share one of float32 / float16 / bfloat16")
    _check(lib().rotattn_quantize_qk_noalloc(
        ctypes.byref(shape), rot, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(rope_table), 1 if smooth_k else 0,
        _ptr(z["q_codes"]), _ptr(z["q_scale"]), _ptr(z["k_codes"]), _ptr(z["k_scale"]), _ptr(z["v_codes"]),
        _ptr(z["v_scale"]), _ptr(z.get("v_colsum")), _stream()), "rotattn_quantize_qk_noalloc")
    z["smooth_q"] = False
    z["seq_lens"] = None
    return z
