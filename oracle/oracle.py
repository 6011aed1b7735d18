"""Python binding of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  The product package never imports it, and it never
imports the product package: the two share no code (only the seeded input
generators in ``int4_quantized_attention_amd.synth`` feed both).

Every function is a thin ctypes wrapper around ``rotattn_oracle.cpp``; the C++
file holds the arithmetic and cites the passages of the RotateAttention pages
each step follows.  Arrays are numpy, C-contiguous.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rotattn_oracle.cpp")
_LIB = os.path.join(_HERE, "liborc.so")

ROT_NONE, ROT_INTERLEAVED, ROT_HALF, ROT_FULL = 0, 1, 2, 3

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with g++ (plain C++17, OpenMP, no fp contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
        _lib.orc_table_entries.restype = ctypes.c_int64
        _lib.orc_c0.restype = ctypes.c_float
        _lib.orc_c0.argtypes = [ctypes.c_int32]
        _lib.orc_l15.restype = ctypes.c_float
        _lib.orc_p_level_bruteforce.restype = ctypes.c_int64
        _lib.orc_p_level_bruteforce.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
        _lib.orc_rope_table.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p]
        _lib.orc_rope_table_f64.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p]
    return _lib


def _p(a):
    return ctypes.c_void_p(0) if a is None else a.ctypes.data_as(ctypes.c_void_p)


def shape_array(shape) -> np.ndarray:
    """shape: mapping with B,H,F,Hs,Ws,D,Df,Dh,Dw,qk_blk,kv_blk."""
    keys = ("B", "H", "F", "Hs", "Ws", "D", "Df", "Dh", "Dw", "qk_blk", "kv_blk")
    return np.array([int(shape[k]) for k in keys], dtype=np.int32)


def n_tokens(shape) -> int:
    return int(shape["F"]) * int(shape["Hs"]) * int(shape["Ws"])


def rope_table(shape, rot: int, base: float = 10000.0, f64: bool = False) -> np.ndarray:
    s = shape_array(shape)
    n = lib().orc_table_entries(_p(s))
    if f64:
        out = np.empty(n, dtype=np.float64)
        lib().orc_rope_table_f64(_p(s), rot, base, _p(out))
    else:
        out = np.empty(n, dtype=np.float32)
        lib().orc_rope_table(_p(s), rot, base, _p(out))
    return out


def rope_rotate(shape, rot: int, table: np.ndarray, x: np.ndarray) -> np.ndarray:
    s = shape_array(shape)
    if x.dtype == np.float64:
        x = np.ascontiguousarray(x)
        out = np.empty_like(x)
        lib().orc_rope_rotate_f64(_p(s), ctypes.c_int32(rot), _p(np.ascontiguousarray(table, np.float64)),
                                  _p(x), _p(out))
    else:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty_like(x)
        lib().orc_rope_rotate(_p(s), ctypes.c_int32(rot), _p(np.ascontiguousarray(table, np.float32)),
                              _p(x), _p(out))
    return out


def _lens(seq_lens, B):
    if seq_lens is None:
        return None
    a = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if a.shape != (B,):
        raise ValueError("seq_lens needs one length per batch element")
    return a


def quantize(shape, rot: int, table: np.ndarray, q, k, v, smooth_k: bool = True, diag: bool = False,
             smooth_q: bool = False, seq_lens=None):
    """Returns dict: qc,kc,vc (int8 [B,H,N,D]), qs,ks ([B,H,nqb]), vs ([B,H,D]),
    vcol ([B,H,nkb,D]); with diag also q_rot, k_rot, k_mu, q_mu.  smooth_q: Q minus
    its channel mean, and k_bias [B,H,N] f32 = mu_q . K_j (pass it to attention).
    seq_lens: B lengths of a variable-length batch (kept in the result for attention)."""
    s = shape_array(shape)
    B, H, D = int(shape["B"]), int(shape["H"]), int(shape["D"])
    N = n_tokens(shape)
    nqb = -(-N // int(shape["qk_blk"]))
    nkb = -(-N // int(shape["kv_blk"]))
    q = np.ascontiguousarray(q, dtype=np.float32).reshape(B, H, N, D)
    k = np.ascontiguousarray(k, dtype=np.float32).reshape(B, H, N, D)
    v = np.ascontiguousarray(v, dtype=np.float32).reshape(B, H, N, D)
    r = dict(
        qc=np.empty((B, H, N, D), np.int8), qs=np.empty((B, H, nqb), np.float32),
        kc=np.empty((B, H, N, D), np.int8), ks=np.empty((B, H, nqb), np.float32),
        vc=np.empty((B, H, N, D), np.int8), vs=np.empty((B, H, D), np.float32),
        vcol=np.empty((B, H, nkb, D), np.int32))
    if diag:
        r["q_rot"] = np.empty((B, H, N, D), np.float32)
        r["k_rot"] = np.empty((B, H, N, D), np.float32)
        r["k_mu"] = np.empty((B, H, D), np.float32)
        r["q_mu"] = np.empty((B, H, D), np.float32)
    if smooth_q:
        r["k_bias"] = np.empty((B, H, N), np.float32)
    flags = (1 if smooth_k else 0) | (2 if smooth_q else 0)
    lens = _lens(seq_lens, B)
    if lens is not None:
        r["seq_lens"] = lens
    lib().orc_quantize_x(_p(s), ctypes.c_int32(rot), _p(np.ascontiguousarray(table, np.float32)),
                         ctypes.c_int32(flags), _p(q), _p(k), _p(v),
                         _p(r["qc"]), _p(r["qs"]), _p(r["kc"]), _p(r["ks"]),
                         _p(r["vc"]), _p(r["vs"]), _p(r["vcol"]),
                         _p(r.get("q_rot")), _p(r.get("k_rot")), _p(r.get("k_mu")), _p(r.get("q_mu")),
                         _p(r.get("k_bias")), _p(lens))
    return r


def key_limit(i, N: int, causal_block: int = 0):
    """Keys a query token i sees: all N for causal_block 0 (bidirectional), else
    the keys of its own block of causal_block tokens and every earlier block."""
    if causal_block <= 0:
        return np.full(np.shape(i), N, dtype=np.int64)
    return np.minimum(N, (np.asarray(i) // causal_block + 1) * causal_block)


def attention(shape, qz: dict, rows=None, dumps: bool = False, pmax: int = 15,
              causal_block: int = 0):
    """Quantised attention for flat rows (b*H + h)*N + i (default: all rows).
    Returns dict with 'out' [rows, D] float64 and, with dumps, 'a_qk' [rows, N]
    int32, 'pcode' [rows, N] int8, 'a_pv' [rows, S, D] int32, 'm' f32, 'l' f64.
    pmax = 15: range-rectified P codes r - 8 in [-8, 7] (the method); pmax = 7: the
    symmetric baseline, codes r = round(7 P) in [0, 7].  causal_block: 0 for
    bidirectional attention, c > 0 for block-causal attention (key_limit); dump
    entries of keys a row does not see stay zero.  A "k_bias" entry in qz (from
    quantize(..., smooth_q=True)) adds the per-key term Q smoothing leaves; a
    "seq_lens" entry (quantize(..., seq_lens=...)) makes the batch variable-length."""
    if pmax not in (7, 15):
        raise ValueError("pmax is 15 (range-rectified) or 7 (symmetric baseline)")
    s = shape_array(shape)
    B, H, D = int(shape["B"]), int(shape["H"]), int(shape["D"])
    N = n_tokens(shape)
    S = -(-N // int(shape["kv_blk"]))
    if rows is None:
        rows = np.arange(B * H * N, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    R = rows.size
    res = {"out": np.empty((R, D), np.float64)}
    if dumps:
        res.update(a_qk=np.zeros((R, N), np.int32), pcode=np.zeros((R, N), np.int8),
                   a_pv=np.zeros((R, S, D), np.int32), m=np.empty(R, np.float32),
                   l=np.empty(R, np.float64))
    c = lambda a, t: np.ascontiguousarray(a, dtype=t)
    lib().orc_attention_x(_p(s), _p(c(qz["qc"], np.int8)), _p(c(qz["qs"], np.float32)),
                        _p(c(qz["kc"], np.int8)), _p(c(qz["ks"], np.float32)),
                        _p(c(qz["vc"], np.int8)), _p(c(qz["vs"], np.float32)),
                        _p(rows), ctypes.c_int64(R), _p(res["out"]),
                        _p(res.get("a_qk")), _p(res.get("pcode")), _p(res.get("a_pv")),
                        _p(res.get("m")), _p(res.get("l")), ctypes.c_int32(pmax),
                        ctypes.c_int32(causal_block),
                        _p(c(qz["k_bias"], np.float32) if qz.get("k_bias") is not None else None),
                        _p(_lens(qz.get("seq_lens"), B)))
    return res


def exact_attention(shape, q, k, v, rows=None, base: float = 10000.0,
                    causal_block: int = 0, seq_lens=None) -> np.ndarray:
    s = shape_array(shape)
    B, H, D = int(shape["B"]), int(shape["H"]), int(shape["D"])
    N = n_tokens(shape)
    if rows is None:
        rows = np.arange(B * H * N, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    tab = rope_table(shape, ROT_NONE, base, f64=True)
    out = np.empty((rows.size, D), np.float64)
    c = lambda a: np.ascontiguousarray(a, dtype=np.float32).reshape(B, H, N, D)
    lib().orc_exact_attention_x(_p(s), _p(tab), _p(c(q)), _p(c(k)), _p(c(v)), _p(rows),
                                ctypes.c_int64(rows.size), _p(out), ctypes.c_int32(causal_block),
                                _p(_lens(seq_lens, B)))
    return out


def fallback_attention(shape, table_plain, q, k, v, rows=None, causal_block: int = 0,
                       seq_lens=None) -> np.ndarray:
    s = shape_array(shape)
    B, H, D = int(shape["B"]), int(shape["H"]), int(shape["D"])
    N = n_tokens(shape)
    if rows is None:
        rows = np.arange(B * H * N, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, D), np.float64)
    c = lambda a: np.ascontiguousarray(a, dtype=np.float32).reshape(B, H, N, D)
    lib().orc_fallback_attention_x(_p(s), _p(np.ascontiguousarray(table_plain, np.float32)),
                                   _p(c(q)), _p(c(k)), _p(c(v)), _p(rows),
                                   ctypes.c_int64(rows.size), _p(out), ctypes.c_int32(causal_block),
                                   _p(_lens(seq_lens, B)))
    return out


def p_thresholds() -> np.ndarray:
    out = np.empty(15, np.float32)
    lib().orc_p_thresholds(_p(out))
    return out


def p_levels(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.int8)
    lib().orc_p_levels(_p(y), ctypes.c_int64(y.size), _p(out))
    return out


def p_level_bruteforce(lo: float, hi: float):
    first = np.zeros(1, np.float32)
    bad = lib().orc_p_level_bruteforce(lo, hi, first.ctypes.data_as(ctypes.c_void_p))
    return int(bad), float(first[0])


def c0(D: int) -> float:
    return float(lib().orc_c0(D))


def l15() -> float:
    return float(lib().orc_l15())


def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16(_p(x), ctypes.c_int64(x.size), _p(out))
    return out


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two signed 4-bit codes per byte along the last axis: element 2i in the low
    nibble, 2i+1 in the high nibble (layout only; used to compare packed codes)."""
    c = codes.astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)
