"""Helpers of the GPU tests: run the library on torch device tensors, unpack its
code layouts, and compare with the oracle.  (Layout helpers only; no arithmetic
of the method.)"""
import numpy as np
import torch

from int4_quantized_attention_amd import rotattn as ra
from int4_quantized_attention_amd import synth

_TDT = {"float16": torch.float16, "float32": torch.float32, "bfloat16": torch.bfloat16}


def to_dev(x: np.ndarray, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def gpu_quantize(cfg, rot: int, Q, K, V, smooth=True, in_dtype=None, smooth_q=False):
    shape = ra.Shape.of(cfg)
    tdt = in_dtype or _TDT[cfg["dtype"]]
    q, k, v = (to_dev(x, tdt) for x in (Q, K, V))
    tab = ra.rotattn_build_rope_table(shape, rot).cuda()
    z = ra.alloc_codes(shape, smooth_q=smooth_q)
    ra.rotattn_quantize_qk(shape, rot, q, k, v, tab, smooth, z, smooth_q=smooth_q)
    torch.cuda.synchronize()
    return shape, z


def unpack_rows(codes_u8: torch.Tensor) -> np.ndarray:
    """[..., n/2] bytes -> [..., n] signed nibbles (element 2i low nibble)."""
    b = codes_u8.cpu().numpy().astype(np.int16)
    lo, hi = b & 0xF, (b >> 4) & 0xF
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int16)
    out[..., 0::2], out[..., 1::2] = lo, hi
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def compare_codes(cfg, z, ref, heads=None):
    """Bit-exact comparison of the library's code tensors with the oracle's
    (restricted to flat head ids `heads` of the library's tensors, which the
    oracle computed as its heads 0..len-1)."""
    B, H, D = cfg["B"], cfg["H"], cfg["D"]
    N = synth.n_tokens(cfg)
    qb, kb = cfg["qk_blk"], cfg["kv_blk"]
    nqb, nkb = -(-N // qb), -(-N // kb)
    sel = list(range(B * H)) if heads is None else list(heads)
    f = lambda t: t.reshape((B * H,) + tuple(t.shape[2:]))[sel]
    qc, kc = unpack_rows(f(z["q_codes"])), unpack_rows(f(z["k_codes"]))
    vc = unpack_rows(f(z["v_codes"]))  # [h, D, Np]
    r = lambda a: a.reshape((-1,) + a.shape[2:])
    assert np.array_equal(qc[:, :N], r(ref["qc"])), "q codes"
    assert np.all(qc[:, N:] == 0), "q padding"
    assert np.array_equal(kc[:, :N], r(ref["kc"])), "k codes"
    assert np.all(kc[:, N:] == 0), "k padding"
    assert np.array_equal(vc[:, :, :N].transpose(0, 2, 1), r(ref["vc"])), "v codes"
    assert np.all(vc[:, :, N:] == 0), "v padding"
    qs, ks = f(z["q_scale"]).cpu().numpy(), f(z["k_scale"]).cpu().numpy()
    assert np.array_equal(qs[:, :nqb].view(np.uint32), r(ref["qs"]).view(np.uint32)), "q scales"
    assert np.array_equal(ks[:, :nqb].view(np.uint32), r(ref["ks"]).view(np.uint32)), "k scales"
    assert np.all(qs[:, nqb:] == 0) and np.all(ks[:, nqb:] == 0)
    vs = f(z["v_scale"]).cpu().numpy()
    assert np.array_equal(vs.view(np.uint32), r(ref["vs"]).view(np.uint32)), "v scales"
    if z.get("v_colsum") is not None:
        assert np.array_equal(f(z["v_colsum"]).cpu().numpy()[:, :nkb], r(ref["vcol"])), "v colsums"
    if z.get("smooth_q"):
        kb = f(z["k_bias"]).cpu().numpy()
        assert np.array_equal(kb[:, :N].view(np.uint32), r(ref["k_bias"]).view(np.uint32)), "k bias"
        assert np.all(kb[:, N:] == 0), "k bias padding"


def assert_close(out: np.ndarray, ref: np.ndarray, max_abs=2e-3, rel_l2=1e-3, what="O"):
    out = out.astype(np.float64)
    err = np.abs(out - ref)
    rl2 = np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-30)
    assert np.isfinite(out).all(), what + " has non-finite values"
    assert err.max() <= max_abs, "%s max-abs err %.3g > %.3g" % (what, err.max(), max_abs)
    assert rl2 <= rel_l2, "%s rel-L2 err %.3g > %.3g" % (what, rl2, rel_l2)
    return float(err.max()), float(rl2)


def rows_sample(N: int, n_rand: int = 32, seed: int = 0):
    """First tile, the ragged last tile and some random rows of one head."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(N, 40))) | set(range(max(0, N - 40), N))
    rows |= set(rng.integers(0, N, n_rand).tolist())
    return np.array(sorted(rows), np.int64)


def pack_rows(codes: np.ndarray) -> np.ndarray:
    """[..., n] signed nibbles -> [..., n/2] bytes (element 2i in the low nibble)."""
    c = codes.astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def upload_codes(cfg, zc: dict) -> dict:
    """Code tensors in the oracle's layout (qc, kc, vc int8 [B,H,N,D]; qs, ks
    [B,H,ceil(N/qk_blk)]; vs [B,H,D]) -> the library's padded device layout, as
    rotattn_quantize_qk would have written them (layout only)."""
    shape = ra.Shape.of(cfg)
    B, H, D = cfg["B"], cfg["H"], cfg["D"]
    N = synth.n_tokens(cfg)
    Np = ra.rotattn_padded_tokens(shape)
    qb = cfg["qk_blk"]
    nqb = -(-N // qb)
    z = ra.alloc_codes(shape, colsum=False)

    def rows(x):
        out = np.zeros((B, H, Np, D), np.int8)
        out[:, :, :N] = x
        return out

    z["q_codes"].copy_(torch.from_numpy(pack_rows(rows(zc["qc"]))))
    z["k_codes"].copy_(torch.from_numpy(pack_rows(rows(zc["kc"]))))
    z["v_codes"].copy_(torch.from_numpy(pack_rows(np.ascontiguousarray(rows(zc["vc"]).transpose(0, 1, 3, 2)))))
    for name in ("qs", "ks"):
        s = np.zeros((B, H, Np // qb), np.float32)
        s[:, :, :nqb] = zc[name]
        z["q_scale" if name == "qs" else "k_scale"].copy_(torch.from_numpy(s))
    z["v_scale"].copy_(torch.from_numpy(np.ascontiguousarray(zc["vs"], np.float32)))
    torch.cuda.synchronize()
    return z


def debug_run(shape, z, out_like, bh, r0, n, **kw):
    """One debug launch of rotattn_int4_attention over rows [r0, r0+n) of head bh;
    returns (dumps as numpy, the output rows as numpy)."""
    dbg = dict(bh=bh, row0=r0, n_rows=n)
    out2 = torch.zeros_like(out_like)
    ra.rotattn_int4_attention(shape, z, out2, debug=dbg, **kw)
    torch.cuda.synchronize()
    H = out_like.shape[1]
    d = {k: dbg[k].cpu().numpy() for k in ("a_qk", "p_codes", "a_pv", "m", "l")}
    return d, out2[bh // H, bh % H, r0:r0 + n].float().cpu().numpy()


def l_rtol(n_keys: int, kv_blk: int) -> float:
    """Relative bound on the GPU's normaliser against the oracle's binary64 sum: each
    lane adds its half of the keys' p in binary32 one at a time (recursive summation
    of positive terms: at most one unit roundoff u = 2^-24 of the total per addition;
    a p below half an ulp of the running sum is dropped, within the same bound), and
    every move of the running maximum rescales it (a product with the hardware exp2,
    within 4 u); the halves meet in one more addition."""
    return max(1e-5, (-(-n_keys // 2) + 4 * -(-n_keys // kv_blk) + 2) * 2.0 ** -24)


def assert_dumps_equal(d: dict, od: dict, what="", n_keys=None, kv_blk=None):
    """Integer dumps bit-exact (A_qk, P codes, per-step P V sums, the running
    maximum's bits); l within 1e-5 of the oracle's binary64 sum, or within the
    binary32 summation bound l_rtol for long rows (n_keys and kv_blk given)."""
    assert np.array_equal(d["a_qk"], od["a_qk"]), what + " a_qk"
    assert np.array_equal(d["p_codes"], od["pcode"]), what + " P codes"
    assert np.array_equal(d["a_pv"], od["a_pv"]), what + " a_pv"
    assert np.array_equal(d["m"].view(np.uint32), od["m"].view(np.uint32)), what + " m"
    rtol = 1e-5 if n_keys is None else l_rtol(n_keys, kv_blk)
    err = float(np.max(np.abs(d["l"] - od["l"]) / od["l"]))
    print("%s: l max rel err %.3g (bound %.3g)" % (what, err, rtol))
    assert err <= rtol, what + " l"
