"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test names what it pins and why that is independent of the oracle's own
arithmetic (closed forms, invariants, exact high-precision arithmetic, library
routines, brute force).  CPU only.
"""
from decimal import Decimal, getcontext
from fractions import Fraction
import math
import os

import numpy as np
import pytest

from int4_quantized_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = synth.CONFIGS["tiny"]


def _f32_next_above(x: Decimal) -> np.float32:
    """Smallest binary32 strictly above the decimal x (exact decimal compare)."""
    f = np.float32(float(x))
    while not Decimal(float(f)) > x:
        f = np.nextafter(f, np.float32(np.inf))
    while Decimal(float(np.nextafter(f, np.float32(-np.inf)))) > x:
        f = np.nextafter(f, np.float32(-np.inf))
    return f


# --- P code (Key design 2) -------------------------------------------------------

def test_p_thresholds_match_50_digit_decimal(orc):
    """The 15 level thresholds equal log2(k - 1/2) computed with 50-digit decimal
    arithmetic (independent of the oracle's x87 log2l)."""
    getcontext().prec = 50
    ln2 = Decimal(2).ln()
    want = [np.nextafter(np.float32(-1.0), np.float32(0.0))]
    for k in range(2, 16):
        want.append(_f32_next_above((Decimal(k) - Decimal("0.5")).ln() / ln2))
    got = orc.p_thresholds()
    assert np.array_equal(np.array(want, np.float32).view(np.uint32), got.view(np.uint32))


def test_p_level_bruteforce_all_floats(orc):
    """Every binary32 y with |y| in [2^-10, 4]: the threshold-decided level equals
    round-half-even(exp2(y)) from libm's binary64 exp2 (brute force)."""
    bad, first = orc.p_level_bruteforce(2.0 ** -10, 4.0)
    assert bad == 0, "first mismatch at y=%r" % first
    # |y| < 2^-10: 2^y is within 0.07% of 1, so the level is 1; far below -1 it is
    # 0; at and above log2(15.5) it saturates at 15.
    small = np.float32(np.linspace(-2.0 ** -10, 2.0 ** -10, 10001))
    assert np.all(orc.p_levels(small) == 1)
    assert np.all(orc.p_levels(np.float32([-1.0, -1.5, -30.0, -1e30])) == 0)
    assert np.all(orc.p_levels(np.float32([np.log2(15.5) + 1e-6, 7.0, 1e30])) == 15)


def test_p_code_golden_endpoints(orc):
    """Worked values of the fixed-scale/zero-point map (golden fixture)."""
    rows = []
    with open(os.path.join(GOLDEN, "p_rectify_endpoints.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                expr, code = line.split(";")
                rows.append((sum(Fraction(t) for t in expr.strip().split("+")), int(code)))
    getcontext().prec = 50
    ln2 = Decimal(2).ln()
    for P, code in rows:
        x = 15 * P
        # exact tie 15 P = 1/2 is reached by y' = -1 exactly
        y = np.float32(-1.0) if x == Fraction(1, 2) else np.float32(
            float((Decimal(x.numerator) / Decimal(x.denominator)).ln() / ln2))
        assert int(orc.p_levels(np.array([y]))[0]) - 8 == code, (P, code)


def test_p_levels_monotone_and_complete(orc):
    y = np.float32(np.linspace(-3.0, 4.2, 200001))
    r = orc.p_levels(y).astype(int)
    assert np.all(np.diff(r) >= 0)
    assert set(r.tolist()) == set(range(16))


# --- RoPE and rotation (Key design 1) --------------------------------------------

def _one_head(cfg, x):
    N = synth.n_tokens(cfg)
    return x.reshape(1, 1, N, cfg["D"])


def _shape1(cfg):
    s = dict(cfg)
    s["B"], s["H"] = 1, 1
    return s


def test_rope_relative_position_property(orc):
    """<RoPE(q, p), RoPE(k, p')> depends only on p - p' per axis (textbook RoPE)."""
    cfg = _shape1(synth.custom(1, 1, 5, 6, 7, 64, 24, 20, 20, 16, 16))
    N, D = synth.n_tokens(cfg), 64
    tab = orc.rope_table(cfg, orc.ROT_NONE, f64=True)
    rng = np.random.default_rng(7)
    qv, kv = rng.standard_normal(D), rng.standard_normal(D)
    tok = lambda f, y, x: (f * cfg["Hs"] + y) * cfg["Ws"] + x
    X = np.zeros((N, D))
    X[:] = qv
    Rq = orc.rope_rotate(cfg, orc.ROT_NONE, tab, _one_head(cfg, X))[0, 0]
    X[:] = kv
    Rk = orc.rope_rotate(cfg, orc.ROT_NONE, tab, _one_head(cfg, X))[0, 0]
    for (p1, p2, dd) in [((0, 0, 0), (1, 2, 3), (2, 1, 1)), ((1, 3, 2), (0, 0, 6), (3, 2, 0)),
                         ((4, 5, 6), (4, 5, 6), (-4, -5, -6))]:
        a = Rq[tok(*p1)] @ Rk[tok(*p2)]
        sh = lambda p: tuple(p[i] + dd[i] for i in range(3))
        b = Rq[tok(*sh(p1))] @ Rk[tok(*sh(p2))]
        assert abs(a - b) <= 1e-12 * (abs(a) + 1)
    # position (0,0,0) is the identity; norms are preserved everywhere
    assert np.allclose(Rq[0], qv, atol=0, rtol=0)
    assert np.allclose(np.linalg.norm(Rq, axis=1), np.linalg.norm(qv), rtol=1e-14)
    # a half-turn sanity value: theta_{j,0} = 1, so frame position 1 rotates the
    # first frame pair by exactly 1 radian
    c, s = math.cos(1.0), math.sin(1.0)
    want = np.array([qv[0] * c - qv[1] * s, qv[0] * s + qv[1] * c])
    assert np.allclose(Rq[tok(1, 0, 0)][:2], want, rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("rot", [1, 2])
def test_rotation_is_orthogonal_block_2x2(orc, rot):
    """At position 0 RoPE is the identity, so the pipeline applies R itself:
    R R^T = I (the pages require R in O(D)), and R only mixes 2x2 channel pairs --
    (2i, 2i+1) for Interleaved, (o+i, o+Dj/2+i) -> (o+2i, o+2i+1) for Half."""
    D, Df, Dh, Dw = 64, 24, 20, 20
    cfg = synth.custom(1, D, 1, 1, 1, D, Df, Dh, Dw, 1, 1)  # one token per head
    tab = orc.rope_table(cfg, rot, f64=True)
    E = np.eye(D).reshape(1, D, 1, D)
    R = orc.rope_rotate(cfg, rot, tab, E)[0, :, 0, :].T  # column j = R e_j
    assert np.max(np.abs(R @ R.T - np.eye(D))) <= 1e-15
    assert np.max(np.abs(R - np.eye(D))) > 0.1
    nz = np.abs(R) > 1e-12
    assert np.all(nz.sum(axis=0) == 2) and np.all(nz.sum(axis=1) == 2)
    for o, dj in [(0, Df), (Df, Dh), (Df + Dh, Dw)]:
        for i in range(dj // 2):
            if rot == 1:
                src, dst = [o + 2 * i, o + 2 * i + 1], [o + 2 * i, o + 2 * i + 1]
            else:
                src, dst = [o + i, o + dj // 2 + i], [o + 2 * i, o + 2 * i + 1]
            assert np.allclose(np.abs(R[np.ix_(dst, src)]), 1 / np.sqrt(2), rtol=1e-15)


@pytest.mark.parametrize("rot", [1, 2])
def test_qk_invariance_under_rotation(orc, rot):
    """Q K^T = (Q R)(K R)^T for orthogonal R (pages: Key design 1), in binary64."""
    cfg = dict(TINY)
    q, k, _ = synth.make_inputs(cfg)
    q, k = q.astype(np.float64), k.astype(np.float64)
    t0 = orc.rope_table(cfg, 0, f64=True)
    tr = orc.rope_table(cfg, rot, f64=True)
    for h in range(cfg["H"]):
        a = orc.rope_rotate(cfg, 0, t0, q)[0, h] @ orc.rope_rotate(cfg, 0, t0, k)[0, h].T
        b = orc.rope_rotate(cfg, rot, tr, q)[0, h] @ orc.rope_rotate(cfg, rot, tr, k)[0, h].T
        assert np.max(np.abs(a - b)) <= 1e-13 * np.max(np.abs(a))


def test_interleaved_fused_equals_rotate_after_rope(orc):
    """Fused table (alpha, beta) == H2 applied after plain RoPE (M' = R M)."""
    cfg = dict(TINY)
    q, _, _ = synth.make_inputs(cfg)
    t0 = orc.rope_table(cfg, 0, f64=True)
    t1 = orc.rope_table(cfg, 1, f64=True)
    x = q.astype(np.float64)
    plain = orc.rope_rotate(cfg, 0, t0, x)
    fused = orc.rope_rotate(cfg, 1, t1, x)
    seq = np.empty_like(plain)
    seq[..., 0::2] = (plain[..., 0::2] + plain[..., 1::2]) / np.sqrt(2)
    seq[..., 1::2] = (plain[..., 0::2] - plain[..., 1::2]) / np.sqrt(2)
    assert np.max(np.abs(fused - seq)) <= 1e-14 * np.max(np.abs(seq))
    # binary32 spec path: same up to a few ulp (not bit-identical by design)
    f32 = orc.rope_rotate(cfg, 1, orc.rope_table(cfg, 1), q.astype(np.float32))
    rel = np.abs(f32 - seq) / (np.abs(seq) + 1e-30)
    assert np.median(rel) < 1e-6 and np.max(np.abs(f32 - seq)) < 1e-5 * np.max(np.abs(seq))


def test_rope_table_closed_form(orc):
    """Table entries equal cos/sin(pos * 10000^(-2i/Dj)) (plain) and the H2-folded
    (cos+sin)/sqrt2, (cos-sin)/sqrt2 (Interleaved), rounded to binary32."""
    cfg = dict(TINY)
    t0, t1 = orc.rope_table(cfg, 0), orc.rope_table(cfg, 1)
    # width axis (third block): Ws=4 positions x Dw/2=10 pairs
    off = 2 * (cfg["F"] * 12 + cfg["Hs"] * 10)
    p, i = 3, 7
    ang = p * 10000.0 ** (-2.0 * i / 20)
    e = off + 2 * (p * 10 + i)
    assert t0[e] == np.float32(math.cos(ang)) and t0[e + 1] == np.float32(math.sin(ang))
    assert abs(t1[e] - (math.cos(ang) + math.sin(ang)) / math.sqrt(2)) <= 6e-8
    assert abs(t1[e + 1] - (math.cos(ang) - math.sin(ang)) / math.sqrt(2)) <= 6e-8


# --- quantisation ---------------------------------------------------------------

@pytest.mark.parametrize("rot,qb,kv", [(1, 16, 16), (2, 16, 16), (2, 1, 16), (1, 2, 32), (2, 16, 256)])
def test_quantize_invariants(orc, rot, qb, kv):
    """qb = 1 is the per-token Q/K quantiser (paper.gecl.asia analysis, "Key
    Insight"); kv = 256 a column-sum block longer than the sequence."""
    cfg = dict(TINY, qk_blk=qb, kv_blk=kv)
    q, k, v = synth.make_inputs(cfg)
    tab = orc.rope_table(cfg, rot)
    z = orc.quantize(cfg, rot, tab, q, k, v, smooth_k=True, diag=True)
    N, D, qb = synth.n_tokens(cfg), cfg["D"], cfg["qk_blk"]
    # q_rot is the rotation of q (binary32 pipeline)
    assert np.array_equal(z["q_rot"], orc.rope_rotate(cfg, rot, tab, q))
    # smoothing: mu is the per-channel mean of the rotated K (binary64 mean)
    mu = z["k_rot"].astype(np.float64).mean(axis=2)
    assert np.max(np.abs(z["k_mu"] - mu)) <= 1e-6 * np.max(np.abs(mu)) + 1e-12
    ks_in = (z["k_rot"] - z["k_mu"][:, :, None, :]).astype(np.float32)
    for name, x, c, sc in [("q", z["q_rot"], z["qc"], z["qs"]), ("k", ks_in, z["kc"], z["ks"])]:
        for b in range(sc.shape[2]):
            blk = x[0, :, b * qb:(b + 1) * qb]
            cb = c[0, :, b * qb:(b + 1) * qb].astype(np.float64)
            s = sc[0, :, b]
            amax = np.abs(blk).reshape(cfg["H"], -1).max(axis=1)
            assert np.allclose(s, amax / 7, rtol=1e-7)
            err = np.abs(blk - s[:, None, None] * cb)
            assert np.all(err <= s[:, None, None] / 2 * (1 + 2 ** -20)), name
            # the block maximum lands on +-7
            for h in range(cfg["H"]):
                idx = np.unravel_index(np.argmax(np.abs(blk[h])), blk[h].shape)
                assert abs(cb[h][idx]) == 7
    vq = z["vc"].astype(np.float64) * z["vs"][:, :, None, :]
    assert np.all(np.abs(vq - v) <= z["vs"][:, :, None, :] / 2 * (1 + 2 ** -20))
    # column sums of the V codes per kv block (brute force)
    kb = cfg["kv_blk"]
    for sblk in range(z["vcol"].shape[2]):
        assert np.array_equal(z["vcol"][:, :, sblk], z["vc"][:, :, sblk * kb:(sblk + 1) * kb].sum(axis=2))
    assert z["qc"].min() >= -7 and z["qc"].max() <= 7


def test_quantize_zero_block_and_v_scale(orc):
    cfg = dict(TINY)
    q, k, v = synth.make_inputs(cfg)
    q[0, 0, :16] = 0
    v[0, 1, :, 5] = 0
    z = orc.quantize(cfg, 1, orc.rope_table(cfg, 1), q, k, v)
    assert z["qs"][0, 0, 0] == 0 and np.all(z["qc"][0, 0, :16] == 0)
    assert z["vs"][0, 1, 5] == 0 and np.all(z["vc"][0, 1, :, 5] == 0)


# --- quantised attention --------------------------------------------------------

def _ints(rng, shape):
    return rng.integers(-7, 8, size=shape).astype(np.int8)


def test_attention_integer_accumulators_bruteforce(orc):
    cfg = dict(TINY)
    rng = np.random.default_rng(3)
    B, H, N, D = 1, 2, 32, 64
    z = dict(qc=_ints(rng, (B, H, N, D)), kc=_ints(rng, (B, H, N, D)), vc=_ints(rng, (B, H, N, D)),
             qs=rng.uniform(0.05, 0.5, (B, H, 2)).astype(np.float32),
             ks=rng.uniform(0.05, 0.5, (B, H, 2)).astype(np.float32),
             vs=rng.uniform(0.1, 1, (B, H, D)).astype(np.float32))
    r = orc.attention(cfg, z, dumps=True)
    qc, kc, vc = (z[n].astype(np.int64) for n in ("qc", "kc", "vc"))
    want = np.einsum("bhid,bhjd->bhij", qc, kc).reshape(B * H * N, N)
    assert np.array_equal(r["a_qk"], want)
    # per-step P.V accumulators: sum_j (code_j + 8) * vc_jd over the step (brute force)
    lev = r["pcode"].astype(np.int64) + 8
    for row in range(B * H * N):
        bh = row // N
        for st in range(2):
            sl = slice(16 * st, 16 * st + 16)
            assert np.array_equal(r["a_pv"][row, st], lev[row, sl] @ vc.reshape(B * H, N, D)[bh, sl])
    assert r["pcode"].min() >= -8 and r["pcode"].max() <= 7


def _dequant_v(z):
    return z["vc"].astype(np.float64) * z["vs"][:, :, None, :].astype(np.float64)


def test_attention_single_token_returns_value(orc):
    """N = 1: P = 1 -> code 7, so the output is the dequantised V row (closed form)."""
    cfg = synth.custom(1, 3, 1, 1, 1, 64, 24, 20, 20, 16, 16)
    q, k, v = synth.make_inputs(cfg)
    z = orc.quantize(cfg, 2, orc.rope_table(cfg, 2), q, k, v)
    r = orc.attention(cfg, z, dumps=True)
    assert np.all(r["pcode"] == 7)
    assert np.allclose(r["out"], _dequant_v(z).reshape(3, 64), rtol=1e-6, atol=0)


@pytest.mark.parametrize("kv", [16, 32])
def test_attention_zero_query_is_mean_of_values(orc, kv):
    """Q = 0: every score is 0, every P is 1 (code 7): output = mean of dequantised V."""
    cfg = dict(TINY, kv_blk=kv)
    q, k, v = synth.make_inputs(cfg)
    q[:] = 0
    z = orc.quantize(cfg, 1, orc.rope_table(cfg, 1), q, k, v)
    r = orc.attention(cfg, z, dumps=True)
    assert np.all(r["pcode"] == 7)
    want = np.repeat(_dequant_v(z).mean(axis=2), 32, axis=1).reshape(-1, 64)
    assert np.allclose(r["out"], want, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("kv", [16, 32, 64])
def test_attention_within_rounding_bound_of_exact_softmax(orc, kv):
    """Lossless Q/K/V codes: the only approximation left is rounding 15 P to an
    integer level (error <= 1/2 per key, with running-max rescales <= 1), so the
    output is within 1/2 sum_j |v_j| / l of textbook softmax attention on the
    dequantised scores (numpy softmax, binary64)."""
    rng = np.random.default_rng(11)
    B, H, F, Hs, Ws, D = 1, 2, 2, 4, 8, 64
    cfg = synth.custom(B, H, F, Hs, Ws, D, 24, 20, 20, 16, kv)
    N = F * Hs * Ws
    z = dict(qc=_ints(rng, (B, H, N, D)), kc=_ints(rng, (B, H, N, D)), vc=_ints(rng, (B, H, N, D)),
             qs=rng.uniform(0.02, 0.1, (B, H, N // 16)).astype(np.float32),
             ks=rng.uniform(0.02, 0.1, (B, H, N // 16)).astype(np.float32),
             vs=rng.uniform(0.5, 1, (B, H, D)).astype(np.float32))
    r = orc.attention(cfg, z, dumps=True)
    V = _dequant_v(z).reshape(B * H, N, D)
    sq = np.repeat(z["qs"].astype(np.float64), 16, axis=2).reshape(B * H, N)
    sk = np.repeat(z["ks"].astype(np.float64), 16, axis=2).reshape(B * H, N)
    A = np.einsum("hid,hjd->hij", z["qc"].reshape(B * H, N, D).astype(np.float64),
                  z["kc"].reshape(B * H, N, D).astype(np.float64))
    S = A * sq[:, :, None] * sk[:, None, :] / math.sqrt(D)
    P = np.exp(S - S.max(axis=2, keepdims=True))
    exact = np.einsum("hij,hjd->hid", P / P.sum(axis=2, keepdims=True), V).reshape(-1, D)
    # the normaliser of the definition, 15 sum_j P_ij (P against the row maximum),
    # computed here rather than read back from the oracle
    l_def = 15.0 * P.sum(axis=2).reshape(-1)
    bound = 0.5 * np.abs(V).sum(axis=1)[:, None, :].repeat(N, axis=1).reshape(-1, D) / l_def[:, None]
    assert np.all(np.abs(r["out"] - exact) <= bound * (1 + 1e-5) + 1e-9)
    cos = np.sum(r["out"] * exact) / np.linalg.norm(r["out"]) / np.linalg.norm(exact)
    assert cos > 0.95


def _definition_attention(z, N, D, qk_blk, kv):
    """The method's quantised attention written out in binary64 numpy, from the
    definition rather than from the oracle's steps (papernotes.org note, Key design
    2: P = exp(S - m) with m the running row maximum, level round(15 P), zero point
    folded; the normaliser is the plain softmax sum of the unquantised P).
    Returns (level, weight, l, x) per [head, row, key]: the exact level of 15 P
    against the running maximum of its kv-step, the rescale 2^(m_s - m) of its
    step, the normaliser 15 sum_j 2^(S_j - max S) and the unrounded 15 P."""
    BH = z["qc"].shape[0] * z["qc"].shape[1]
    sq = np.repeat(z["qs"].astype(np.float64), qk_blk, axis=2).reshape(BH, -1)[:, :N]
    sk = np.repeat(z["ks"].astype(np.float64), qk_blk, axis=2).reshape(BH, -1)[:, :N]
    A = np.einsum("hid,hjd->hij", z["qc"].reshape(BH, N, D).astype(np.int64),
                  z["kc"].reshape(BH, N, D).astype(np.int64)).astype(np.float64)
    S2 = A * sq[:, :, None] * sk[:, None, :] * (math.log2(math.e) / math.sqrt(D))  # log2 units
    S = -(-N // kv)
    step_max = np.stack([S2[:, :, s * kv:(s + 1) * kv].max(axis=2) for s in range(S)], axis=2)
    m_run = np.maximum.accumulate(step_max, axis=2)           # running maximum after each step
    m_key = np.repeat(m_run, kv, axis=2)[:, :, :N]            # the maximum a key's level sees
    x = 15.0 * np.exp2(S2 - m_key)                             # 15 P against the running maximum
    level = np.minimum(np.rint(x), 15.0)                       # numpy rint: round half to even
    weight = np.exp2(m_key - m_run[:, :, -1:])                 # later rescales of the key's step
    l = 15.0 * np.exp2(S2 - S2.max(axis=2, keepdims=True)).sum(axis=2)
    return level, weight, l, x


@pytest.mark.parametrize("kv,lo,hi,qb", [(16, 0.5, 1.0, 16), (64, 0.5, 1.0, 16), (16, 0.15, 0.4, 16),
                                         (64, 0.15, 0.4, 16), (256, 0.15, 0.4, 16), (64, 0.15, 0.4, 1),
                                         (256, 0.5, 1.0, 1)])
def test_normaliser_codes_and_output_against_definition(orc, kv, lo, hi, qb):
    """Peaked scores (lossless codes, Q/K scales in [lo, hi]: score spreads of 1.5 to
    10 nat, so most levels are 0 while 15 P is not): the oracle's normaliser l, its
    P codes and its output against the definition evaluated here in binary64
    (_definition_attention).  l must be the sum of the unquantised 15 P (a sum of
    the levels, or a missing rescale, is off by far more than the 5e-5 allowed for
    the binary32 score pipeline).  Codes must equal round(15 P) against the running
    maximum except for keys whose 15 P lies within 1e-4 (relative) of a rounding
    boundary, where the binary32 exponent may fall on either side; each such key
    widens the output bound by its |v| weight.  qb: tokens per Q/K scale (1: the
    per-token scales of the paper.gecl.asia analysis, "Key Insight")."""
    rng = np.random.default_rng(23 + kv + qb)
    B, H, F, Hs, Ws, D = 1, 2, 4, 8, 8, 64
    cfg = synth.custom(B, H, F, Hs, Ws, D, 24, 20, 20, qb, kv)
    N = F * Hs * Ws
    z = dict(qc=_ints(rng, (B, H, N, D)), kc=_ints(rng, (B, H, N, D)), vc=_ints(rng, (B, H, N, D)),
             qs=rng.uniform(lo, hi, (B, H, N // qb)).astype(np.float32),
             ks=rng.uniform(lo, hi, (B, H, N // qb)).astype(np.float32),
             vs=rng.uniform(0.5, 1, (B, H, D)).astype(np.float32))
    r = orc.attention(cfg, z, dumps=True)
    level, weight, l, x = _definition_attention(z, N, D, qb, kv)
    level, weight, x = (a.reshape(B * H * N, N) for a in (level, weight, x))
    l = l.reshape(-1)
    # normaliser
    assert np.allclose(r["l"], l, rtol=5e-5, atol=0)
    # codes: exact except at rounding boundaries
    ambiguous = np.abs(x - (np.floor(x) + 0.5)) <= 1e-4 * np.maximum(x, 0.5)
    got = r["pcode"].astype(np.int64) + 8
    assert np.array_equal(got[~ambiguous], level[~ambiguous])
    assert np.all(np.abs(got - level) <= 1)
    assert ambiguous.mean() < 1e-3
    # output: sum_j level_j weight_j sv vc_j / l, from the definition
    V = _dequant_v(z).reshape(B * H, N, D)
    Vrow = np.repeat(V, N, axis=0)                            # [rows, keys, D] of each row's head
    want = np.einsum("rj,rjd->rd", level * weight, Vrow) / l[:, None]
    slack = np.einsum("rj,rjd->rd", ambiguous * weight, np.abs(Vrow)) / l[:, None]
    scale = np.einsum("rj,rjd->rd", level * weight, np.abs(Vrow)) / l[:, None]
    assert np.all(np.abs(r["out"] - want) <= slack + 1e-4 * scale + 1e-12)
    # the levels are far from the unquantised P here: summing them instead of 15 P
    # would move l of some rows by much more than the tolerance above
    assert np.max(np.abs((level * weight).sum(axis=1) - l) / l) > 1e-2


def test_attention_key_permutation_within_step_and_v_scaling(orc):
    """Invariants: permuting keys inside one online-softmax step leaves the output
    unchanged; scaling V by 2 doubles it exactly."""
    cfg = dict(TINY)
    q, k, v = synth.make_inputs(cfg)
    tab = orc.rope_table(cfg, 1)
    z = orc.quantize(cfg, 1, tab, q, k, v)
    base = orc.attention(cfg, z)["out"]
    perm = np.concatenate([np.random.default_rng(1).permutation(16), 16 + np.arange(16)])
    z2 = dict(z)
    for n in ("kc", "vc"):
        z2[n] = z[n][:, :, perm]
    assert np.allclose(orc.attention(cfg, z2)["out"], base, rtol=1e-12, atol=1e-14)
    z3 = orc.quantize(cfg, 1, tab, q, k, 2 * v)
    assert np.array_equal(orc.attention(cfg, z3)["out"], 2 * base)


def test_fallback_oracle_close_to_exact(orc):
    """The fallback oracle is exact attention on binary16-rounded RoPE'd Q, K:
    within binary16 rounding of the binary64 reference."""
    cfg = dict(TINY)
    q, k, v = synth.make_inputs(cfg)
    q, k = q / 8, k / 8
    fb = orc.fallback_attention(cfg, orc.rope_table(cfg, 0), q, k, v)
    ex = orc.exact_attention(cfg, q, k, v)
    assert np.max(np.abs(fb - ex)) < 5e-3 * np.max(np.abs(ex))


def test_f16_rounding_matches_numpy(orc):
    """binary16 round-half-even used by the fallback oracle == numpy's cast."""
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s
                        for s in (1e-8, 1e-6, 1e-4, 1, 100, 6e4)] +
                       [np.float32([0.0, -0.0, 65504, 65520, 1e9, -1e9, 2 ** -24, 2 ** -25, 3 * 2 ** -26])])
    assert np.array_equal(orc.f32_to_f16_bits(x), x.astype(np.float16).view(np.uint16))


def test_report_cosine_vs_exact_tiny(orc, capsys):
    """Reported (no threshold -- the pages give none): cosine / rel-L2 of the
    quantised output against exact attention on the tiny config."""
    cfg = dict(TINY)
    q, k, v = synth.make_inputs(cfg)
    ex = orc.exact_attention(cfg, q, k, v)
    for rot in (0, 1, 2):
        z = orc.quantize(cfg, rot, orc.rope_table(cfg, rot), q, k, v)
        o = orc.attention(cfg, z)["out"]
        cos = float(np.sum(o * ex) / np.linalg.norm(o) / np.linalg.norm(ex))
        rel = float(np.linalg.norm(o - ex) / np.linalg.norm(ex))
        print("tiny rot=%d cosine=%.4f relL2=%.4f" % (rot, cos, rel))
        assert cos > 0.5


# ---- ablation variants ------------------------------------------------------------

def test_full_rotation_is_the_orthonormal_hadamard_after_rope(orc):
    """rot 3 (Full): the butterfly transform after plain RoPE equals the dense
    Sylvester-Hadamard product H_D / sqrt(D) applied to the RoPE output (a different
    algorithm: scipy's matrix, one binary64 matmul), and keeps the norm."""
    from scipy.linalg import hadamard
    for D, split in [(64, (24, 20, 20)), (128, (44, 42, 42))]:
        cfg = synth.custom(1, 2, 2, 3, 4, D, *split, 16, 16, recipe="tiny")
        q, _, _ = synth.make_inputs(cfg)
        tab = orc.rope_table(cfg, 0, f64=True)
        x = q.astype(np.float64)
        plain = orc.rope_rotate(cfg, 0, tab, x)
        full = orc.rope_rotate(cfg, 3, tab, x)
        Hn = hadamard(D).astype(np.float64) / np.sqrt(D)
        want = plain @ Hn.T
        assert np.max(np.abs(full - want)) <= 1e-12 * np.max(np.abs(want))
        assert np.allclose(np.linalg.norm(full, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
        # binary32 path: the same transform within a few binary32 roundings per stage
        full32 = orc.rope_rotate(cfg, 3, orc.rope_table(cfg, 0), q)
        assert np.max(np.abs(full32 - want)) <= 16 * 2.0**-24 * np.sqrt(D) * np.max(np.abs(x))


def test_full_rotation_keeps_qk(orc):
    """Q K^T is unchanged by the Full rotation (orthogonal), in binary64."""
    cfg = dict(TINY)
    q, k, _ = synth.make_inputs(cfg)
    q, k = q.astype(np.float64), k.astype(np.float64)
    t0 = orc.rope_table(cfg, 0, f64=True)
    for h in range(cfg["H"]):
        a = orc.rope_rotate(cfg, 0, t0, q)[0, h] @ orc.rope_rotate(cfg, 0, t0, k)[0, h].T
        b = orc.rope_rotate(cfg, 3, t0, q)[0, h] @ orc.rope_rotate(cfg, 3, t0, k)[0, h].T
        assert np.max(np.abs(a - b)) <= 1e-13 * np.max(np.abs(a))


def test_symmetric_p_single_token_and_zero_query(orc):
    """Symmetric baseline (pmax 7): with one key, or with Q = 0, every P is 1, so
    every code is round(7 * 1) = 7 with no zero point, and the output is the
    dequantised V row / the mean of the dequantised V rows (closed form)."""
    cfg = synth.custom(1, 3, 1, 1, 1, 64, 24, 20, 20, 16, 16)
    q, k, v = synth.make_inputs(cfg)
    z = orc.quantize(cfg, 2, orc.rope_table(cfg, 2), q, k, v)
    r = orc.attention(cfg, z, dumps=True, pmax=7)
    assert np.all(r["pcode"] == 7)
    assert np.allclose(r["out"], _dequant_v(z).reshape(3, 64), rtol=1e-6, atol=0)
    cfg = dict(TINY, kv_blk=16)
    q, k, v = synth.make_inputs(cfg)
    q[:] = 0
    z = orc.quantize(cfg, 1, orc.rope_table(cfg, 1), q, k, v)
    r = orc.attention(cfg, z, dumps=True, pmax=7)
    assert np.all(r["pcode"] == 7)
    want = np.repeat(_dequant_v(z).mean(axis=2), 32, axis=1).reshape(-1, 64)
    assert np.allclose(r["out"], want, rtol=1e-6, atol=1e-7)


def test_symmetric_p_codes_are_round_7p(orc):
    """Symmetric baseline: code = round-half-even(7 P) with P = 2^(t - m_s), m_s the
    running maximum (binary64 recomputation from the dumped integer scores; ties and
    near-ties, where binary32 and binary64 may decide differently, are skipped)."""
    cfg = dict(TINY, kv_blk=16)
    q, k, v = synth.make_inputs(cfg)
    z = orc.quantize(cfg, 2, orc.rope_table(cfg, 2), q, k, v)
    r = orc.attention(cfg, z, dumps=True, pmax=7)
    N, D = 32, 64
    C0 = np.float32(orc.c0(D))
    checked = 0
    for row in range(2 * N):
        bh, i = divmod(row, N)
        sq = z["qs"][0, bh, i // 16]
        m = -np.inf
        for s0 in range(0, N, 16):
            cs = np.float32(np.float32(sq) * z["ks"][0, bh, np.arange(s0, s0 + 16) // 16]) * C0
            t = (r["a_qk"][row, s0:s0 + 16].astype(np.float32) * cs).astype(np.float32)
            m = max(m, float(t.max()))
            x = 7.0 * np.exp2(r["a_qk"][row, s0:s0 + 16].astype(np.float64) * cs.astype(np.float64) - m)
            frac = np.abs(x - np.floor(x) - 0.5)
            ok = frac > 1e-5
            want = np.rint(x)
            assert np.array_equal(r["pcode"][row, s0:s0 + 16][ok], want[ok].astype(np.int8))
            checked += int(ok.sum())
    assert checked > 0.99 * 2 * N * N
    assert r["pcode"].min() >= 0 and r["pcode"].max() <= 7


# --- block-causal attention -------------------------------------------------------
# Query token i sees key j iff j // c <= i // c (c = 1 token-causal, c = Hs*Ws
# frame-causal, c = 0 bidirectional).  The pins below hold it to the bidirectional
# oracle on the visible prefix (pinned above) and to a masked binary64 softmax.

def _causal_case(orc, seed=21):
    cfg = synth.custom(1, 2, 3, 4, 6, 64, 24, 20, 20, 16, 16)   # N = 72: 4.5 steps
    q, k, v = synth.make_inputs(cfg, seed=seed)
    z = orc.quantize(cfg, 2, orc.rope_table(cfg, 2), q, k, v)
    return cfg, q, k, v, z


def _prefix(z, n, qk_blk):
    nb = -(-n // qk_blk)
    return dict(qc=z["qc"][:, :, :n], kc=z["kc"][:, :, :n], vc=z["vc"][:, :, :n],
                qs=z["qs"][:, :, :nb], ks=z["ks"][:, :, :nb], vs=z["vs"])


@pytest.mark.parametrize("cb", [1, 5, 16, 24])
def test_causal_row_equals_bidirectional_on_its_prefix(orc, cb):
    """Row i of block-causal attention == bidirectional attention over the first
    key_limit(i) tokens (codes and scales sliced, nothing recomputed), bit for bit,
    dumps included; the entries of keys the row does not see stay zero."""
    cfg, _, _, _, z = _causal_case(orc)
    N = orc.n_tokens(cfg)
    rows = np.array([0, 3, cb - 1, cb, 17, 40, 47, 48, N - 1], np.int64)
    rows = np.unique(np.concatenate([rows, rows + N]))       # both heads
    r = orc.attention(cfg, z, rows=rows, dumps=True, causal_block=cb)
    for idx, row in enumerate(rows):
        h, i = divmod(int(row), N)
        lim = int(orc.key_limit(i, N, cb))
        sub = synth.custom(1, 2, 1, 1, lim, 64, 24, 20, 20, 16, 16)
        p = orc.attention(sub, _prefix(z, lim, 16), rows=np.array([h * lim + i]), dumps=True)
        assert np.array_equal(r["out"][idx], p["out"][0]), (cb, row)
        assert np.array_equal(r["a_qk"][idx, :lim], p["a_qk"][0])
        assert np.array_equal(r["pcode"][idx, :lim], p["pcode"][0])
        assert r["m"][idx] == p["m"][0] and r["l"][idx] == p["l"][0]
        sp = p["a_pv"].shape[1]
        assert np.array_equal(r["a_pv"][idx, :sp], p["a_pv"][0])
        assert not r["a_qk"][idx, lim:].any() and not r["pcode"][idx, lim:].any()
        assert not r["a_pv"][idx, sp:].any()


def test_causal_block_at_least_n_is_bidirectional(orc):
    cfg, q, k, v, z = _causal_case(orc)
    N = orc.n_tokens(cfg)
    base = orc.attention(cfg, z, dumps=True)
    for cb in (N, N + 7, 10 ** 6):
        r = orc.attention(cfg, z, dumps=True, causal_block=cb)
        for key in ("out", "a_qk", "pcode", "a_pv", "m", "l"):
            assert np.array_equal(r[key], base[key]), (cb, key)
    assert np.array_equal(orc.exact_attention(cfg, q, k, v, causal_block=N),
                          orc.exact_attention(cfg, q, k, v))


@pytest.mark.parametrize("cb", [1, 7, 24])
def test_causal_exact_equals_masked_softmax(orc, cb):
    """The binary64 exact oracle with a causal block == textbook masked softmax of
    the RoPE'd scores (numpy, binary64): -inf where j // c > i // c."""
    cfg, q, k, v, _ = _causal_case(orc)
    B, H, N, D = 1, 2, orc.n_tokens(cfg), 64
    tab = orc.rope_table(cfg, 0, f64=True)
    qr = orc.rope_rotate(cfg, 0, tab, q.astype(np.float64).reshape(B, H, N, D)).reshape(H, N, D)
    kr = orc.rope_rotate(cfg, 0, tab, k.astype(np.float64).reshape(B, H, N, D)).reshape(H, N, D)
    S = np.einsum("hid,hjd->hij", qr, kr) / math.sqrt(D)
    i = np.arange(N)
    S[:, (i[None, :] // cb) > (i[:, None] // cb)] = -np.inf
    P = np.exp(S - S.max(axis=2, keepdims=True))
    want = np.einsum("hij,hjd->hid", P / P.sum(axis=2, keepdims=True),
                     v.astype(np.float64).reshape(H, N, D)).reshape(-1, D)
    got = orc.exact_attention(cfg, q, k, v, causal_block=cb)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12)
    # row 0 under token-causal attention sees only itself: its own value row
    if cb == 1:
        assert np.allclose(got[0], v.reshape(H, N, D)[0, 0], rtol=1e-12, atol=0)


def test_causal_quantised_and_fallback_close_to_exact(orc):
    """Frame-causal: the quantised oracle (Half rotation) and the fallback oracle
    stay as close to exact masked attention as their bidirectional forms do."""
    cfg, q, k, v, z = _causal_case(orc)
    cb = 24
    ex = orc.exact_attention(cfg, q, k, v, causal_block=cb)
    qa = orc.attention(cfg, z, causal_block=cb)["out"]
    fb = orc.fallback_attention(cfg, orc.rope_table(cfg, 0), q / 8, k / 8, v, causal_block=cb)
    ex8 = orc.exact_attention(cfg, q / 8, k / 8, v, causal_block=cb)
    cosine = lambda a, b: np.sum(a * b) / np.linalg.norm(a) / np.linalg.norm(b)
    qb = orc.attention(cfg, z)["out"]
    cos_bi = cosine(qb, orc.exact_attention(cfg, q, k, v))
    assert cosine(qa, ex) > min(0.85, cos_bi - 0.05)
    assert np.max(np.abs(fb - ex8)) < 5e-3 * np.max(np.abs(ex8))
    # first-frame rows see only the first frame: they differ from bidirectional rows;
    # last-frame rows see every key: they equal them
    assert not np.allclose(qa[:24], qb[:24])
    assert np.array_equal(qa[48:72], qb[48:72])


# --- Q smoothing (mu_q subtracted from Q; the per-key term mu_q . K_j added back) ----

def _offset_q_case(orc, seed=5):
    """Wan-like heads whose queries share a large offset in the slow (last) RoPE
    pairs of each segment, where rotation by position is mild: the case Q smoothing
    is for."""
    cfg = synth.custom(1, 2, 3, 8, 10, 64, 24, 20, 20, 16, 16)
    q, k, v = synth.make_inputs(cfg, seed=seed)
    rng = np.random.default_rng(seed)
    off = np.zeros(64, np.float32)
    for o, w in ((0, 24), (24, 20), (44, 20)):
        off[o + w - 4:o + w] = rng.uniform(4, 8, 4) * rng.choice([-1, 1], 4)
    return cfg, (q + off).astype(np.float32), k, v


def test_q_smoothing_statistics(orc):
    """mu_q is the channel mean of the rotated Q, the Q codes quantise Q - mu_q, the
    K codes do not change, and k_bias_j = mu_q . (K_j - mu_k) (binary64 numpy)."""
    cfg, q, k, v = _offset_q_case(orc)
    tab = orc.rope_table(cfg, 2)
    z = orc.quantize(cfg, 2, tab, q, k, v, diag=True, smooth_q=True)
    z0 = orc.quantize(cfg, 2, tab, q, k, v)
    H, N, D = 2, orc.n_tokens(cfg), 64
    qr = z["q_rot"].astype(np.float64).reshape(H, N, D)
    mu = qr.mean(axis=1)
    assert np.allclose(z["q_mu"].reshape(H, D), mu, rtol=2e-7, atol=1e-7)
    assert np.abs(mu).max() > 1.0
    # Q codes: within half a step of Q - mu_q in every 16-token block
    x = (z["q_rot"] - z["q_mu"][:, :, None, :]).reshape(H, N // 16, 16, D)
    deq = z["qc"].reshape(H, N // 16, 16, D) * z["qs"].reshape(H, N // 16, 1, 1)
    assert np.all(np.abs(deq - x) <= 0.5 * z["qs"].reshape(H, N // 16, 1, 1) * (1 + 1e-5) + 1e-6)
    for key in ("kc", "ks", "vc", "vs"):
        assert np.array_equal(z[key], z0[key]), key
    kt = (z["k_rot"] - z["k_mu"][:, :, None, :]).astype(np.float32).astype(np.float64).reshape(H, N, D)
    want = np.einsum("hd,hnd->hn", z["q_mu"].reshape(H, D).astype(np.float64), kt)
    mag = np.einsum("hd,hnd->hn", np.abs(z["q_mu"].reshape(H, D)).astype(np.float64), np.abs(kt))
    assert np.all(np.abs(z["k_bias"].reshape(H, N) - want) <= 1e-6 * mag + 1e-30)


@pytest.mark.parametrize("kv", [16, 32])
def test_k_bias_attention_within_rounding_bound(orc, kv):
    """Lossless codes plus a per-key bias dS_j: the output is within the level
    rounding bound of textbook softmax of (A_ij sq_i sk_j + dS_j) / sqrt(D)
    (numpy, binary64); a transposed, unscaled or dropped bias fails it."""
    rng = np.random.default_rng(17)
    B, H, F, Hs, Ws, D = 1, 2, 2, 4, 8, 64
    cfg = synth.custom(B, H, F, Hs, Ws, D, 24, 20, 20, 16, kv)
    N = F * Hs * Ws
    z = dict(qc=_ints(rng, (B, H, N, D)), kc=_ints(rng, (B, H, N, D)), vc=_ints(rng, (B, H, N, D)),
             qs=rng.uniform(0.02, 0.1, (B, H, N // 16)).astype(np.float32),
             ks=rng.uniform(0.02, 0.1, (B, H, N // 16)).astype(np.float32),
             vs=rng.uniform(0.5, 1, (B, H, D)).astype(np.float32),
             k_bias=rng.normal(0, 12, (B, H, N)).astype(np.float32))
    r = orc.attention(cfg, z, dumps=True)
    V = _dequant_v(z).reshape(B * H, N, D)
    sq = np.repeat(z["qs"].astype(np.float64), 16, axis=2).reshape(B * H, N)
    sk = np.repeat(z["ks"].astype(np.float64), 16, axis=2).reshape(B * H, N)
    A = np.einsum("hid,hjd->hij", z["qc"].reshape(B * H, N, D).astype(np.float64),
                  z["kc"].reshape(B * H, N, D).astype(np.float64))
    S = (A * sq[:, :, None] * sk[:, None, :] + z["k_bias"].reshape(B * H, 1, N)) / math.sqrt(D)
    P = np.exp(S - S.max(axis=2, keepdims=True))
    exact = np.einsum("hij,hjd->hid", P / P.sum(axis=2, keepdims=True), V).reshape(-1, D)
    # the normaliser of the definition, 15 sum_j P_ij (P against the row maximum),
    # computed here rather than read back from the oracle
    l_def = 15.0 * P.sum(axis=2).reshape(-1)
    bound = 0.5 * np.abs(V).sum(axis=1)[:, None, :].repeat(N, axis=1).reshape(-1, D) / l_def[:, None]
    assert np.all(np.abs(r["out"] - exact) <= bound * (1 + 1e-5) + 1e-9)
    # the bias matters here: without it the output is far outside the bound
    z0 = dict(z)
    del z0["k_bias"]
    assert np.max(np.abs(orc.attention(cfg, z0)["out"] - exact) - bound) > 0.05


def test_q_smoothing_recovers_offset_queries(orc):
    """On queries with a shared offset, Q smoothing brings the quantised output
    closer to exact attention than quantising Q as it is."""
    cfg, q, k, v = _offset_q_case(orc)
    tab = orc.rope_table(cfg, 2)
    ex = orc.exact_attention(cfg, q, k, v)
    cos = lambda a: float(np.sum(a * ex) / np.linalg.norm(a) / np.linalg.norm(ex))
    plain = orc.attention(cfg, orc.quantize(cfg, 2, tab, q, k, v))["out"]
    smooth = orc.attention(cfg, orc.quantize(cfg, 2, tab, q, k, v, smooth_q=True))["out"]
    print("cosine vs exact: plain %.4f, Q smoothing %.4f" % (cos(plain), cos(smooth)))
    assert cos(smooth) > cos(plain) + 0.02


# --- variable-length batches (per-element valid lengths in the padded layout) --------

def _varlen_case(orc, lens, seed=31):
    cfg = synth.custom(3, 2, 3, 4, 6, 64, 24, 20, 20, 16, 16)   # N = 72, one frame = 24 tokens
    q, k, v = synth.make_inputs(cfg, seed=seed)
    for b, n in enumerate(lens):   # padding holds NaN: nothing may read it
        for x in (q, k, v):
            x[b, :, n:] = np.nan
    return cfg, q, k, v


@pytest.mark.parametrize("smooth_q", [False, True])
def test_varlen_equals_each_sequence_alone(orc, smooth_q):
    """Whole frames: batch element b of a variable-length batch == the plain oracle
    on that element alone with F = seq_lens[b] / (Hs Ws) frames (same positions),
    codes, scales, sums, k_bias and the attention of every row; padding codes 0."""
    lens = [72, 48, 24]
    cfg, q, k, v = _varlen_case(orc, lens)
    tab = orc.rope_table(cfg, 2)
    z = orc.quantize(cfg, 2, tab, q, k, v, smooth_q=smooth_q, seq_lens=lens)
    N = 72
    o = orc.attention(cfg, z, rows=np.array([(b * 2 + h) * N + i for b in range(3) for h in range(2)
                                             for i in range(lens[b])]), dumps=True)
    at = 0
    for b, n in enumerate(lens):
        sub = synth.custom(1, 2, n // 24, 4, 6, 64, 24, 20, 20, 16, 16)
        zs = orc.quantize(sub, 2, orc.rope_table(sub, 2), q[b:b + 1, :, :n], k[b:b + 1, :, :n],
                          v[b:b + 1, :, :n], smooth_q=smooth_q)
        nb = -(-n // 16)
        assert np.array_equal(z["qc"][b, :, :n], zs["qc"][0]) and not z["qc"][b, :, n:].any()
        assert np.array_equal(z["kc"][b, :, :n], zs["kc"][0]) and not z["kc"][b, :, n:].any()
        assert np.array_equal(z["vc"][b, :, :n], zs["vc"][0]) and not z["vc"][b, :, n:].any()
        assert np.array_equal(z["qs"][b, :, :nb], zs["qs"][0]) and not z["qs"][b, :, nb:].any()
        assert np.array_equal(z["ks"][b, :, :nb], zs["ks"][0]) and not z["ks"][b, :, nb:].any()
        assert np.array_equal(z["vs"][b], zs["vs"][0])
        assert np.array_equal(z["vcol"][b, :, :nb], zs["vcol"][0]) and not z["vcol"][b, :, nb:].any()
        if smooth_q:
            assert np.array_equal(z["k_bias"][b, :, :n], zs["k_bias"][0]) and not z["k_bias"][b, :, n:].any()
        os_ = orc.attention(sub, zs, dumps=True)
        cnt = 2 * n
        assert np.array_equal(o["out"][at:at + cnt], os_["out"])
        assert np.array_equal(o["pcode"][at:at + cnt, :n], os_["pcode"]) and not o["pcode"][at:at + cnt, n:].any()
        assert np.array_equal(o["m"][at:at + cnt], os_["m"])
        at += cnt


def test_varlen_ragged_equals_zero_padding(orc):
    """A length that cuts a frame: without smoothing, the codes equal those of the
    plain oracle on zero-filled padding (zeros move no amax and no column sum),
    and each row attends over exactly its element's first seq_lens[b] keys
    (bidirectional oracle on that prefix)."""
    lens = [72, 30, 7]
    cfg, q, k, v = _varlen_case(orc, lens)
    tab = orc.rope_table(cfg, 1)
    z = orc.quantize(cfg, 1, tab, q, k, v, smooth_k=False, seq_lens=lens)
    q0, k0, v0 = (np.nan_to_num(x, nan=0.0) for x in (q, k, v))
    zp = orc.quantize(cfg, 1, tab, q0, k0, v0, smooth_k=False)
    for key in ("qc", "kc", "vc", "qs", "ks", "vs", "vcol"):
        assert np.array_equal(z[key], zp[key]), key
    N = 72
    for b, n in enumerate(lens):
        rows = np.array([(b * 2 + 1) * N + i for i in (0, n // 2, n - 1)], np.int64)
        r = orc.attention(cfg, z, rows=rows)
        sub = synth.custom(1, 1, 1, 1, n, 64, 24, 20, 20, 16, 16)
        pre = dict(qc=z["qc"][b, 1:2, :n], kc=z["kc"][b, 1:2, :n], vc=z["vc"][b, 1:2, :n],
                   qs=z["qs"][b, 1:2, :-(-n // 16)], ks=z["ks"][b, 1:2, :-(-n // 16)], vs=z["vs"][b, 1:2])
        p = orc.attention(sub, {kk: vv[None] for kk, vv in pre.items()}, rows=rows % N)
        assert np.array_equal(r["out"], p["out"]), b


def test_varlen_exact_and_fallback_see_only_their_prefix(orc):
    lens = [72, 30, 7]
    cfg, q, k, v = _varlen_case(orc, lens)
    N = 72
    rows = np.array([(b * 2 + h) * N + i for b, n in enumerate(lens) for h in range(2) for i in (0, n - 1)])
    ex = orc.exact_attention(cfg, q, k, v, rows=rows, seq_lens=lens)
    fb = orc.fallback_attention(cfg, orc.rope_table(cfg, 0), q / 8, k / 8, v, rows=rows, seq_lens=lens)
    ex8 = orc.exact_attention(cfg, q / 8, k / 8, v, rows=rows, seq_lens=lens)
    assert np.isfinite(ex).all() and np.isfinite(fb).all()
    assert np.max(np.abs(fb - ex8)) < 5e-3 * np.max(np.abs(ex8))
    # the binary64 oracle against numpy softmax over the prefix (RoPE'd with the
    # oracle's own rotation, pinned above)
    tab = orc.rope_table(cfg, 0, f64=True)
    qz, kz = (np.nan_to_num(x, nan=0.0).astype(np.float64) for x in (q, k))
    qr = orc.rope_rotate(cfg, 0, tab, qz)
    kr = orc.rope_rotate(cfg, 0, tab, kz)
    for t, row in enumerate(rows):
        bh, i = divmod(int(row), N)
        b, h = divmod(bh, 2)
        n = lens[b]
        sc = kr[b, h, :n] @ qr[b, h, i] / 8.0
        p = np.exp(sc - sc.max())
        want = p @ v[b, h, :n].astype(np.float64) / p.sum()
        assert np.allclose(ex[t], want, rtol=1e-10, atol=1e-12)
