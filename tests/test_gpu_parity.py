"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs.  Integer work (INT4 codes, scales' bits, P codes, integer
accumulators, the running maximum) is bit-exact; the output O is within max-abs
2e-3 and rel-L2 1e-3 of the oracle's binary64 result."""
import numpy as np
import pytest
import torch

from int4_quantized_attention_amd import rotattn as ra
from int4_quantized_attention_amd import synth

from gpu_util import assert_close, compare_codes, gpu_quantize, rows_sample, to_dev

pytestmark = pytest.mark.gpu

ROTS = {"interleaved": 1, "half": 2, "none": 0, "full": 3}


def _oracle_head_cfg(cfg):
    c = dict(cfg)
    c["B"], c["H"] = 1, 1
    return c


def _run_case(orc, cfg, rot, smooth=True, debug_rows=None, out_dtype=torch.float32, in_dtype=None, pmax=15,
              causal=0, smooth_q=False, inputs=None):
    Q, K, V = inputs if inputs is not None else synth.make_inputs(cfg)
    shape, z = gpu_quantize(cfg, rot, Q, K, V, smooth, in_dtype, smooth_q=smooth_q)
    ref = orc.quantize(cfg, rot, orc.rope_table(cfg, rot), Q, K, V, smooth_k=smooth, smooth_q=smooth_q)
    compare_codes(cfg, z, ref)
    N, D = synth.n_tokens(cfg), cfg["D"]
    out = torch.full((cfg["B"], cfg["H"], N, D), float("nan"), dtype=out_dtype, device="cuda")
    ra.rotattn_int4_attention(shape, z, out, symmetric_p=pmax == 7, causal_block=causal)
    torch.cuda.synchronize()
    o = orc.attention(cfg, ref, pmax=pmax, causal_block=causal)
    if out_dtype == torch.float32:
        tol = (2e-3, 1e-3)
    elif out_dtype == torch.float16:
        tol = (4e-3, 1.5e-3)
    else:  # bfloat16 output: its rounding (unit roundoff 2^-8) on top of the fp32 bar
        tol = (2e-3 + 2.0**-8 * float(np.abs(o["out"]).max()), 1e-3 + 2.0**-8)
    assert_close(out.float().cpu().numpy().reshape(-1, D), o["out"], *tol)
    if debug_rows:
        BH = cfg["B"] * cfg["H"]
        for bh in range(BH):
            for (r0, n) in debug_rows:
                n = min(n, N - r0)
                dbg = dict(bh=bh, row0=r0, n_rows=n)
                out2 = torch.zeros_like(out)
                ra.rotattn_int4_attention(shape, z, out2, debug=dbg, symmetric_p=pmax == 7, causal_block=causal)
                torch.cuda.synchronize()
                rows = np.arange(bh * N + r0, bh * N + r0 + n)
                od = orc.attention(cfg, ref, rows=rows, dumps=True, pmax=pmax, causal_block=causal)
                assert np.array_equal(dbg["a_qk"].cpu().numpy(), od["a_qk"]), "a_qk"
                assert np.array_equal(dbg["p_codes"].cpu().numpy(), od["pcode"]), "P codes"
                assert np.array_equal(dbg["a_pv"].cpu().numpy(), od["a_pv"]), "a_pv"
                assert np.array_equal(dbg["m"].cpu().numpy().view(np.uint32), od["m"].view(np.uint32)), "m"
                assert np.allclose(dbg["l"].cpu().numpy(), od["l"], rtol=1e-5), "l"
                o2 = out2.float().cpu().numpy()[bh // cfg["H"], bh % cfg["H"], r0:r0 + n]
                assert_close(o2, od["out"])
                # the production kernel (all-zero level tiles skipped, exact path only
                # when a margin is unclear) adds exactly what the dense debug run adds
                o1 = out.float().cpu().numpy()[bh // cfg["H"], bh % cfg["H"], r0:r0 + n]
                assert np.array_equal(o1, o2), "production and debug outputs differ"
    return z, ref


@pytest.mark.parametrize("rot", ["interleaved", "half", "none", "full"])
def test_tiny_full_parity(orc, rot):
    cfg = dict(synth.CONFIGS["tiny"])
    _run_case(orc, cfg, ROTS[rot], debug_rows=[(0, 32)])


@pytest.mark.parametrize("qk,kv", [(1, 16), (1, 256), (16, 256), (4, 32)])
def test_tiny_block_sizes(orc, qk, kv):
    """The tiny case with per-token Q/K scales (qk_blk 1, the paper.gecl.asia
    analysis, "Key Insight"), other small scale blocks, and a 256-key online-softmax
    step (longer than the sequence): codes, dumps and output against the oracle."""
    cfg = dict(synth.CONFIGS["tiny"], qk_blk=qk, kv_blk=kv)
    _run_case(orc, cfg, 2, debug_rows=[(0, 32)])


MEDIUM = [
    # (id, config overrides)
    ("wan_half_kv64", dict(rot="half")),
    ("wan_inter_kv16_qk16", dict(rot="interleaved", qk_blk=16, kv_blk=16)),
    ("wan_half_kv32_qk32", dict(rot="half", qk_blk=32, kv_blk=32)),
    ("wan_half_kv128_qk128", dict(rot="half", qk_blk=128, kv_blk=128)),
    ("wan_half_kv128_qk16", dict(rot="half", qk_blk=16, kv_blk=128)),
    ("hunyuan_inter_B2", dict(rot="interleaved", recipe="hunyuan", Df=16, Dh=56, Dw=56, B=2)),
    ("peaked_none_nosmooth", dict(rot="none", recipe="peaked")),
    ("wan_half_kv64_qk1", dict(rot="half", qk_blk=1)),
    ("wan_inter_kv256_qk64", dict(rot="interleaved", qk_blk=64, kv_blk=256)),
    ("wan_half_kv256_qk1", dict(rot="half", qk_blk=1, kv_blk=256)),
    ("wan_half_kv128_qk2", dict(rot="half", qk_blk=2, kv_blk=128)),
    ("peaked_half_kv16_qk1", dict(rot="half", qk_blk=1, kv_blk=16, recipe="peaked")),
    ("hunyuan_inter_kv32_qk8_B2", dict(rot="interleaved", recipe="hunyuan", Df=16, Dh=56, Dw=56, B=2, qk_blk=8,
                                       kv_blk=32)),
]


@pytest.mark.parametrize("case", MEDIUM, ids=[c[0] for c in MEDIUM])
def test_medium_ragged_parity(orc, case):
    name, over = case
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    cfg.update(over)
    smooth = "nosmooth" not in name
    _run_case(orc, cfg, ROTS[cfg["rot"]], smooth=smooth, debug_rows=[(0, 40), (1133, 40)])


def test_d64_and_float32_and_bf16_inputs(orc):
    cfg = synth.custom(1, 2, 5, 7, 9, 64, 24, 20, 20, 32, 64, dtype="float32", recipe="tiny")
    _run_case(orc, cfg, 2)
    # bf16 storage: the oracle sees the same bf16 values as floats
    cfg2 = dict(cfg)
    Q, K, V = synth.make_inputs(cfg2)
    tb = lambda x: torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    Qb, Kb, Vb = tb(Q), tb(K), tb(V)
    shape, z = gpu_quantize(cfg2, 1, Qb, Kb, Vb, True, in_dtype=torch.bfloat16)
    ref = orc.quantize(cfg2, 1, orc.rope_table(cfg2, 1), Qb, Kb, Vb)
    compare_codes(cfg2, z, ref)


def test_fp16_output(orc):
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    _run_case(orc, cfg, 2, out_dtype=torch.float16)


@pytest.mark.parametrize("rot", ["full", "half"])
def test_ablation_full_rotation_and_symmetric_p(orc, rot):
    """Ablation variants: the Full (D x D Hadamard) rotation in the quantiser with the
    method's P codes, and the symmetric 8-level P baseline."""
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    if rot == "full":
        _run_case(orc, cfg, ROTS[rot], debug_rows=[(0, 40), (1133, 40)])
    else:
        _run_case(orc, cfg, ROTS[rot], debug_rows=[(0, 40), (1133, 40)], pmax=7)


def test_bf16_output(orc):
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    _run_case(orc, cfg, 2, out_dtype=torch.bfloat16)


def test_edge_single_token_and_zero_query(orc):
    cfg = synth.custom(2, 3, 1, 1, 1, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    _run_case(orc, cfg, 2, debug_rows=[(0, 1)])
    cfg = synth.custom(1, 2, 2, 5, 7, 128, 44, 42, 42, 16, 16, dtype="float16", recipe="wan")
    Q, K, V = synth.make_inputs(cfg)
    Q[:] = 0
    K[0, 1, :20] = 0  # an all-zero K scale block
    shape, z = gpu_quantize(cfg, 1, Q, K, V)
    ref = orc.quantize(cfg, 1, orc.rope_table(cfg, 1), Q, K, V)
    compare_codes(cfg, z, ref)
    out = torch.empty((1, 2, 70, 128), dtype=torch.float32, device="cuda")
    ra.rotattn_int4_attention(shape, z, out)
    assert_close(out.cpu().numpy().reshape(-1, 128), orc.attention(cfg, ref)["out"])


def test_edge_tiny_magnitudes(orc):
    """Blocks whose amax lies in [2^-126, 7 / FLT_MAX): 7 / amax overflows to inf, the
    scale amax / 7 is subnormal, and the clamp of the code turns +-inf into +-7 and the
    NaN of 0 * inf into -7.  Codes and scale bits against the oracle."""
    cfg = synth.custom(1, 2, 1, 4, 8, 64, 24, 20, 20, 16, 16, dtype="float32", recipe="wan")
    Q, K, V = synth.make_inputs(cfg)
    rng = np.random.default_rng(7)
    tiny = np.array([0.0, 1.2e-38, -1.2e-38, 1.5e-38, -1.5e-38, 2.0e-38, -2.0e-38], np.float32)
    assert np.all(np.isinf(np.float32(7.0) / tiny[1:]))
    # Q and K are multiplied by constants of about 1.4 before their blocks are
    # quantised: scaled by 0.9 they land in the same band
    qk_tiny = tiny[:5] * np.float32(0.9)
    Q[0, 0, :16] = rng.choice(qk_tiny, size=(16, 64))  # one whole Q scale block
    K[0, 1, 16:32] = rng.choice(qk_tiny, size=(16, 64))
    K[0, 1, 16, :] = 0.0
    V[0, 0, :, 5] = rng.choice(tiny, size=V.shape[2])  # one V channel
    shape, z = gpu_quantize(cfg, 0, Q, K, V, smooth=False)
    ref = orc.quantize(cfg, 0, orc.rope_table(cfg, 0), Q, K, V, smooth_k=False)
    for name, blk in (("qs", (0, 0)), ("ks", (1, 1)), ("vs", (0, 5))):
        sc = ref[name].reshape(2, -1)[blk]
        assert 0 < sc < np.finfo(np.float32).tiny, (name, sc)  # the regime is reached
    assert np.any(ref["qc"].reshape(2, -1, 64)[0, :16][Q[0, 0, :16] == 0] == -7)
    compare_codes(cfg, z, ref)
    # ragged: the last Q/K block and the last V tile hold tokens that do not exist,
    # whose codes stay 0 (and out of the column sums)
    cfg = synth.custom(1, 1, 1, 3, 7, 64, 24, 20, 20, 16, 16, dtype="float32", recipe="wan")
    Q, K, V = synth.make_inputs(cfg)
    Q[0, 0, 16:] = rng.choice(qk_tiny, size=(5, 64))
    K[0, 0, 16:] = rng.choice(qk_tiny, size=(5, 64))
    V[0, 0, :, 3] = rng.choice(tiny, size=V.shape[2])
    shape, z = gpu_quantize(cfg, 0, Q, K, V, smooth=False)
    ref = orc.quantize(cfg, 0, orc.rope_table(cfg, 0), Q, K, V, smooth_k=False)
    assert 0 < ref["qs"].reshape(-1)[1] < np.finfo(np.float32).tiny
    compare_codes(cfg, z, ref)


def test_head_subset_leaves_other_heads(orc):
    cfg = synth.custom(1, 4, 3, 10, 11, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    Q, K, V = synth.make_inputs(cfg)
    shape, z = gpu_quantize(cfg, 2, Q, K, V)
    ref = orc.quantize(cfg, 2, orc.rope_table(cfg, 2), Q, K, V)
    out = torch.full((1, 4, 330, 128), 7.0, dtype=torch.float32, device="cuda")
    ra.rotattn_int4_attention(shape, z, out, heads=[3, 1])
    o = out.cpu().numpy()
    full = orc.attention(cfg, ref)["out"].reshape(1, 4, 330, 128)
    assert np.all(o[0, 0] == 7.0) and np.all(o[0, 2] == 7.0)
    assert_close(o[0, 1], full[0, 1])
    assert_close(o[0, 3], full[0, 3])


def test_more_heads_than_one_launch(orc):
    """B*H above the per-launch head limit (512): the INT4 attention and the fallback
    are split into several launches and every head is computed (heads on both sides
    of the split are checked against the oracle)."""
    cfg = synth.custom(1, 520, 1, 2, 16, 64, 24, 20, 20, 16, 16, dtype="float32", recipe="tiny", rot="half")
    N, D = synth.n_tokens(cfg), 64
    Q, K, V = synth.make_inputs(cfg)
    shape, z = gpu_quantize(cfg, 2, Q, K, V)
    out = torch.empty((1, 520, N, D), dtype=torch.float32, device="cuda")
    ra.rotattn_int4_attention(shape, z, out)
    q, k, v = (to_dev(x) for x in (Q, K, V))
    tab0 = ra.rotattn_build_rope_table(shape, 0).cuda()
    ws = torch.empty(ra.rotattn_fp16_fallback_workspace(shape), dtype=torch.uint8, device="cuda")
    out_fb = torch.empty((1, 520, N, D), dtype=torch.float32, device="cuda")
    ra.rotattn_fp16_fallback(shape, q, k, v, tab0, out_fb, ws)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(h * N, (h + 1) * N) for h in (0, 511, 512, 519)])
    ref = orc.quantize(cfg, 2, orc.rope_table(cfg, 2), Q, K, V)
    assert_close(out.cpu().numpy().reshape(-1, D)[rows], orc.attention(cfg, ref, rows=rows)["out"])
    want_fb = orc.fallback_attention(cfg, orc.rope_table(cfg, 0), Q, K, V, rows=rows)
    assert_close(out_fb.cpu().numpy().reshape(-1, D)[rows], want_fb)


def test_quantize_without_column_sums():
    """The V column sums are optional (the benchmark passes NULL for them): every other
    output of the quantiser, padding included, and the attention on it are
    bit-identical with and without them."""
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    Q, K, V = synth.make_inputs(cfg)
    shape = ra.Shape.of(cfg)
    q, k, v = (to_dev(x, torch.float16) for x in (Q, K, V))
    tab = ra.rotattn_build_rope_table(shape, 2).cuda()
    runs = []
    for colsum in (True, False):
        z = ra.alloc_codes(shape, colsum=colsum)
        ra.rotattn_quantize_qk(shape, 2, q, k, v, tab, True, z)
        out = torch.empty((1, 2, synth.n_tokens(cfg), 128), dtype=torch.float32, device="cuda")
        ra.rotattn_int4_attention(shape, z, out)
        torch.cuda.synchronize()
        runs.append((z, out))
    (za, oa), (zb, ob) = runs
    assert za["v_colsum"] is not None and zb["v_colsum"] is None
    for key in ("q_codes", "q_scale", "k_codes", "k_scale", "v_codes", "v_scale"):
        assert torch.equal(za[key], zb[key]), key
    assert torch.equal(oa, ob)


CAUSAL = [
    # (id, config overrides, causal block): token-causal, frame-causal (one frame is
    # 391 tokens, so tiles straddle frames), a block that does not divide N, a block
    # smaller than a step, each kv_blk and D 64
    ("token_kv64", dict(), 1),
    ("frame_kv64", dict(), 391),
    ("block100_kv128_qk128", dict(qk_blk=128, kv_blk=128), 100),
    ("frame_kv16_qk16", dict(qk_blk=16, kv_blk=16), 391),
    ("block5_kv32_qk32_symmetric", dict(qk_blk=32, kv_blk=32), 5),
    ("block_ge_n", dict(), 5000),
    ("frame_kv256_qk1", dict(qk_blk=1, kv_blk=256), 391),
    ("block100_kv256", dict(kv_blk=256), 100),
]


@pytest.mark.parametrize("case", CAUSAL, ids=[c[0] for c in CAUSAL])
def test_causal_parity(orc, case):
    """Block-causal attention (query i sees key j iff j // c <= i // c) against the
    oracle's, dumps included, on rows around tile and frame boundaries."""
    name, over, cb = case
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    cfg.update(over)
    pmax = 7 if "symmetric" in name else 15
    _run_case(orc, cfg, 2, debug_rows=[(0, 40), (360, 48), (1133, 40)], pmax=pmax, causal=cb)


def test_causal_d64(orc):
    cfg = synth.custom(1, 2, 5, 7, 9, 64, 24, 20, 20, 32, 64, dtype="float32", recipe="tiny")
    _run_case(orc, cfg, 1, debug_rows=[(0, 64), (250, 65)], causal=63)


def _offset_queries(cfg, seed=7):
    """Inputs whose queries share a large offset in the slow RoPE pairs of each
    segment (where Q smoothing matters), in the config's storage dtype."""
    Q, K, V = synth.make_inputs(cfg)
    rng = np.random.default_rng(seed)
    off = np.zeros(cfg["D"], np.float32)
    o = 0
    for w in (cfg["Df"], cfg["Dh"], cfg["Dw"]):
        off[o + w - 4:o + w] = rng.uniform(4, 8, 4) * rng.choice([-1, 1], 4)
        o += w
    return (Q.astype(np.float32) + off).astype(Q.dtype), K, V


QSMOOTH = [
    # (id, config overrides, rotation, smooth_k, causal block)
    ("half_kv64", dict(), 2, True, 0),
    ("inter_kv16_qk16", dict(qk_blk=16, kv_blk=16), 1, True, 0),
    ("half_kv128_qk16_nosmoothk", dict(qk_blk=16, kv_blk=128), 2, False, 0),
    ("full_kv32_frame_causal", dict(qk_blk=32, kv_blk=32), 3, True, 391),
    ("half_kv64_qk1", dict(qk_blk=1), 2, True, 0),
    ("inter_kv256_qk2_frame_causal", dict(qk_blk=2, kv_blk=256), 1, True, 391),
]


@pytest.mark.parametrize("case", QSMOOTH, ids=[c[0] for c in QSMOOTH])
def test_q_smoothing_parity(orc, case):
    """Q smoothing: Q codes of Q - mu_q and the per-key term k_bias bit-exact, the
    attention with the term added back (P codes, m, sums bit-exact; O within the bar)."""
    name, over, rot, smooth_k, cb = case
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    cfg.update(over)
    _run_case(orc, cfg, rot, smooth=smooth_k, debug_rows=[(0, 40), (1133, 40)], causal=cb, smooth_q=True,
              inputs=_offset_queries(cfg))


def test_q_smoothing_d64_f32(orc):
    cfg = synth.custom(1, 2, 5, 7, 9, 64, 24, 20, 20, 32, 64, dtype="float32", recipe="tiny")
    _run_case(orc, cfg, 2, debug_rows=[(0, 64)], smooth_q=True, inputs=_offset_queries(cfg))


VARLEN = [
    # (id, lengths of the three batch elements, rotation, Q smoothing, causal block, kv_blk[, qk_blk])
    ("frames_and_ragged_kv64", [1173, 782, 500], 2, False, 0, 64),
    ("ragged_smoothq_kv16", [1173, 129, 1], 1, True, 0, 16),
    ("ragged_frame_causal_kv128", [600, 1173, 391], 2, False, 391, 128),
    ("ragged_kv256_qk1", [1173, 300, 77], 2, False, 0, 256, 1),
]


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_varlen_parity(orc, case):
    """Variable-length batch in the padded layout: padding holds NaN (nothing may read
    it), codes and scales bit-exact with the oracle's, valid rows within the bar with
    dumps bit-exact, rows past each length left untouched."""
    name, lens, rot, smooth_q, cb, kv = case[:6]
    qk = case[6] if len(case) > 6 else min(kv, 64)
    cfg = synth.custom(3, 2, 3, 17, 23, 128, 44, 42, 42, qk, kv, dtype="float16", recipe="wan")
    Q, K, V = synth.make_inputs(cfg)
    for b, n in enumerate(lens):
        for x in (Q, K, V):
            x[b, :, n:] = np.nan
    shape = ra.Shape.of(cfg)
    q, k, v = (to_dev(x) for x in (Q, K, V))
    tab = ra.rotattn_build_rope_table(shape, rot).cuda()
    z = ra.alloc_codes(shape, smooth_q=smooth_q)
    ra.rotattn_quantize_qk(shape, rot, q, k, v, tab, True, z, smooth_q=smooth_q, seq_lens=lens)
    ref = orc.quantize(cfg, rot, orc.rope_table(cfg, rot), Q, K, V, smooth_q=smooth_q, seq_lens=lens)
    compare_codes(cfg, z, ref)
    N, D = synth.n_tokens(cfg), 128
    out = torch.full((3, 2, N, D), float("nan"), dtype=torch.float32, device="cuda")
    ra.rotattn_int4_attention(shape, z, out, causal_block=cb)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for b, n in enumerate(lens):
        assert np.isnan(o[b, :, n:]).all(), "rows past the length were written"
        rows = np.array([(b * 2 + h) * N + i for h in range(2) for i in rows_sample(n, 16, seed=b)], np.int64)
        want = orc.attention(cfg, ref, rows=rows, causal_block=cb)["out"]
        assert_close(o.reshape(-1, D)[rows], want)
    # dumps of the last rows of the shortest element
    b = int(np.argmin(lens))
    n = lens[b]
    r0 = max(0, n - 40)
    dbg = dict(bh=2 * b + 1, row0=r0, n_rows=n - r0)
    out2 = torch.zeros_like(out)
    ra.rotattn_int4_attention(shape, z, out2, debug=dbg, causal_block=cb)
    torch.cuda.synchronize()
    od = orc.attention(cfg, ref, rows=np.arange((2 * b + 1) * N + r0, (2 * b + 1) * N + n), dumps=True,
                       causal_block=cb)
    assert np.array_equal(dbg["a_qk"].cpu().numpy(), od["a_qk"]), "a_qk"
    assert np.array_equal(dbg["p_codes"].cpu().numpy(), od["pcode"]), "P codes"
    assert np.array_equal(dbg["a_pv"].cpu().numpy(), od["a_pv"]), "a_pv"
    assert np.array_equal(dbg["m"].cpu().numpy().view(np.uint32), od["m"].view(np.uint32)), "m"
    assert_close(out2.cpu().numpy()[b, 1, r0:n], od["out"])
    assert np.array_equal(out2.cpu().numpy()[b, 1, r0:n], o[b, 1, r0:n]), "production and debug outputs differ"


def _random_config(rng, i):
    D = int(rng.choice([64, 128]))
    if D == 64:
        Df, Dh, Dw = 24, 20, 20
    else:
        Df, Dh, Dw = [(44, 42, 42), (16, 56, 56)][int(rng.integers(2))]
    kv = int(rng.choice([16, 32, 64, 128, 256]))
    qk = int(rng.choice([1, 2, 16, 32, 64, 128]))
    F, Hs, Ws = int(rng.integers(1, 4)), int(rng.integers(3, 19)), int(rng.integers(3, 29))
    B = int(rng.integers(1, 3))
    dtype = str(rng.choice(["float16", "float32"]))
    cfg = synth.custom(B, 2, F, Hs, Ws, D, Df, Dh, Dw, qk, kv, dtype=dtype,
                       recipe=str(rng.choice(["wan", "peaked"])) if D == 128 else "tiny")
    N = F * Hs * Ws
    # the options alternate with the case number so that every combination class is
    # covered; the rest is drawn
    opts = dict(rot=i % 4, smooth_k=bool(rng.integers(2)), smooth_q=i % 2 == 1,
                causal=[0, 1, Hs * Ws, int(rng.integers(2, 200))][(i // 2) % 4],
                lens=[int(rng.integers(1, N + 1)) for _ in range(B)] if i % 3 == 0 else None,
                pmax=7 if i % 5 == 4 else 15)
    return cfg, opts


@pytest.mark.parametrize("i", range(32))
def test_random_configs_parity(orc, i):
    """Seeded random combinations of shape, head split, block sizes, rotation, K and Q
    smoothing, causal block, variable lengths and P code: codes bit-exact, sampled
    rows within the bar, and on two row ranges the production output equal to the
    dense debug run bit for bit with its dumps equal to the oracle's."""
    rng = np.random.default_rng(1000 + i)
    cfg, o = _random_config(rng, i)
    print("case", i, cfg, o, flush=True)
    B, H, D = cfg["B"], cfg["H"], cfg["D"]
    N = synth.n_tokens(cfg)
    Q, K, V = synth.make_inputs(cfg, seed=i)
    lens = o["lens"]
    if lens is not None:
        for b, n in enumerate(lens):
            for x in (Q, K, V):
                x[b, :, n:] = np.nan
    shape = ra.Shape.of(cfg)
    q, k, v = (to_dev(x) for x in (Q, K, V))
    tab = ra.rotattn_build_rope_table(shape, o["rot"]).cuda()
    z = ra.alloc_codes(shape, smooth_q=o["smooth_q"])
    ra.rotattn_quantize_qk(shape, o["rot"], q, k, v, tab, o["smooth_k"], z, smooth_q=o["smooth_q"], seq_lens=lens)
    ref = orc.quantize(cfg, o["rot"], orc.rope_table(cfg, o["rot"]), Q, K, V, smooth_k=o["smooth_k"],
                       smooth_q=o["smooth_q"], seq_lens=lens)
    compare_codes(cfg, z, ref)
    out = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device="cuda")
    ra.rotattn_int4_attention(shape, z, out, causal_block=o["causal"], symmetric_p=o["pmax"] == 7)
    torch.cuda.synchronize()
    ob = out.cpu().numpy()
    for bh in range(B * H):
        n = lens[bh // H] if lens is not None else N
        rows = rows_sample(n, 12, seed=bh)
        want = orc.attention(cfg, ref, rows=bh * N + rows, causal_block=o["causal"], pmax=o["pmax"])["out"]
        assert_close(ob[bh // H, bh % H][rows], want)
        assert np.isnan(ob[bh // H, bh % H, n:]).all()
    for bh, r0 in ((0, 0), (B * H - 1, None)):
        n = lens[bh // H] if lens is not None else N
        r0 = max(0, n - 33) if r0 is None else 0
        cnt = min(33, n - r0)
        dbg = dict(bh=bh, row0=r0, n_rows=cnt)
        out2 = torch.zeros_like(out)
        ra.rotattn_int4_attention(shape, z, out2, debug=dbg, causal_block=o["causal"], symmetric_p=o["pmax"] == 7)
        torch.cuda.synchronize()
        od = orc.attention(cfg, ref, rows=np.arange(bh * N + r0, bh * N + r0 + cnt), dumps=True,
                           causal_block=o["causal"], pmax=o["pmax"])
        assert np.array_equal(dbg["p_codes"].cpu().numpy(), od["pcode"]), "P codes"
        assert np.array_equal(dbg["a_pv"].cpu().numpy(), od["a_pv"]), "a_pv"
        assert np.array_equal(out2.cpu().numpy()[bh // H, bh % H, r0:r0 + cnt], ob[bh // H, bh % H, r0:r0 + cnt])


def test_empty_head_list_writes_nothing(orc):
    cfg = synth.custom(1, 2, 2, 5, 7, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    Q, K, V = synth.make_inputs(cfg)
    shape, z = gpu_quantize(cfg, 2, Q, K, V)
    out = torch.full((1, 2, 70, 128), float("nan"), dtype=torch.float32, device="cuda")
    ra.rotattn_int4_attention(shape, z, out, heads=[])
    tab = ra.rotattn_build_rope_table(shape, 0).cuda()
    ws = torch.empty(ra.rotattn_fp16_fallback_workspace(shape), dtype=torch.uint8, device="cuda")
    ra.rotattn_fp16_fallback(shape, to_dev(Q), to_dev(K), to_dev(V), tab, out, ws, heads=[])
    torch.cuda.synchronize()
    assert torch.isnan(out).all()


def test_plain_c_device_caller(orc, tmp_path):
    """The device path through the C ABI alone: a C99 program (tests/c_abi_device.c)
    allocates with the HIP runtime's C API, quantises and runs the attention on the
    tiny shape, and checks codes, scales and output against the oracle's C entry
    points."""
    import os
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg, odir = os.path.join(root, "int4_quantized_attention_amd"), os.path.join(root, "oracle")
    exe = str(tmp_path / "c_abi_device")
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                         "-I" + os.path.join(root, "include"), "-I/opt/rocm/include",
                         os.path.join(root, "tests", "c_abi_device.c"), "-L" + pkg, "-lrotattn", "-L" + odir,
                         "-lorc", "-L/opt/rocm/lib", "-lamdhip64", "-lm",
                         "-Wl,-rpath," + ":".join((pkg, odir, "/opt/rocm/lib")), "-o", exe],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, "check %d failed: %s" % (run.returncode, run.stderr)
    assert run.stdout.startswith("c device abi ok")
