"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: codes of sampled heads bit-exact, outputs of sampled rows (first
tile, ragged last tile, random rows) within tolerance of the oracle; the FP16
fallback; per-head routing of the mixed-precision config."""
import numpy as np
import pytest
import torch

from int4_quantized_attention_amd import rotattn as ra
from int4_quantized_attention_amd import synth

from gpu_util import assert_close, compare_codes, gpu_quantize, rows_sample, to_dev

pytestmark = pytest.mark.gpu
ROTS = {"interleaved": 1, "half": 2, "none": 0}


def _one_head(cfg, b, h):
    c = dict(cfg)
    c["B"], c["H"] = 1, 1
    q, k, v = synth.make_head(cfg, b, h)
    dt = np.float16 if cfg["dtype"] == "float16" else np.float32
    f = lambda x: x.astype(dt)[None, None]
    return c, f(q), f(k), f(v)


def test_fallback_parity_medium(orc):
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="peaked")
    Q, K, V = synth.make_inputs(cfg)
    shape = ra.Shape.of(cfg)
    tab = ra.rotattn_build_rope_table(shape, 0).cuda()
    ws = torch.empty(ra.rotattn_fp16_fallback_workspace(shape), dtype=torch.uint8, device="cuda")
    N = synth.n_tokens(cfg)
    out = torch.full((1, 2, N, 128), float("nan"), dtype=torch.float32, device="cuda")
    ra.rotattn_fp16_fallback(shape, to_dev(Q), to_dev(K), to_dev(V), tab, out, ws)
    ref = orc.fallback_attention(cfg, orc.rope_table(cfg, 0), Q, K, V)
    assert_close(out.cpu().numpy().reshape(-1, 128), ref)


@pytest.mark.parametrize("cb", [1, 391, 100])
def test_fallback_causal(orc, cb):
    """Block-causal fallback (query i sees key j iff j // c <= i // c) against the
    fallback oracle with the same mask."""
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="peaked")
    Q, K, V = synth.make_inputs(cfg)
    shape = ra.Shape.of(cfg)
    tab = ra.rotattn_build_rope_table(shape, 0).cuda()
    ws = torch.empty(ra.rotattn_fp16_fallback_workspace(shape), dtype=torch.uint8, device="cuda")
    N = synth.n_tokens(cfg)
    out = torch.full((1, 2, N, 128), float("nan"), dtype=torch.float32, device="cuda")
    ra.rotattn_fp16_fallback(shape, to_dev(Q), to_dev(K), to_dev(V), tab, out, ws, causal_block=cb)
    ref = orc.fallback_attention(cfg, orc.rope_table(cfg, 0), Q, K, V, causal_block=cb)
    assert_close(out.cpu().numpy().reshape(-1, 128), ref)


def test_fallback_varlen(orc):
    """Variable-length fallback: NaN padding never read, rows past each length left
    untouched, valid rows against the fallback oracle (also frame-causal)."""
    cfg = synth.custom(3, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="peaked")
    lens = [1173, 500, 37]
    Q, K, V = synth.make_inputs(cfg)
    for b, n in enumerate(lens):
        for x in (Q, K, V):
            x[b, :, n:] = np.nan
    shape = ra.Shape.of(cfg)
    tab = ra.rotattn_build_rope_table(shape, 0).cuda()
    ws = torch.empty(ra.rotattn_fp16_fallback_workspace(shape), dtype=torch.uint8, device="cuda")
    N = synth.n_tokens(cfg)
    for cb in (0, 391):
        out = torch.full((3, 2, N, 128), float("nan"), dtype=torch.float32, device="cuda")
        ra.rotattn_fp16_fallback(shape, to_dev(Q), to_dev(K), to_dev(V), tab, out, ws, causal_block=cb,
                                 seq_lens=lens)
        o = out.cpu().numpy()
        for b, n in enumerate(lens):
            assert np.isnan(o[b, :, n:]).all()
            rows = np.array([(b * 2 + h) * N + i for h in range(2) for i in rows_sample(n, 16, seed=b)])
            ref = orc.fallback_attention(cfg, orc.rope_table(cfg, 0), Q, K, V, rows=rows, causal_block=cb,
                                         seq_lens=lens)
            assert_close(o.reshape(-1, 128)[rows], ref)


@pytest.mark.parametrize("in_dt,out_dt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float16)])
def test_fallback_input_output_dtypes(orc, in_dt, out_dt):
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float32", recipe="peaked")
    Q, K, V = synth.make_inputs(cfg)
    # the oracle sees exactly the values the library reads
    Qd, Kd, Vd = (torch.from_numpy(x).to(in_dt) for x in (Q, K, V))
    Qf, Kf, Vf = (x.float().numpy() for x in (Qd, Kd, Vd))
    shape = ra.Shape.of(cfg)
    tab = ra.rotattn_build_rope_table(shape, 0).cuda()
    ws = torch.empty(ra.rotattn_fp16_fallback_workspace(shape), dtype=torch.uint8, device="cuda")
    N = synth.n_tokens(cfg)
    out = torch.full((1, 2, N, 128), float("nan"), dtype=out_dt, device="cuda")
    ra.rotattn_fp16_fallback(shape, Qd.cuda(), Kd.cuda(), Vd.cuda(), tab, out, ws)
    ref = orc.fallback_attention(cfg, orc.rope_table(cfg, 0), Qf, Kf, Vf)
    if out_dt == torch.bfloat16:  # bf16 rounding (unit roundoff 2^-8) on top of the binary32 bar
        tol = (2e-3 + 2.0**-8 * float(np.abs(ref).max()), 1e-3 + 2.0**-8)
    else:
        tol = (4e-3, 1.5e-3)
    assert_close(out.float().cpu().numpy().reshape(-1, 128), ref, *tol)


@pytest.mark.parametrize("name", ["wan480p", "wan720p", "hunyuan720p"])
def test_full_config_int4(orc, name):
    cfg = synth.CONFIGS[name]
    rot = ROTS[cfg["rot"]]
    N, D, H = synth.n_tokens(cfg), cfg["D"], cfg["H"]
    print("case", name, flush=True)
    Q, K, V = synth.make_inputs(cfg)
    shape, z = gpu_quantize(cfg, rot, Q, K, V)
    out = torch.empty((1, H, N, D), dtype=torch.float32, device="cuda")
    ra.rotattn_int4_attention(shape, z, out)
    torch.cuda.synchronize()
    del Q, K, V
    for h in (0, H - 1):
        c1, q, k, v = _one_head(cfg, 0, h)
        ref = orc.quantize(c1, rot, orc.rope_table(c1, rot), q, k, v)
        compare_codes(cfg, z, ref, heads=[h])
        rows = rows_sample(N, 24, seed=h)
        o = orc.attention(c1, ref, rows=rows)["out"]
        assert_close(out[0, h].cpu().numpy()[rows], o)


def test_mixed_routing_full(orc):
    """Half of the heads (even flat ids) take the FP16 fallback, the other half the
    INT4 path with Half rotation, both writing one output tensor."""
    cfg = synth.CONFIGS["mixed_ragged"]
    B, H, D = cfg["B"], cfg["H"], cfg["D"]
    N = synth.n_tokens(cfg)
    Q, K, V = synth.make_inputs(cfg)
    shape = ra.Shape.of(cfg)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    fb_heads = [i for i in range(B * H) if i % 2 == 0]
    q4_heads = [i for i in range(B * H) if i % 2 == 1]
    tab0 = ra.rotattn_build_rope_table(shape, 0).cuda()
    tab2 = ra.rotattn_build_rope_table(shape, 2).cuda()
    ws = torch.empty(ra.rotattn_fp16_fallback_workspace(shape), dtype=torch.uint8, device="cuda")
    z = ra.alloc_codes(shape)
    out = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device="cuda")
    ra.rotattn_fp16_fallback(shape, q, k, v, tab0, out, ws, heads=fb_heads)
    ra.rotattn_quantize_qk(shape, 2, q, k, v, tab2, True, z)
    ra.rotattn_int4_attention(shape, z, out, heads=q4_heads)
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(B * H, N, D)
    assert np.isfinite(o).all()
    for flat in (0, 1, B * H - 2, B * H - 1):
        b, h = divmod(flat, H)
        c1, qh, kh, vh = _one_head(cfg, b, h)
        rows = rows_sample(N, 16, seed=flat)
        if flat % 2 == 0:
            ref = orc.fallback_attention(c1, orc.rope_table(c1, 0), qh, kh, vh, rows=rows)
        else:
            zq = orc.quantize(c1, 2, orc.rope_table(c1, 2), qh, kh, vh)
            compare_codes(cfg, z, zq, heads=[flat])
            ref = orc.attention(c1, zq, rows=rows)["out"]
        assert_close(o[flat][rows], ref)
