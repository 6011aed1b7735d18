"""Ablation on synthetic inputs, from the oracle (CPU): attention-output cosine and
rel-L2 against exact binary64 attention for each rotation mode (none, Interleaved,
Half, Full D x D Hadamard) with the method's range-rectified P codes and with the
symmetric 8-level baseline, plus Half without K smoothing and Half / Full with Q
smoothing as well.  The GPU computes the
same variants within the parity tolerance of the oracle (tests/test_gpu_parity.py),
so these figures are the library's too.

The inputs are the Wan-like recipe (outlier channels in the first half of each RoPE
segment) at a medium shape.  The asserted orderings are the pages' claims (papernotes,
Key design 1 and 2; Ablation): rotating along the RoPE segment structure helps, and
range-rectified P is no worse than the symmetric code."""
import numpy as np

from int4_quantized_attention_amd import synth


def _cos_rel(o, ex):
    cos = np.sum(o * ex, axis=1) / np.linalg.norm(o, axis=1) / np.linalg.norm(ex, axis=1)
    return float(cos.mean()), float(np.linalg.norm(o - ex) / np.linalg.norm(ex))


def test_ablation_rotation_and_p_code(orc, capsys):
    cfg = synth.custom(1, 4, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    Q, K, V = synth.make_inputs(cfg)
    ex = orc.exact_attention(cfg, Q, K, V)
    res = {}
    for rot, name in [(0, "none"), (1, "interleaved"), (2, "half"), (3, "full")]:
        z = orc.quantize(cfg, rot, orc.rope_table(cfg, rot), Q, K, V)
        for pmax in (15, 7):
            res[(name, pmax)] = _cos_rel(orc.attention(cfg, z, pmax=pmax)["out"], ex)
    z = orc.quantize(cfg, 2, orc.rope_table(cfg, 2), Q, K, V, smooth_k=False)
    res[("half, no K smoothing", 15)] = _cos_rel(orc.attention(cfg, z)["out"], ex)
    for rot, name in [(2, "half"), (3, "full")]:
        z = orc.quantize(cfg, rot, orc.rope_table(cfg, rot), Q, K, V, smooth_q=True)
        res[(name + ", Q smoothing", 15)] = _cos_rel(orc.attention(cfg, z)["out"], ex)
    with capsys.disabled():
        print("\nablation (Wan-like inputs, B1 H4 N1173 D128, qk_blk 64, kv_blk 64):")
        for (name, pmax), (c, r) in res.items():
            print("  %-22s P %-17s mean cos %.4f  rel-L2 %.4f"
                  % (name, "range-rectified" if pmax == 15 else "symmetric [0,7]", c, r))
    cos = {k: v[0] for k, v in res.items()}
    assert cos[("full", 15)] > cos[("half", 15)] + 0.02
    assert cos[("half", 15)] > max(cos[("none", 15)], cos[("interleaved", 15)]) + 0.02
    assert cos[("half", 15)] > cos[("half, no K smoothing", 15)]
    for name in ("none", "interleaved", "half", "full"):
        assert cos[(name, 15)] >= cos[(name, 7)]
    for name in ("half", "full"):
        assert cos[(name + ", Q smoothing", 15)] > cos[(name, 15)]
