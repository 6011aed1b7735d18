"""Benchmark of the RotateAttention INT4 hot path on one MI355X.

One step = the whole INT4 path over one batch of synthetic input already in HBM:
rotattn_quantize_qk (fused RoPE -> Half rotation -> K smoothing -> INT4 codes)
then rotattn_int4_attention, on the Wan-14B-720p-like layer (B=1, H=40, grid
21x45x80 -> N=75600, D=128 split 44/42/42).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_F16_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
PEAK_FP8_TOPS = 5000.0    # MI355X dense fp8 MFMA (the P V form the attention issues)
PEAK_FP6_TOPS = 10100.0   # MI355X dense fp6 MFMA (the Q K^T form the attention issues)
CONFIG = "wan720p"
WORKLOADS = {
    "wan480p": "Wan-1.3B-480p-like attention layer",
    "wan720p": "Wan-14B-720p-like attention layer",
    "hunyuan720p": "HunyuanVideo-720p-like attention layer",
    "mixed_ragged": "mixed-precision ragged layer (even heads FP16 fallback, odd heads INT4)",
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-fallback", action="store_true", help="skip timing the FP16 fallback")
    ap.add_argument("--config", default=CONFIG)
    ap.add_argument("--kv", type=int, default=0, help="override kv_blk (keys per online-softmax step)")
    ap.add_argument("--qk", type=int, default=0, help="override qk_blk (tokens per Q/K scale)")
    ap.add_argument("--rot", default="", choices=["", "none", "interleaved", "half", "full"],
                    help="override the rotation mode (full: the D x D Hadamard ablation)")
    ap.add_argument("--causal", type=int, default=0,
                    help="block-causal attention with this block of tokens (0: bidirectional); the "
                         "operation count is then that of the visible query/key pairs")
    ap.add_argument("--smooth-q", action="store_true",
                    help="Q smoothing as well (rotattn_quantize_qk_ex with smooth_q set, and the per-key score term)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates the HBM byte counters)")
    ap.add_argument("--no-diffuse", action="store_true",
                    help="skip the second attention timing on the diffuse (skip-free) recipe")
    ap.add_argument("--torch-sdpa", action="store_true",
                    help="also time torch's flash scaled-dot-product attention on the same shape (context)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on exactly one GPU (the path shards by head with no "
              "communication; see the design notes); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from int4_quantized_attention_amd import rotattn as ra
    from int4_quantized_attention_amd import synth

    torch.cuda.set_device(0)
    if args.calib_copy:
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": x.numel() * 4, "launches": 3}))
        return
    cfg = dict(synth.CONFIGS[args.config])
    if args.kv:
        cfg["kv_blk"] = args.kv
    if args.qk:
        cfg["qk_blk"] = args.qk
    if args.rot:
        cfg["rot"] = args.rot
    B, H, D = cfg["B"], cfg["H"], cfg["D"]
    N = synth.n_tokens(cfg)
    rot = ra.ROT_BY_NAME[cfg["rot"]]
    shape = ra.Shape.of(cfg)
    ops = 4.0 * N * N * D * H * B
    if args.causal:
        # query i sees keys [0, min(N, (i // c + 1) c))
        i = np.arange(N, dtype=np.int64)
        ops = 4.0 * float(np.minimum(N, (i // args.causal + 1) * args.causal).sum()) * D * H * B

    Q, K, V = synth.make_inputs(cfg)
    q, k, v = (torch.from_numpy(x).cuda() for x in (Q, K, V))
    del Q, K, V
    tab = ra.rotattn_build_rope_table(shape, rot).cuda()
    # the column sums of V are an optional output that the attention does not read
    z = ra.alloc_codes(shape, colsum=False, smooth_q=args.smooth_q)
    out = torch.empty((B, H, N, D), dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream()

    # the mixed-precision workload routes even flat heads to the FP16 fallback and odd
    # ones to the INT4 path (both write the one output tensor); the others are all INT4
    mixed = args.config == "mixed_ragged"
    q4_heads = [i for i in range(B * H) if i % 2 == 1] if mixed else None
    fb_heads = [i for i in range(B * H) if i % 2 == 0] if mixed else None
    if mixed:
        ws_fb = torch.empty(ra.rotattn_fp16_fallback_workspace(shape), dtype=torch.uint8, device="cuda")
        tab_fb = ra.rotattn_build_rope_table(shape, 0).cuda()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        ra.rotattn_quantize_qk(shape, rot, q, k, v, tab, True, z, smooth_q=args.smooth_q)
        if ev is not None:
            ev[1].record(stream)
        ra.rotattn_int4_attention(shape, z, out, heads=q4_heads, causal_block=args.causal)
        if ev is not None:
            ev[2].record(stream)
        if mixed:
            ra.rotattn_fp16_fallback(shape, q, k, v, tab_fb, out, ws_fb, heads=fb_heads, causal_block=args.causal)
            if ev is not None:
                ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stats = skip_stats(lambda st: ra.rotattn_int4_attention(shape, z, out, heads=q4_heads, causal_block=args.causal,
                                                            skip_stats=st))
    k1_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    k2_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    k3_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) if mixed else None
    ms_step = wall * 1e3 / args.steps
    ops_q4 = ops / 2 if mixed else ops  # the INT4 kernel's share of the work

    # K1 algorithmic bytes: read Q, K, V (fp16) once, write three INT4 code tensors
    # and the scales: 3*2 + 3*0.5 bytes per element.
    k1_bytes = (3 * 2.0 + 3 * 0.5) * N * D * H * B
    k2_tops = ops_q4 / (k2_ms * 1e-3) / 1e12
    headline = args.config == CONFIG and not (args.kv or args.qk or args.rot or args.causal or args.smooth_q)

    result = {
        "metric": "effective attention TOPS (4*N^2*D*H/s) at Wan-720p-like shape; % int8 MFMA peak",
        "value": round(ops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d H=%d grid %dx%dx%d N=%d D=%d "
                               "(%d/%d/%d), %s rotation, qk_blk=%d kv_blk=%d, %s%s"
                               % (WORKLOADS.get(args.config, args.config), B, H, cfg["F"], cfg["Hs"], cfg["Ws"], N,
                                  D, cfg["Df"], cfg["Dh"], cfg["Dw"], cfg["rot"], cfg["qk_blk"], cfg["kv_blk"],
                                  io_label(cfg["dtype"]),
                                  (", block-causal c=%d (ops of visible pairs)" % args.causal if args.causal else "")
                                  + (", Q smoothing" if args.smooth_q else "")),
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)"},
        "roofline": dict({"bound": "mfma", "kernel": "k2_attention (rotattn_int4_attention)",
                          "achieved": round(k2_tops, 1), "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                          "frac": round(k2_tops / PEAK_INT8_TOPS, 4),
                          "traffic": counted_traffic() if headline else None},
                         **issued_mfma(ops_q4, k2_ms, stats),
                         **(counted_limiter(N * N * H * B, k2_ms) if headline else {})),
        "skips": stats,
        "kernels_ms": dict({"quantize_qk": round(k1_ms, 4), "int4_attention": round(k2_ms, 4)},
                           **({"fp16_fallback_even_heads": round(k3_ms, 4)} if mixed else {})),
        "quantize_qk_GBps": round(k1_bytes / (k1_ms * 1e-3) / 1e9, 1),
        "attention_only_TOPS": round(k2_tops, 1),
    }

    if not args.no_fallback and not mixed:
        ws = torch.empty(ra.rotattn_fp16_fallback_workspace(shape), dtype=torch.uint8, device="cuda")
        tab0 = ra.rotattn_build_rope_table(shape, 0).cuda()
        ra.rotattn_fp16_fallback(shape, q, k, v, tab0, out, ws, causal_block=args.causal)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 2
        e0.record(stream)
        for _ in range(reps):
            ra.rotattn_fp16_fallback(shape, q, k, v, tab0, out, ws, causal_block=args.causal)
        e1.record(stream)
        torch.cuda.synchronize()
        fb_ms = e0.elapsed_time(e1) / reps
        fb_tops = ops / (fb_ms * 1e-3) / 1e12
        result["fallback"] = {"ms": round(fb_ms, 3), "TFLOPS": round(fb_tops, 1),
                              "frac_f16_peak": round(fb_tops / PEAK_F16_TFLOPS, 4),
                              "int4_attention_speedup": round(fb_ms / k2_ms, 3)}

    if headline and not args.no_diffuse:
        result["diffuse"] = diffuse_floor(shape, rot, q, k, v, tab, z, out, ops, stream)

    if args.torch_sdpa and not mixed and not args.causal:
        result["torch_sdpa"] = torch_sdpa(B, H, N, D, ops, k2_ms)

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg, rot, causal=args.causal)
    print(json.dumps(result))


def torch_sdpa(B, H, N, D, ops, k2_ms) -> dict:
    """torch's scaled-dot-product attention, flash backend forced (no math-path
    fallback), on fp16 random tensors of the workload's shape: context for the FP16
    fallback, not part of the step."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    g = torch.Generator(device="cuda").manual_seed(0)
    q, k, v = (torch.randn((B, H, N, D), dtype=torch.float16, device="cuda", generator=g) for _ in range(3))
    with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
        torch.nn.functional.scaled_dot_product_attention(q, k, v)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 2
        e0.record()
        for _ in range(reps):
            torch.nn.functional.scaled_dot_product_attention(q, k, v)
        e1.record()
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"ms": round(ms, 3), "TFLOPS": round(ops / (ms * 1e-3) / 1e12, 1),
            "int4_attention_speedup": round(ms / k2_ms, 3), "backend": "flash, fp16, torch " + torch.__version__}


def skip_stats(run) -> dict:
    """One untimed attention call with the skip counters: the share of P V units
    skipped because every level is 0, of score tiles whose exps were skipped (below
    half an ulp of l), and of units that took the exact-level path."""
    import torch
    st = torch.zeros(5, dtype=torch.int64, device="cuda")
    run(st)
    torch.cuda.synchronize()
    n = [int(x) for x in st.cpu().tolist()]
    return {"pv_units": n[0], "pv_units_skipped_frac": round(n[1] / max(n[0], 1), 4),
            "exp_tiles_skipped_frac": round(n[3] / max(n[2], 1), 4),
            "exact_path_frac": round(n[4] / max(n[0], 1), 6)}


def issued_mfma(ops, ms, stats) -> dict:
    """The attention's time against the peaks of the MFMA forms it issues: Q K^T on
    fp6 (every score tile is computed) and P V on fp8 (the units not skipped).
    dense_frac prices all of the algorithmic work at those peaks; issued_frac prices
    the work actually issued (roughly the MFMA pipe's busy share)."""
    qk, pv = ops / 2, ops / 2
    t_dense = qk / (PEAK_FP6_TOPS * 1e12) + pv / (PEAK_FP8_TOPS * 1e12)
    t_issued = qk / (PEAK_FP6_TOPS * 1e12) + pv * (1 - stats["pv_units_skipped_frac"]) / (PEAK_FP8_TOPS * 1e12)
    t = ms * 1e-3
    return {"issued_forms": "QK^T fp6 at %.1f PF, PV fp8 at %.1f PF" % (PEAK_FP6_TOPS / 1e3, PEAK_FP8_TOPS / 1e3),
            "dense_frac_at_issued_peaks": round(t_dense / t, 4), "issued_frac_at_issued_peaks": round(t_issued / t, 4)}


def diffuse_floor(shape, rot, q, k, v, tab, z, out, ops, stream) -> dict:
    """The attention on the same shape with the diffuse recipe (no outlier channels,
    unit-variance logits: flat softmax rows, no all-zero units), the floor when the
    exact skips find nothing to skip.  Reuses the input and code buffers."""
    import numpy as np
    import torch
    from int4_quantized_attention_amd import rotattn as ra
    from int4_quantized_attention_amd import synth
    Q, K, V = synth.make_inputs(synth.CONFIGS["wan720p_diffuse"])
    for dst, src in ((q, Q), (k, K), (v, V)):
        dst.copy_(torch.from_numpy(src))
    del Q, K, V
    ra.rotattn_quantize_qk(shape, rot, q, k, v, tab, True, z)
    ra.rotattn_int4_attention(shape, z, out)
    torch.cuda.synchronize()
    reps = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        ra.rotattn_int4_attention(shape, z, out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tops = ops / (ms * 1e-3) / 1e12
    st = skip_stats(lambda s: ra.rotattn_int4_attention(shape, z, out, skip_stats=s))
    return {"recipe": "diffuse: Q, K ~ N(0,1) without outlier channels, V N(0,1) Hadamard-rotated (flat softmax)",
            "int4_attention_ms": round(ms, 3), "TOPS": round(tops, 1), "frac_int8_peak": round(tops / PEAK_INT8_TOPS, 4),
            "skips": st, **issued_mfma(ops, ms, st)}


PEAK_VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9  # CUs x SIMDs x lanes x clock: 39.3e12 lane-ops/s


def counted_limiter(elements: int, k2_ms: float) -> dict:
    """What limits k2_attention, from the committed SQ counter summary (VALU active
    vs MFMA busy share of the launch), and the launch against the VALU roofline (its
    counted VALU lane-ops at one lane-op per lane per clock), or nothing when the
    attention source has changed since the counters were taken."""
    summ = os.path.join(ROOT, "profiles", "k2_attention_wan720p_sq_counters.md")
    try:
        text = open(summ).read()
        cur = attention_source_sha()
    except OSError:
        return {}
    f = dict(l.split(":", 1) for l in text.splitlines()
             if l.startswith(("valu_active_frac:", "mfma_busy_frac:", "valu_lane_ops_per_element:",
                              "attention_source_sha256_16:")))
    if f.get("attention_source_sha256_16", "").strip() != cur or "valu_active_frac" not in f:
        return {}
    valu, mfma = float(f["valu_active_frac"]), float(f["mfma_busy_frac"])
    out = {"limiter": "valu" if valu > mfma else "mfma",
           "counters": {"valu_active_frac": valu, "mfma_busy_frac": mfma}}
    if "valu_lane_ops_per_element" in f:
        ops = float(f["valu_lane_ops_per_element"]) * elements
        floor_ms = ops / PEAK_VALU_LANE_OPS * 1e3
        out["valu_roofline"] = {"lane_ops_per_element": float(f["valu_lane_ops_per_element"]),
                                "lane_ops_per_launch": ops, "peak_lane_ops_per_s": PEAK_VALU_LANE_OPS,
                                "floor_ms": round(floor_ms, 3), "frac": round(floor_ms / k2_ms, 4)}
    return out


def io_label(dtype: str) -> str:
    """Input and output types of the workload (the output is always fp16)."""
    short = {"float16": "fp16", "float32": "fp32", "bfloat16": "bf16"}[dtype]
    return "fp16 in/out" if short == "fp16" else "%s in, fp16 out" % short


ATTENTION_SOURCES = ("attention_impl.h", "attention.hip", "attention_inst.hip")


def attention_source_sha() -> str:
    """First 16 hex digits of the sha256 of the K2 sources, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for name in ATTENTION_SOURCES:
        with open(os.path.join(ROOT, "int4_quantized_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counted_traffic():
    """HBM bytes per k2_attention launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known size), or None when
    the attention source has changed since the counters were taken."""
    summ = os.path.join(ROOT, "profiles", "wan720p_hbm_counters.md")
    try:
        text = open(summ).read()
        cur = attention_source_sha()
    except OSError:
        return None
    fields = dict(l.split(":", 1) for l in text.splitlines()
                  if l.startswith(("traffic_bytes_per_launch:", "attention_source_sha256_16:")))
    if fields.get("attention_source_sha256_16", "").strip() != cur:
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_baseline(cfg, rot, rows_target=40000, causal=0):
    """The oracle on the host cores: quantisation of one head, then quantised
    attention for a bounded sample of that head's query rows; scaled to TOPS."""
    import numpy as np
    from int4_quantized_attention_amd import synth
    from oracle import oracle as orc
    orc.build()
    N, D = synth.n_tokens(cfg), cfg["D"]
    c1 = dict(cfg)
    c1["B"], c1["H"] = 1, 1
    q, k, v = synth.make_head(cfg, 0, 0)
    f = lambda x: x.astype(np.float16)[None, None]
    t0 = time.perf_counter()
    z = orc.quantize(c1, rot, orc.rope_table(c1, rot), f(q), f(k), f(v))
    tq = time.perf_counter() - t0
    rows = np.linspace(0, N - 1, rows_target).astype(np.int64)
    t0 = time.perf_counter()
    orc.attention(c1, z, rows=rows, causal_block=causal)
    ta = time.perf_counter() - t0
    ops = 4.0 * D * float(orc.key_limit(rows, N, causal).sum())
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(ops / ta / 1e12, 6), "unit": "TOPS", "cores": cores, "kind": "oracle",
            "sample": "head 0 of the same workload: quantisation of all %d tokens (%.2f s) and "
                      "attention for %d of its query rows over the keys each sees (%.2f s)" % (N, tq, rows.size, ta)}


if __name__ == "__main__":
    main()
