"""Micro-benchmarks of one MI355X (libkb.so, built with the library):

* back-to-back MFMA throughput of each instruction form the kernels use, against
  the published dense peaks;
* HBM streaming bandwidth (16-byte copy and read);
* LDS read bandwidth (ds_read_b128), alone and feeding one f16 MFMA per kilobyte
  read (an attention kernel's ratio with 32 query rows per wave);
* the error of the hardware exp2 (v_exp_f32) over every binary32 exponent the P
  level code meets, in units of 2^-24 relative, against binary64 exp2.

    python -m int4_quantized_attention_amd.kb [--quick]

Prints a table and one JSON line.  Inputs are synthetic; nothing here uses the
attention library.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkb.so")

# form -> (name, ops per instruction 2*M*N*K, published dense peak in TOPS)
FORMS = {
    0: ("i8 32x32x32", 2 * 32 * 32 * 32, 5000.0),
    1: ("f16 32x32x16", 2 * 32 * 32 * 16, 2500.0),
    2: ("bf16 32x32x16", 2 * 32 * 32 * 16, 2500.0),
    3: ("fp8 e4m3 32x32x64", 2 * 32 * 32 * 64, 5000.0),
    4: ("fp6 e2m3 32x32x64", 2 * 32 * 32 * 64, 10100.0),
    5: ("fp4 e2m1 32x32x64", 2 * 32 * 32 * 64, 10100.0),
}
HBM_PEAK_GBPS = 8000.0


def lib():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkb.so is not built (python -m int4_quantized_attention_amd.build_lib)")
    L = ctypes.CDLL(LIB_PATH)
    VP, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.kb_mfma_launch.argtypes = [I32, I32, I32, VP, VP]
    L.kb_copy_launch.argtypes = [VP, VP, I64, I32, VP]
    L.kb_read_launch.argtypes = [VP, I64, I32, VP, VP]
    L.kb_exp2_launch.argtypes = [ctypes.c_uint32, I64, VP, VP]
    L.kb_lds_launch.argtypes = [I32, I32, I32, VP, VP, VP]
    return L


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _time(fn, reps=3):
    """Best of reps, ms (HIP events on the current stream)."""
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return best


def mfma_rates(L, blocks=1024, iters=50000):
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    chains = L.kb_mfma_chains()
    res = {}
    for form, (name, ops, peak) in FORMS.items():
        run = lambda: L.kb_mfma_launch(form, blocks, iters, ctypes.c_void_p(out.data_ptr()), _stream())
        assert run() == 0
        torch.cuda.synchronize()
        ms = _time(lambda: run())
        tops = blocks * 4 * chains * iters * ops / (ms * 1e-3) / 1e12
        res[name] = {"TOPS": round(tops, 1), "frac_of_published_peak": round(tops / peak, 4), "ms": round(ms, 3)}
    return res


def hbm_rates(gib=4):
    L = lib()
    n = gib << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    blocks = 256 * 8 * 4
    part = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    sp, dp = ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr())
    assert L.kb_copy_launch(sp, dp, n, blocks, _stream()) == 0
    ms_c = _time(lambda: L.kb_copy_launch(sp, dp, n, blocks, _stream()))
    ms_r = _time(lambda: L.kb_read_launch(sp, n, blocks, ctypes.c_void_p(part.data_ptr()), _stream()))
    return {"copy_GBps": round(2 * n / (ms_c * 1e-3) / 1e9, 1), "read_GBps": round(n / (ms_r * 1e-3) / 1e9, 1),
            "bytes": n}


def lds_rates(L, iters=20000):
    """LDS read bandwidth, alone and feeding f16 MFMAs, with one and two workgroups
    of 4 waves (64 KiB of LDS each) per CU.  Bytes per clock per CU come from the
    shader clocks each workgroup counts around its loop; the GB/s from HIP events."""
    res = {}
    for mode, name in ((0, "reads"), (1, "reads+f16 mfma")):
        for per_cu in (1, 2):
            blocks = 256 * per_cu
            out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            cyc = torch.zeros(blocks, dtype=torch.int64, device="cuda")
            run = lambda: L.kb_lds_launch(mode, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                          ctypes.c_void_p(cyc.data_ptr()), _stream())
            assert run() == 0
            torch.cuda.synchronize()
            ms = _time(run)
            wg_bytes = 4 * iters * 8 * 1024
            clocks = float(cyc.double().median())
            r = {"GBps": round(blocks * wg_bytes / (ms * 1e-3) / 1e9, 1),
                 "bytes_per_clock_per_cu": round(per_cu * wg_bytes / clocks, 1), "ms": round(ms, 3)}
            if mode == 1:
                r["TFLOPS"] = round(blocks * 4 * iters * 8 * 2 * 32 * 32 * 16 / (ms * 1e-3) / 1e12, 1)
            res["%s, %d workgroup%s per CU" % (name, per_cu, "s" if per_cu > 1 else "")] = r
    return res


def exp2_error(lo=-4.0, hi=4.0, skip_below=2.0 ** -12, chunk=1 << 25):
    """Largest relative error of v_exp_f32 over every binary32 y in [lo, hi] with
    |y| >= skip_below, in units of 2^-24."""
    L = lib()
    bits = lambda x: int(np.array([x], np.float32).view(np.uint32)[0])
    ranges = [(bits(-skip_below), bits(lo)), (bits(skip_below), bits(hi))]
    out = torch.empty(chunk, dtype=torch.float32, device="cuda")
    worst, worst_y, count = 0.0, 0.0, 0
    for a, b in ranges:
        for first in range(a, b + 1, chunk):
            n = min(chunk, b + 1 - first)
            assert L.kb_exp2_launch(first, n, ctypes.c_void_p(out.data_ptr()), _stream()) == 0
            p = out[:n].cpu().numpy().astype(np.float64)
            y = np.arange(first, first + n, dtype=np.uint64).astype(np.uint32).view(np.float32).astype(np.float64)
            ref = np.exp2(y)
            err = np.abs(p - ref) / ref * 2.0 ** 24
            i = int(np.argmax(err))
            if err[i] > worst:
                worst, worst_y = float(err[i]), float(y[i])
            count += n
    return {"max_rel_err_units_2^-24": round(worst, 4), "at_y": worst_y, "values": count,
            "range": "binary32 y in [%g, %g], |y| >= %g" % (lo, hi, skip_below)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true", help="shorter MFMA loops and a 1 GiB stream")
    args = ap.parse_args()
    torch.cuda.set_device(0)
    L = lib()
    res = {"mfma": mfma_rates(L, iters=5000 if args.quick else 50000),
           "hbm": hbm_rates(1 if args.quick else 4),
           "lds": lds_rates(L, iters=2000 if args.quick else 20000),
           "exp2": exp2_error()}
    for name, r in res["mfma"].items():
        print("MFMA %-20s %9.1f TOPS  %5.1f%% of the published dense peak" % (name, r["TOPS"],
                                                                            100 * r["frac_of_published_peak"]))
    h = res["hbm"]
    print("HBM copy %.1f GB/s (%.1f%% of 8 TB/s), read %.1f GB/s (%.1f%%)" % (
        h["copy_GBps"], 100 * h["copy_GBps"] / HBM_PEAK_GBPS, h["read_GBps"], 100 * h["read_GBps"] / HBM_PEAK_GBPS))
    for name, r in res["lds"].items():
        print("LDS %-36s %8.1f GB/s  %6.1f B/clock/CU%s" % (
            name, r["GBps"], r["bytes_per_clock_per_cu"], ("  %.1f TFLOPS" % r["TFLOPS"]) if "TFLOPS" in r else ""))
    e = res["exp2"]
    print("v_exp_f32: max relative error %.4f x 2^-24 at y = %r over %d values" % (
        e["max_rel_err_units_2^-24"], e["at_y"], e["values"]))
    print(json.dumps(res))


if __name__ == "__main__":
    sys.exit(main())
