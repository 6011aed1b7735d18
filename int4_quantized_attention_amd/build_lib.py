"""Compile the rotattn HIP library for gfx950 (hipcc), in-tree.

    python -m int4_quantized_attention_amd.build_lib

Each source is compiled to an object in parallel, then linked into
``int4_quantized_attention_amd/librotattn.so`` (and the micro-benchmarks of
``kb.hip`` into ``libkb.so``).  Every HIP source is built with
IEEE-exact single precision (no fp contraction, correctly rounded division) so
that the code-deciding arithmetic is bit-reproducible, and with packed fp32
instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "librotattn.so")
KB_OUT = os.path.join(HERE, "libkb.so")  # micro-benchmarks (kb.py), not part of the product library
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.cpp", "quantize.hip", "attention.hip", "fallback.hip"]
# the K2 kernels: attention_inst.hip once per (head dimension, kv step), in parallel
ATT_INSTANCES = [(d, kv) for d in (128, 64) for kv in (64, 128, 256, 32, 16)]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(job) -> str:
    src, defines, tag = job
    obj = os.path.join(BUILD, src + tag + ".o")
    cmd = [HIPCC] + FLAGS + defines + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on %s %s" % (src, " ".join(defines)))
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [("attention_inst.hip", ["-DATT_D=%d" % d, "-DATT_KVB=%d" % kv], ".d%d_kv%d" % (d, kv))
            for d, kv in ATT_INSTANCES] + [(src, [], "") for src in SOURCES] + [("kb.hip", [], "")]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, jobs))
    kb_obj = objs.pop()  # the micro-benchmarks go into a library of their own
    _link(objs, OUT)
    _link([kb_obj], KB_OUT)
    return OUT


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build())
