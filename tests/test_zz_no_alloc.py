"""rotattn_quantize_qk_noalloc (the quantiser for callers that cannot allocate,
using the library's fixed per-device scratch) against rotattn_quantize_qk with a
caller workspace, through the C ABI: two calls in a row, the second with a smaller
input, each bit-identical to the workspace call on the same input (codes, scales,
column sums); a shape whose scratch exceeds the fixed array is refused before any
launch."""
import ctypes

import numpy as np
import pytest
import torch

from int4_quantized_attention_amd import rotattn as ra
from int4_quantized_attention_amd import synth

pytestmark = pytest.mark.gpu

KEYS = ("q_codes", "q_scale", "k_codes", "k_scale", "v_codes", "v_scale", "v_colsum")


def _both(cfg, rot, seed):
    shape = ra.Shape.of(cfg)
    Q, K, V = synth.make_inputs(cfg, seed=seed)
    q, k, v = (torch.from_numpy(x).cuda() for x in (Q, K, V))
    tab = ra.rotattn_build_rope_table(shape, rot).cuda()
    za = ra.alloc_codes(shape)
    zb = ra.alloc_codes(shape)
    for t in KEYS:  # different garbage in the two sets, so nothing passes by accident
        za[t].fill_(7 if za[t].dtype == torch.uint8 else 3)
        zb[t].fill_(9 if zb[t].dtype == torch.uint8 else -5)
    ra.rotattn_quantize_qk(shape, rot, q, k, v, tab, True, za)
    ra.rotattn_quantize_qk_noalloc(shape, rot, q, k, v, tab, True, zb)
    torch.cuda.synchronize()
    for t in KEYS:
        assert torch.equal(za[t], zb[t]), t
    return shape, za, zb


def test_noalloc_matches_workspace_call_twice():
    big = synth.custom(2, 3, 5, 17, 23, 128, 44, 42, 42, 64, 256, dtype="float16", recipe="wan", rot="half")
    small = synth.custom(1, 2, 3, 5, 7, 64, 24, 20, 20, 1, 16, dtype="float32", recipe="tiny", rot="interleaved")
    print("case noalloc big", flush=True)
    shape, za, zb = _both(big, 2, seed=3)
    # the attention on the no-allocation codes equals the one on the workspace codes
    N = synth.n_tokens(big)
    oa = torch.empty((2, 3, N, 128), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    ra.rotattn_int4_attention(shape, za, oa)
    ra.rotattn_int4_attention(shape, zb, ob)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    print("case noalloc small", flush=True)
    _both(small, 1, seed=4)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    L = ra.lib()
    cap = L.rotattn_quantize_qk_noalloc_max_scratch()
    assert cap == 64 << 20
    ok = ra.Shape.of(synth.CONFIGS["wan720p"])
    assert 48e6 < L.rotattn_quantize_qk_noalloc_scratch(ctypes.byref(ok)) <= cap
    too_big = ra.Shape.of(dict(synth.CONFIGS["wan720p"], H=64))
    assert L.rotattn_quantize_qk_noalloc_scratch(ctypes.byref(too_big)) > cap
    fake = ctypes.c_void_p(16)  # never dereferenced: the size check comes first
    st = L.rotattn_quantize_qk_noalloc(ctypes.byref(too_big), 2, 1, fake, fake, fake, fake, 1, fake, fake, fake,
                                       fake, fake, fake, None, None)
    assert st == 4  # ROTATTN_E_WORKSPACE
