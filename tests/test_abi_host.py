"""Host-only checks of the C ABI (no GPU): the library loads, exports every symbol
the header declares, validates arguments before any launch, and its host-built
RoPE tables equal the oracle's bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

from int4_quantized_attention_amd import rotattn as ra
from int4_quantized_attention_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rotattn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ra.LIB_PATH):
        from int4_quantized_attention_amd import build_lib
        build_lib.build()
    return ra.lib()


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(rotattn_[a-z0-9_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n


def _shape(**kw):
    cfg = dict(synth.CONFIGS["tiny"])
    cfg.update(kw)
    return ra.Shape.of(cfg)


def test_check_shape_statuses(L):
    assert ra.rotattn_check_shape(_shape()) == 0
    assert ra.rotattn_check_shape(_shape(Df=26)) == 2          # D != Df+Dh+Dw
    assert ra.rotattn_check_shape(_shape(Df=23, Dh=21)) == 2   # odd segments
    assert ra.rotattn_check_shape(_shape(D=96, Df=32, Dh=32, Dw=32)) == 3
    assert ra.rotattn_check_shape(_shape(qk_blk=1)) == 0       # per-token scales
    assert ra.rotattn_check_shape(_shape(qk_blk=8)) == 0
    assert ra.rotattn_check_shape(_shape(kv_blk=256)) == 0
    assert ra.rotattn_check_shape(_shape(qk_blk=3)) == 3
    assert ra.rotattn_check_shape(_shape(qk_blk=256)) == 3
    assert ra.rotattn_check_shape(_shape(kv_blk=8)) == 3
    assert ra.rotattn_check_shape(_shape(kv_blk=512)) == 3
    assert ra.rotattn_check_shape(_shape(F=0)) == 2
    assert L.rotattn_check_shape(None) == 1


def test_padded_tokens_and_workspace(L):
    s = ra.Shape.of(synth.CONFIGS["wan720p"])
    assert ra.rotattn_padded_tokens(s) == 75776
    assert ra.rotattn_quantize_qk_workspace(s) > 0
    assert ra.rotattn_fp16_fallback_workspace(s) >= 3 * 40 * 75776 * 128 * 2
    # one LDS image per 128-key group: K rows of packed fp6 (3D/4 bytes) + 16 pad,
    # V^T rows of 128+16 bytes, a 128-byte table, rounded up to 4 KiB
    img = -(-(128 * (96 + 16) + 128 * (128 + 16) + 128) // 4096) * 4096
    assert img == 36864
    assert ra.rotattn_int4_attention_workspace(s) == 40 * (75776 // 128) * img


def test_null_and_bad_args_return_before_launch(L):
    s = _shape()
    nul = None
    st = L.rotattn_quantize_qk(ctypes.byref(s), 1, 0, nul, nul, nul, nul, 1, nul, nul, nul, nul, nul,
                               nul, nul, nul, 0, nul)
    assert st == 1
    st = L.rotattn_int4_attention(ctypes.byref(s), nul, nul, nul, nul, nul, nul, nul, 0, 0, nul, nul, nul, 0,
                                  nul)
    assert st == 1
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    bad_heads = (ctypes.c_int32 * 1)(5)  # B*H = 2
    big = 1 << 40
    st = L.rotattn_int4_attention(ctypes.byref(s), fake, fake, fake, fake, fake, fake, bad_heads, 1, 0,
                                  fake, nul, fake, big, nul)
    assert st == 6
    st = L.rotattn_int4_attention(ctypes.byref(s), fake, fake, fake, fake, fake, fake, nul, 0, 0,
                                  fake, nul, fake, 64, nul)
    assert st == 4  # attention workspace too small
    st = L.rotattn_int4_attention(ctypes.byref(s), fake, fake, fake, fake, fake, fake, nul, 0, 0,
                                  fake, nul, ctypes.c_void_p(24), big, nul)
    assert st == 4  # attention workspace not 16-byte aligned
    st = L.rotattn_quantize_qk(ctypes.byref(s), 1, 0, fake, fake, fake, fake, 1, fake, fake, fake, fake,
                               fake, fake, nul, fake, 16, nul)
    assert st == 4  # workspace too small
    st = L.rotattn_fp16_fallback(ctypes.byref(s), 7, fake, fake, fake, fake, nul, 0, 0, fake, fake,
                                 1 << 30, nul)
    assert st == 6  # input dtype outside F32 / F16 / BF16
    st = L.rotattn_fp16_fallback(ctypes.byref(s), 2, fake, fake, fake, fake, nul, 0, 5, fake, fake,
                                 1 << 30, nul)
    assert st == 6  # output dtype outside F32 / F16 / BF16
    st = L.rotattn_int4_attention(ctypes.byref(s), fake, fake, fake, fake, fake, fake, nul, 0, 3,
                                  fake, nul, fake, big, nul)
    assert st == 6  # output dtype outside F32 / F16 / BF16
    # options: negative causal block, P maximum other than 15 / 7
    for opts in (ra.AttentionOpts(15, -1, None), ra.AttentionOpts(8, 4, None)):
        st = L.rotattn_int4_attention_ex(ctypes.byref(s), fake, fake, fake, fake, fake, fake, nul, 0,
                                         ctypes.byref(opts), 0, fake, nul, fake, big, nul)
        assert st == 6
    # Q smoothing without its k_bias output; lengths outside [1, N]; too many elements
    bad_len = (ctypes.c_int32 * 1)(0)
    big_len = (ctypes.c_int32 * 1)(10 ** 6)
    for opts, want in ((ra.QuantizeOpts(1, 1, None, None), 1),
                       (ra.QuantizeOpts(1, 0, None, ctypes.cast(bad_len, ctypes.c_void_p)), 6),
                       (ra.QuantizeOpts(1, 0, None, ctypes.cast(big_len, ctypes.c_void_p)), 6)):
        st = L.rotattn_quantize_qk_ex(ctypes.byref(s), 1, 0, fake, fake, fake, fake, ctypes.byref(opts), fake,
                                      fake, fake, fake, fake, fake, nul, fake, 1 << 30, nul)
        assert st == want
    s65 = _shape(B=65)
    lens65 = (ctypes.c_int32 * 65)(*([1] * 65))
    opts = ra.AttentionOpts(15, 0, None, ctypes.cast(lens65, ctypes.c_void_p))
    st = L.rotattn_int4_attention_ex(ctypes.byref(s65), fake, fake, fake, fake, fake, fake, nul, 0,
                                     ctypes.byref(opts), 0, fake, nul, fake, big, nul)
    assert st == 3
    st = L.rotattn_fp16_fallback_ex(ctypes.byref(s), 1, fake, fake, fake, fake, nul, 0,
                                    ctypes.byref(ra.FallbackOpts(0, ctypes.cast(bad_len, ctypes.c_void_p))),
                                    0, fake, fake, 1 << 30, nul)
    assert st == 6
    st = L.rotattn_fp16_fallback_ex(ctypes.byref(s), 1, fake, fake, fake, fake, nul, 0,
                                    ctypes.byref(ra.FallbackOpts(-3, None)), 0, fake, fake, 1 << 30, nul)
    assert st == 6
    assert L.rotattn_status_str(0) == b"ok"


def test_images_beyond_a_32bit_range_per_head_are_unsupported(L):
    """A head's group images are addressed through a buffer resource with a 32-bit
    range: shapes whose images exceed 2^31 bytes per head return UNSUPPORTED before
    any launch (the fallback keeps 36 KiB per 64 keys at D = 128, the INT4 path 36 KiB
    per 128 keys)."""
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    nul = None
    big = 1 << 44
    base = dict(synth.CONFIGS["wan720p"], B=1, H=1, F=1, Hs=2048, Ws=2048)  # N = 4.19M tokens
    s = ra.Shape.of(base)
    assert ra.rotattn_check_shape(s) == 0
    st = L.rotattn_fp16_fallback(ctypes.byref(s), 1, fake, fake, fake, fake, nul, 0, 1, fake, fake, big, nul)
    assert st == 3
    # the INT4 images still fit at this length, so the call gets as far as the
    # workspace check; at twice the length they do not
    st = L.rotattn_int4_attention(ctypes.byref(s), fake, fake, fake, fake, fake, fake, nul, 0, 0,
                                  fake, nul, fake, 64, nul)
    assert st == 4
    s2 = ra.Shape.of(dict(base, F=2))
    st = L.rotattn_int4_attention(ctypes.byref(s2), fake, fake, fake, fake, fake, fake, nul, 0, 0,
                                  fake, nul, fake, big, nul)
    assert st == 3


@pytest.mark.parametrize("cfgname", ["tiny", "wan480p", "hunyuan720p"])
@pytest.mark.parametrize("rot", [0, 1, 2])
def test_rope_table_matches_oracle(L, orc, cfgname, rot):
    cfg = synth.CONFIGS[cfgname]
    mine = ra.rotattn_build_rope_table(ra.Shape.of(cfg), rot).numpy()
    ref = orc.rope_table(cfg, rot)
    assert mine.shape == ref.shape
    assert np.array_equal(mine.view(np.uint32), ref.view(np.uint32))


def test_plain_c_caller(tmp_path):
    """The header is a C ABI: a strict C99 program (tests/c_abi_host.c) compiles
    against it with every warning as an error, links the library, and its host-side
    calls answer as documented."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "int4_quantized_attention_amd")
    exe = str(tmp_path / "c_abi_host")
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                         "-I" + os.path.join(root, "include"), os.path.join(root, "tests", "c_abi_host.c"),
                         "-L" + pkg, "-lrotattn", "-Wl,-rpath," + pkg, "-o", exe], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, "check %d failed" % run.returncode
    assert run.stdout.strip() == "c abi ok"
