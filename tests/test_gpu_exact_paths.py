"""GPU tests of the attention's rare and exact-skip branches, through the C ABI.

* The P level decision (rotattn_p_level_probe, the device function the attention
  calls) against the oracle's threshold levels for every binary32 exponent the
  attention can form in [-32, L15 + 2^-5] outside |y| < 2^-12, plus the zeros and
  subnormals.
* A unit whose exact levels are all 0 while the hardware exp reads level 1 at a key
  with y' just below -1 (the tie 2^-1 rounds to 0): the production run skips it,
  the dense debug run adds its exact (zero) levels, and the two outputs must be
  bit-identical, with the debug dumps equal to the oracle's.
* Row maxima of at least 2^18 (fp16-sized Q/K values of about 150), where every
  non-skipped unit takes the exact-level path: dumps bit-exact, production equal to
  debug.
* The skip counters: units visited and units skipped as all-zero equal what the
  oracle's P codes imply.
"""
import numpy as np
import pytest
import torch

from int4_quantized_attention_amd import rotattn as ra
from int4_quantized_attention_amd import synth

import crafted
from gpu_util import assert_close, assert_dumps_equal, debug_run, gpu_quantize, upload_codes

pytestmark = pytest.mark.gpu


def _bits(x):
    return int(np.array([x], np.float32).view(np.uint32)[0])


def test_p_level_sweep(orc):
    """Every binary32 y with |y| in [2^-12, 32] below 0 and [2^-12, L15 + 2^-5] above
    it, and the first 2^20 patterns above +0 and -0: the attention's level decision
    (fast level when its margin is clear, else the threshold fix) and the threshold
    fix on its own both equal the oracle's level."""
    ranges = [(_bits(-2.0 ** -12), _bits(-32.0)), (_bits(2.0 ** -12), _bits(3.9375)),
              (0x00000000, 0x000FFFFF), (0x80000000, 0x800FFFFF)]
    chunk = 1 << 25
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda")
    total = 0
    for lo, hi in ranges:
        print("sweep", hex(lo), hex(hi), flush=True)
        for first in range(lo, hi + 1, chunk):
            n = min(chunk, hi + 1 - first)
            ra.rotattn_p_level_probe(first, n, out)
            got = out[:n].cpu().numpy()
            y = np.arange(first, first + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
            want = orc.p_levels(y).astype(np.uint8)
            dec, fix = got & 0xF, got >> 4
            bad = np.nonzero((dec != want) | (fix != want))[0]
            assert bad.size == 0, "y=%r: decided %d, fixed %d, oracle %d" % (
                float(y[bad[0]]), dec[bad[0]], fix[bad[0]], want[bad[0]])
            total += n
    assert total > 2.5e8


def _exact_case(orc, cfg, zc, **kw):
    """Production and dense debug runs over every row of a hand-built code set:
    dumps equal to the oracle's, outputs within the bar and bit-identical."""
    shape = ra.Shape.of(cfg)
    z = upload_codes(cfg, zc)
    N, D = synth.n_tokens(cfg), cfg["D"]
    out = torch.full((1, 1, N, D), float("nan"), dtype=torch.float32, device="cuda")
    stats = torch.zeros(5, dtype=torch.int64, device="cuda")
    ra.rotattn_int4_attention(shape, z, out, skip_stats=stats, **kw)
    torch.cuda.synchronize()
    od = orc.attention(cfg, zc, dumps=True)
    o1 = out[0, 0].cpu().numpy()
    assert_close(o1, od["out"])
    d, o2 = debug_run(shape, z, out, 0, 0, N, **kw)
    assert_dumps_equal(d, od)
    assert np.array_equal(o1, o2), "production and debug outputs differ"
    return stats.cpu().numpy()


def test_tie_window_unit_is_skipped_exactly(orc):
    cfg, zc, info = crafted.tie_window_case(orc)
    print("tie window key", info, flush=True)
    st = _exact_case(orc, cfg, zc)
    # 8 waves x 4 units; the unit under test (keys 128..191) is skipped in all of them
    assert st[0] == 32 and st[1] >= 8


def test_row_max_guard(orc):
    cfg, zc = crafted.guard_case(orc)
    st = _exact_case(orc, cfg, zc)
    assert st[0] == 4 * 8 and st[4] == st[0] - st[1]  # the guard sends every non-skipped unit to the exact path


def test_skip_counters_match_oracle_codes(orc):
    """Wan-like ragged case (N 1173, kv_blk 64): units visited = waves x steps; units
    skipped = units of fully valid waves whose oracle levels are all 0 (a wave with
    padded rows never skips: their scores are 0 and their levels 15)."""
    cfg = synth.custom(1, 2, 3, 17, 23, 128, 44, 42, 42, 64, 64, dtype="float16", recipe="wan")
    Q, K, V = synth.make_inputs(cfg)
    shape, z = gpu_quantize(cfg, 2, Q, K, V)
    ref = orc.quantize(cfg, 2, orc.rope_table(cfg, 2), Q, K, V)
    N, D, H = synth.n_tokens(cfg), 128, 2
    out = torch.empty((1, H, N, D), dtype=torch.float32, device="cuda")
    stats = torch.zeros(5, dtype=torch.int64, device="cuda")
    ra.rotattn_int4_attention(shape, z, out, skip_stats=stats)
    torch.cuda.synchronize()
    st = stats.cpu().numpy()
    od = orc.attention(cfg, ref, dumps=True)
    lev0 = (od["pcode"] == -8).reshape(H, N, N)
    nsteps = -(-N // 64)
    waves = -(-N // 128) * 4
    want_skip = 0
    for h in range(H):
        for w in range(waves):
            if 32 * w + 31 >= N:
                continue
            for s in range(nsteps):
                want_skip += bool(lev0[h, 32 * w:32 * w + 32, 64 * s:min(N, 64 * s + 64)].all())
    assert st[0] == H * waves * nsteps
    assert st[1] == want_skip
    assert st[2] == 2 * st[0]
    assert 0 <= st[3] <= 2 * st[1] and 0 <= st[4] <= st[0] - st[1]
    print("units %d, all-zero %d, exp tiles skipped %d, exact path %d" % (st[0], st[1], st[3], st[4]))
