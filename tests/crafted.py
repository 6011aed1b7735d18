"""Hand-built INT4 code sets that drive the attention into its rare branches (input
generators only: integer codes and scales chosen on the host, no arithmetic of the
method beyond locating the inputs).

  guard_case()       row maxima of at least 2^18 in log2 units, where the kernel
                     sends every non-skipped unit down the exact-level path;
  tie_window_case()  a 64-key unit whose largest exponent y' lies in
                     [-1 - 1.7e-5, -1]: its exact levels are all 0 (2^-1 is a tie
                     that rounds to even, and anything below rounds down), while the
                     hardware-exp level of that key reads 1 with an unclear margin.
                     The running maximum moved before it, so the output accumulator
                     holds non-integers when the unit comes up.

Exponents are located with y' = fma(A, c, fl(L15 - m)) evaluated exactly: A c is
exact in binary64 (|A| < 2^13, c a binary32), the sum with a binary32 is exact in
binary64 at these magnitudes, and one rounding to binary32 is the fused result.
"""
import numpy as np

from int4_quantized_attention_amd import synth


def fma32(a, c, b):
    return np.float32(np.float64(a) * np.float64(c) + np.float64(b))


def _k_rows_with_sums(sums, D, rng):
    """Rows of D codes in [-7, 7] whose sums are the given integers (|s| <= 7 D),
    with the mass spread over random channels."""
    out = np.zeros((len(sums), D), np.int8)
    for i, s in enumerate(sums):
        sign = 1 if s >= 0 else -1
        left = abs(int(s))
        order = rng.permutation(D)
        for d in order:
            if left == 0:
                break
            t = min(7, left)
            out[i, d] = sign * t
            left -= t
        assert left == 0
    return out


def tie_window_case(orc, seed=0):
    """B1 H1, grid 1x8x32 (N 256), D 128, qk_blk 16, kv_blk 64.  Every query row has
    all codes 1 and scale 1, so A_j is the sum of key j's codes and c = fl(sk C0) is
    the same for every key.  Steps: 0 sets the maximum with A = 400; 1 raises it to
    A = 470 (a rescale by a non-power of two); 2 holds the unit under test, one key
    in the tie window and the rest far below it; 3 adds non-zero levels again."""
    rng = np.random.default_rng(seed)
    cfg = synth.custom(1, 1, 1, 8, 32, 128, 44, 42, 42, 16, 64, dtype="float32", recipe="tiny", rot="none")
    N, D = 256, 128
    C0, L15 = np.float32(orc.c0(D)), np.float32(orc.l15())
    lo_win, hi_win = np.float32(-1.000017), np.float32(-1.0)
    found = None
    sk = np.float32(0.05)
    for _ in range(20000):
        sk = np.nextafter(sk, np.float32(1))
        c = np.float32(np.float32(np.float32(1.0) * sk) * C0)
        m = np.float32(np.float32(470) * c)
        nm = np.float32(L15 - m)
        a0 = int(np.floor((np.float64(m) - np.float64(L15) - 1.0) / np.float64(c)))
        for A in (a0 - 1, a0, a0 + 1):
            y = fma32(A, c, nm)
            if lo_win <= y <= hi_win:
                found = (sk, c, m, A, y)
                break
        if found:
            break
    assert found, "no scale puts an integer score in the tie window"
    sk, c, m, Aw, yw = found
    A = np.empty(N, np.int64)
    A[0:64] = rng.integers(250, 380, 64)
    A[5] = 400
    A[64:128] = rng.integers(250, 460, 64)
    A[70] = 470
    A[128:192] = rng.integers(Aw - 400, Aw - 12, 64)   # y' <= -1 - 0.07: level 0, clear margins
    kw = 128 + 37                                        # lane half 0 of tile 5
    A[kw] = Aw
    A[192:256] = rng.integers(300, 468, 64)
    kc = _k_rows_with_sums(A, D, rng)
    qc = np.ones((N, D), np.int8)
    vc = rng.integers(-7, 8, (N, D)).astype(np.int8)
    z = dict(qc=qc[None, None], kc=kc[None, None], vc=vc[None, None],
             qs=np.ones((1, 1, N // 16), np.float32), ks=np.full((1, 1, N // 16), sk, np.float32),
             vs=np.ones((1, 1, D), np.float32))
    info = dict(key=kw, y=float(yw), A=int(Aw), c=float(c), m=float(m))
    return cfg, z, info


def guard_case(orc, seed=0):
    """B1 H1, grid 1x4x64 (N 256), D 128, qk_blk 16, kv_blk 64.  Query codes all 7
    with scale 150/7 (the codes of fp16 values of about 150), so A_j = 7 x the sum of
    key j's codes.  Key block 0 holds the largest score (A = 6272 with c about 58.6:
    m is about 3.7e5 >= 2^18); every other 16-key block gets the K scale that puts
    its largest score 0.2 to 8 (log2 units) below m, so that levels from 0 to 15
    occur."""
    rng = np.random.default_rng(seed)
    cfg = synth.custom(1, 1, 1, 4, 64, 128, 44, 42, 42, 16, 64, dtype="float32", recipe="tiny", rot="none")
    N, D = 256, 128
    C0 = np.float32(orc.c0(D))
    sq = np.float32(150.0 / 7.0)
    nb = N // 16
    S = np.empty(N, np.int64)                 # key code sums; A = 7 S
    S[0:16] = 896 - rng.integers(0, 3, 16)
    S[3] = 896
    ks = np.empty(nb, np.float32)
    ks[0] = sq
    c0 = np.float32(np.float32(sq * ks[0]) * C0)
    m = np.float64(np.float32(np.float32(7 * 896) * c0))
    for b in range(1, nb):
        S[16 * b:16 * b + 16] = 700 + rng.integers(0, 150, 16)
        top = 7 * int(S[16 * b:16 * b + 16].max())
        delta = rng.uniform(0.2, 8.0)
        ks[b] = np.float32((m - delta) / (top * np.float64(sq) * np.float64(C0)))
    kc = _k_rows_with_sums(S, D, rng)
    qc = np.full((N, D), 7, np.int8)
    vc = rng.integers(-7, 8, (N, D)).astype(np.int8)
    z = dict(qc=qc[None, None], kc=kc[None, None], vc=vc[None, None],
             qs=np.full((1, 1, nb), sq, np.float32), ks=ks[None, None], vs=np.full((1, 1, D), 0.25, np.float32))
    return cfg, z
