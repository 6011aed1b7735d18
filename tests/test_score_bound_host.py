"""Host check of the score bound that the attention kernel uses with per-key K
scales (qk_blk < 16): with c_j = fl(fl(sq sk_j) C0) and t_j = fl(A_j c_j), the
bound fl(fl(fl(W sq) C0) f) + 2^-126, W = max_j fl(A_j sk_j), f = 1 +- 2^-20 by the
sign of W, is at least every t_j.  numpy float32 arithmetic rounds to nearest even
like the kernel's binary32 operations."""
import numpy as np

F32 = np.float32


def _bound(A, sk, sq, C0):
    w = (A * sk).astype(F32)
    W = w.max()
    f = F32(1.0 + 2.0 ** -20) if W >= 0 else F32(1.0 - 2.0 ** -20)
    return F32(F32(F32(F32(W * sq) * C0) * f) + F32(2.0 ** -126))


def _tmax(A, sk, sq, C0):
    c = ((sq * sk).astype(F32) * C0).astype(F32)
    return (A * c).astype(F32).max()


def test_score_bound_holds():
    rng = np.random.default_rng(3)
    C0 = F32(np.log2(np.e) / np.sqrt(128.0))
    worst = 0.0
    for it in range(20000):
        n = 16
        A = rng.integers(-6272, 6273, n).astype(F32)
        if it % 3 == 0:
            A = -np.abs(A) - 1  # every score negative
        e = rng.integers(-40, 10) if it % 5 else rng.integers(-140, -120)  # include underflow
        sk = (rng.random(n) * 2.0 ** float(e)).astype(F32)
        sq = F32(rng.random() * 2.0 ** float(rng.integers(-40, 10)))
        t, b = _tmax(A, sk, sq, C0), _bound(A, sk, sq, C0)
        assert b >= t, (it, t, b)
        if np.isfinite(t) and abs(t) >= 2.0 ** -100:  # (the 2^-126 term dominates below)
            worst = max(worst, float((b - t) / abs(t)))
    assert worst < 2.0 ** -18  # tight enough for the skip tests


def test_score_bound_ties_and_zeros():
    C0 = F32(np.log2(np.e) / np.sqrt(64.0))
    for sq in (F32(0.0), F32(1.0), F32(3.0e-39), F32(1e-20)):
        for sk in (np.zeros(16, F32), np.full(16, F32(1e-30)), np.linspace(0, 1, 16, dtype=F32)):
            for A in (np.zeros(16, F32), np.full(16, F32(-7.0)), np.arange(-8, 8, dtype=F32)):
                with np.errstate(all="ignore"):
                    assert _bound(A, sk, sq, C0) >= _tmax(A, sk, sq, C0)
