"""Seeded synthetic inputs for the RotateAttention hot path.

This module holds no arithmetic of the method: it only draws Q, K and V with the
shapes and value structure of the workloads the RotateAttention pages evaluate
(Wan2.2 and HunyuanVideo latent grids, 3D-RoPE channel splits, outlier channels
concentrated in the first half of each RoPE segment, Hadamard-rotated V).  The
same bytes feed the GPU library and the CPU oracle.

Stream layout: one numpy PCG64 stream per (seed, tensor, b, h), tensor ids
Q=0, K=1, V=2, signs=3, so any head can be regenerated on its own.
"""
from __future__ import annotations

import numpy as np

# name -> shape + input recipe.  qk_blk / kv_blk are the scale-block and
# online-softmax step sizes (the tiny case uses 16/16 as its definition states).
CONFIGS = {
    "tiny": dict(B=1, H=2, F=2, Hs=4, Ws=4, D=64, Df=24, Dh=20, Dw=20, qk_blk=16, kv_blk=16,
                 dtype="float32", rot="both", recipe="tiny"),
    "wan480p": dict(B=1, H=12, F=21, Hs=30, Ws=52, D=128, Df=44, Dh=42, Dw=42, qk_blk=64, kv_blk=64,
                    dtype="float16", rot="interleaved", recipe="wan"),
    "wan720p": dict(B=1, H=40, F=21, Hs=45, Ws=80, D=128, Df=44, Dh=42, Dw=42, qk_blk=64, kv_blk=64,
                    dtype="float16", rot="half", recipe="wan"),
    "hunyuan720p": dict(B=1, H=24, F=33, Hs=45, Ws=80, D=128, Df=16, Dh=56, Dw=56, qk_blk=64, kv_blk=64,
                        dtype="float16", rot="interleaved", recipe="hunyuan"),
    "mixed_ragged": dict(B=2, H=12, F=13, Hs=30, Ws=53, D=128, Df=44, Dh=42, Dw=42, qk_blk=64, kv_blk=64,
                         dtype="float16", rot="half", recipe="peaked"),
    # the Wan-720p-like shape on outlier-free inputs: flat, diffuse attention (the
    # text-to-video regime), where no 64-key unit has all its levels 0
    "wan720p_diffuse": dict(B=1, H=40, F=21, Hs=45, Ws=80, D=128, Df=44, Dh=42, Dw=42, qk_blk=64, kv_blk=64,
                            dtype="float16", rot="half", recipe="diffuse"),
}


def n_tokens(cfg) -> int:
    return int(cfg["F"]) * int(cfg["Hs"]) * int(cfg["Ws"])


def _rng(seed: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor, b, h])))


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (power of two), entries +-1."""
    Hm = np.ones((1, 1), dtype=np.float64)
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def _segments(cfg):
    Df, Dh = int(cfg["Df"]), int(cfg["Dh"])
    return [(0, Df), (Df, int(cfg["Dh"])), (Df + Dh, int(cfg["Dw"]))]


def outlier_channels(cfg):
    """Channels drawn heavy-tailed, all in the first half of a RoPE segment."""
    rec = cfg["recipe"]
    segs = _segments(cfg)
    ch = []
    if rec == "tiny":          # 4 per segment, offsets 0..3
        for o, _ in segs:
            ch += [o + i for i in range(4)]
    elif rec == "wan":         # ~8% of channels: round(0.08 * Dj) per segment
        for o, dj in segs:
            ch += [o + i for i in range(int(round(0.08 * dj)))]
    elif rec == "hunyuan":     # ~10%: first 7 of the h segment, first 6 of w
        (_, _), (oh, _), (ow, _) = segs
        ch += [oh + i for i in range(7)] + [ow + i for i in range(6)]
    return ch


def make_head(cfg, b: int, h: int, seed: int = 0):
    """Q, K, V of one head as float32 [N, D] (before the storage cast)."""
    N, D = n_tokens(cfg), int(cfg["D"])
    rec = cfg["recipe"]
    rq, rk, rv, rs = (_rng(seed, t, b, h) for t in range(4))
    q = rq.standard_normal((N, D), dtype=np.float32)
    k = rk.standard_normal((N, D), dtype=np.float32)
    v = rv.standard_normal((N, D), dtype=np.float32)
    ch = outlier_channels(cfg)
    if rec == "tiny":
        q[:, ch] *= 8.0
        k[:, ch] *= 8.0
    elif rec == "wan":
        # heavy channels: sign_c * |N(0, 10^2)|, one sign per (head, channel) shared
        # by Q and K ("matched signs"), magnitudes independent.
        sign = np.where(rs.random(len(ch)) < 0.5, -1.0, 1.0).astype(np.float32)
        q[:, ch] = sign * np.abs(q[:, ch]) * 10.0
        k[:, ch] = sign * np.abs(k[:, ch]) * 10.0
        v = (v.astype(np.float64) @ (hadamard(D) / np.sqrt(D))).astype(np.float32)
    elif rec == "hunyuan":
        q[:, ch] *= 12.0
        k[:, ch] *= 12.0
    elif rec == "peaked":
        q *= 4.0
    elif rec == "diffuse":
        # no outlier channels and unit-variance logits: the softmax of a row is flat
        # over many keys (V Hadamard-rotated as for the Wan recipe)
        v = (v.astype(np.float64) @ (hadamard(D) / np.sqrt(D))).astype(np.float32)
    return q, k, v


def make_inputs(cfg, seed: int = 0, heads=None, threads: int = 16):
    """Full [B, H, N, D] tensors in the config's storage dtype (numpy).
    heads: optional list of flat head ids b*H + h to fill (others left zero).
    Heads are drawn in parallel threads; each head has its own stream, so the
    result does not depend on the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    B, H, D = int(cfg["B"]), int(cfg["H"]), int(cfg["D"])
    N = n_tokens(cfg)
    dt = np.float16 if cfg["dtype"] == "float16" else np.float32
    Q = np.zeros((B, H, N, D), dt)
    K = np.zeros((B, H, N, D), dt)
    V = np.zeros((B, H, N, D), dt)
    todo = [(b, h) for b in range(B) for h in range(H) if heads is None or b * H + h in heads]

    def one(bh):
        b, h = bh
        q, k, v = make_head(cfg, b, h, seed)
        Q[b, h], K[b, h], V[b, h] = q.astype(dt), k.astype(dt), v.astype(dt)

    with ThreadPoolExecutor(max(1, min(threads, len(todo)))) as ex:
        list(ex.map(one, todo))
    return Q, K, V


def custom(B, H, F, Hs, Ws, D, Df, Dh, Dw, qk_blk, kv_blk, dtype="float32", recipe="tiny", rot="half"):
    """A config dict for ad-hoc shapes (tests of ragged tails, odd splits...)."""
    return dict(B=B, H=H, F=F, Hs=Hs, Ws=Ws, D=D, Df=Df, Dh=Dh, Dw=Dw, qk_blk=qk_blk,
                kv_blk=kv_blk, dtype=dtype, rot=rot, recipe=recipe)
