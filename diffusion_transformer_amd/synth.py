"""Seeded synthetic inputs for the DiT hot path (no method arithmetic here).

This module only draws random numbers and rounds them to bf16-representable
values; it computes nothing of the method.  The GPU tests, the benchmark and
the oracle's tests all take their inputs from here, so both sides see the same
numbers.  Every array is returned as float32 values (exactly representable in
bf16 where the GPU stores bf16), plus int8 codes for the int8 weight format.

Workloads (shapes follow the pages' 512- and 1024-pixel DiT: hidden 3072,
24 heads of 128, one image token per 16x16 px tile, at most 512 text rows):
  tiny        hidden 256, 2 heads x 128, ffn 1024, L=8 text + 8x8 image rows
  s1088       hidden 3072, 24 x 128, ffn 12288, L=64 + 32x32 (512 px)
  s4608       hidden 3072, 24 x 128, ffn 12288, L=512 + 64x64 (1024 px)
  s4608_int8  s4608 with the four linears as int8 + one bf16 scale per 32
  dit32       32 blocks of s4608, latent 64 channels, text features 4096-d
Weights ~ N(0, 0.02); activations and text features ~ N(0, 1); norm weights
1 unless asked otherwise; int8 codes uniform in [-127, 127] and their scales
|N(0, 1)| * 0.01.
"""

from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np


def _round_inplace(u: np.ndarray) -> np.ndarray:
    """u: uint32 view of float32 values; rounds them in place to bf16
    (round to nearest, ties to even; finite inputs) and returns u."""
    t = u >> 16
    t &= 1
    t += np.uint32(0x7FFF)
    u += t
    u &= np.uint32(0xFFFF0000)
    return u


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 array of the bf16-rounded values of a (a copy)."""
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    return _round_inplace(u).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The 16-bit patterns (uint16) of the bf16-rounded values of a."""
    return (bf16_round(a).view(np.uint32) >> 16).astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """float32 values of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Shape:
    name: str
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    L: int
    h: int
    w: int
    seed: int
    int8: bool = False
    blocks: int = 1
    w8a8: bool = False
    latent: int = 64
    text_dim: int = 4096
    time_dim: int = 256
    axes: tuple = (16, 56, 56)

    @property
    def N(self) -> int:
        return self.h * self.w

    @property
    def S(self) -> int:
        return self.L + self.N


SHAPES = {
    "tiny": Shape("tiny", 256, 2, 128, 1024, 8, 8, 8, seed=0),
    # the smallest sequences the block takes: image rows only, one row, and
    # fewer rows than one 16-row matrix block
    "t_img": Shape("t_img", 256, 2, 128, 1024, 0, 8, 8, seed=21),
    "t_one": Shape("t_one", 256, 2, 128, 1024, 0, 1, 1, seed=22),
    "t_few": Shape("t_few", 256, 2, 128, 1024, 3, 1, 2, seed=23),
    "s1088": Shape("s1088", 3072, 24, 128, 12288, 64, 32, 32, seed=2),
    # another width: 12 heads, ffn 6144, 40 text + 20x30 image rows
    "m640": Shape("m640", 1536, 12, 128, 6144, 40, 20, 30, seed=24),
    # wider than 3072: 32 heads, ffn 16384, tiny's rows
    "w4096": Shape("w4096", 4096, 32, 128, 16384, 8, 8, 8, seed=25),
    "r1077": Shape("r1077", 3072, 24, 128, 12288, 77, 25, 40, seed=11),
    "s4608": Shape("s4608", 3072, 24, 128, 12288, 512, 64, 64, seed=3),
    "s4608_int8": Shape("s4608_int8", 3072, 24, 128, 12288, 512, 64, 64, seed=4, int8=True),
    "s4608_w8a8": Shape("s4608_w8a8", 3072, 24, 128, 12288, 512, 64, 64, seed=6, w8a8=True),
    "dit32": Shape("dit32", 3072, 24, 128, 12288, 512, 64, 64, seed=5, blocks=32),
}


_CHUNK = 1 << 22
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1)))
    return _POOL


def _normal(rng, shape, std):
    """bf16-rounded N(0, std^2) draws.  Large arrays are filled in chunks of
    4 Mi values, chunk i from its own generator seeded with (s, i) where s is
    drawn from `rng`, so the result is the same whatever the thread count."""
    a = np.empty(shape, dtype=np.float32)
    flat = a.reshape(-1)
    s = int(rng.integers(0, 2 ** 62))
    n = flat.size

    def fill(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.default_rng([s, i])
        part = flat[lo:hi]
        g.standard_normal(hi - lo, dtype=np.float32, out=part)
        part *= np.float32(std)
        _round_inplace(part.view(np.uint32))

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        fill(0) if n else None
    else:
        list(_pool().map(fill, range(nchunks)))
    return a


def int8_weight(rng, out: int, inn: int):
    """int8 codes uniform in [-127, 127] [out, in] and bf16 scales
    |N(0,1)| * 0.01, one per 32 inputs [out, in/32] (float32 values)."""
    q = rng.integers(-127, 128, size=(out, inn), dtype=np.int8)
    s = bf16_round(np.abs(rng.standard_normal((out, inn // 32), dtype=np.float32)) * np.float32(0.01))
    return q, s


def w8a8_weight(rng, out: int, inn: int, std=0.02):
    """INT8 rows q ~ U{-127..127} [out, in] and one fp32 scale a row [out],
    std * sqrt(3) / 127 * (1 + N(0, 0.1^2)), so the weights' spread is about
    std."""
    q = rng.integers(-127, 128, (out, inn), dtype=np.int8)
    s = (np.float32(std * np.sqrt(3.0) / 127.0) * (1.0 + 0.1 * rng.standard_normal(out, dtype=np.float32)))
    return q, s.astype(np.float32)


def block_weights(rng, sh: Shape, std=0.02, norm_std=0.0, int8=None, rms=False, sandwich=False, w8a8=None):
    """Weights of one block as a dict of float32 arrays (bf16 values).
    Keys: w_qkv [3D, D], w_out [D, D], w_up [2F, D], w_down [D, F],
    w_mod [6D, D], q_norm [hd], k_norm [hd] and, with rms=True, norm1/norm2
    [D].  With int8, the four linears are replaced by (codes, scales) pairs
    under keys q_<name> and s_<name>; with w8a8, by INT8 rows and fp32 row
    scales (w8a8_weight) under q8_<name> and s8_<name>.  With sandwich=True, the post norms'
    weights post_attn/post_mlp [D] ~ N(1, 0.2^2), drawn last."""
    D, F, hd = sh.hidden, sh.ffn, sh.head_dim
    int8 = sh.int8 if int8 is None else int8
    w8a8 = sh.w8a8 if w8a8 is None else w8a8
    dims = {"w_qkv": (3 * D, D), "w_out": (D, D), "w_up": (2 * F, D), "w_down": (D, F)}
    out = {}
    for k, (o, i) in dims.items():
        if w8a8:
            out["q8_" + k], out["s8_" + k] = w8a8_weight(rng, o, i, std)
        elif int8:
            out["q_" + k], out["s_" + k] = int8_weight(rng, o, i)
        else:
            out[k] = _normal(rng, (o, i), std)
    out["w_mod"] = _normal(rng, (6 * D, D), std)

    def normw(n):
        if norm_std == 0.0:
            return np.ones(n, np.float32)
        return bf16_round(1.0 + rng.standard_normal(n, dtype=np.float32) * np.float32(norm_std))

    out["q_norm"] = normw(hd)
    out["k_norm"] = normw(hd)
    if rms:
        out["norm1"] = normw(D)
        out["norm2"] = normw(D)
    if sandwich:
        for k in ("post_attn", "post_mlp"):
            out[k] = bf16_round(1.0 + rng.standard_normal(D, dtype=np.float32) * np.float32(0.2))
    return out


def block_case(name: str = "tiny", seed=None, norm_std=0.0, rms=False, t=None, sandwich=False, w8a8=None):
    """Inputs of one block forward: rows x [S, D] ~ N(0,1) (float32, fp32 on
    the GPU too), the time t (0.5 for `tiny`, else U(0,1)), the time MLP
    weights w_t1 [D, 256] and w_t2 [D, D], and the block's weights."""
    sh = SHAPES[name]
    rng = np.random.default_rng(sh.seed if seed is None else seed)
    x = rng.standard_normal((sh.S, sh.hidden), dtype=np.float32)
    if t is None:
        t = 0.5 if name == "tiny" else float(rng.uniform(0.0, 1.0))
    w_t1 = _normal(rng, (sh.hidden, sh.time_dim), 0.02)
    w_t2 = _normal(rng, (sh.hidden, sh.hidden), 0.02)
    bw = block_weights(rng, sh, norm_std=norm_std, rms=rms, sandwich=sandwich, w8a8=w8a8)
    return dict(shape=sh, x=x, t=np.float32(t), w_t1=w_t1, w_t2=w_t2, block=bw)


def model_case(name: str = "dit32", blocks=None, seed=None, hidden=None, heads=None,
               ffn=None, L=None, h=None, w=None, text_dim=None, w8a8=False):
    """Inputs of a whole DiT: latent x_lat [N, 64] ~ N(0,1), text features
    ctx [L, text_dim] ~ N(0,1), and all weights (time MLP, in/out linears,
    final modulation, `blocks` blocks).  Overrides make reduced-size twins."""
    sh = SHAPES[name]
    def pick(v, d):
        return d if v is None else v
    kw = dict(hidden=pick(hidden, sh.hidden), heads=pick(heads, sh.heads), ffn=pick(ffn, sh.ffn),
              L=pick(L, sh.L), h=pick(h, sh.h), w=pick(w, sh.w), blocks=pick(blocks, sh.blocks),
              text_dim=pick(text_dim, sh.text_dim))
    sh = Shape(sh.name, kw["hidden"], kw["heads"], sh.head_dim, kw["ffn"], kw["L"], kw["h"],
               kw["w"], seed=sh.seed if seed is None else seed, blocks=kw["blocks"],
               latent=sh.latent, text_dim=kw["text_dim"], time_dim=sh.time_dim, axes=sh.axes)
    rng = np.random.default_rng(sh.seed)
    D = sh.hidden
    x_lat = rng.standard_normal((sh.N, sh.latent), dtype=np.float32)
    ctx = rng.standard_normal((sh.L, sh.text_dim), dtype=np.float32)
    top = dict(
        w_t1=_normal(rng, (D, sh.time_dim), 0.02),
        w_t2=_normal(rng, (D, D), 0.02),
        w_in=_normal(rng, (D, sh.latent), 0.02),
        w_txt=_normal(rng, (D, sh.text_dim), 0.02),
        w_fmod=_normal(rng, (2 * D, D), 0.02),
        w_final=_normal(rng, (sh.latent, D), 0.02),
    )
    blocks = [block_weights(rng, sh, int8=False, w8a8=w8a8) for _ in range(sh.blocks)]
    return dict(shape=sh, x_lat=x_lat, ctx=ctx, top=top, blocks=blocks)


def normal(shape, seed: int, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """float32 draws N(mean, std^2) from a generator seeded with `seed`."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std) + np.float32(mean)).astype(np.float32)


def rows_sample(S: int, count: int, L: int = 0, seed: int = 123, tile: int = 256) -> np.ndarray:
    """Sorted distinct row indexes for sampled checks: the first and last
    text and image rows, one random row inside every `tile` consecutive rows
    (so no block of rows goes unchecked), plus `count` random ones."""
    rng = np.random.default_rng(seed)
    pick = {0, S - 1}
    if L > 0:
        pick.update({L - 1, L})
    for t0 in range(0, S, tile):
        pick.add(int(rng.integers(t0, min(S, t0 + tile))))
    pick.update(rng.choice(S, size=min(count, S), replace=False).tolist())
    return np.array(sorted(pick), dtype=np.int64)
