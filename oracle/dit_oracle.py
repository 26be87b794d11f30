"""Plain CPU oracle of the AdaLN diffusion-transformer hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the CPU-baseline leg of the benchmark may import or run this module.  The GPU
library never calls it and shares no code with it: no kernels, no tables, no
constant generators, no pre- or post-processing.

Every function is the plain definition of one step, written in NumPy float64
unless a page fixes another precision (the rotary tables and the Euler update
are float32 there).  Inputs are whatever values the caller passes (normally
bf16-representable numbers drawn by the seeded generators).  The one place
the oracle rounds to bf16 is where a page puts a rounding into the method
itself: an int8 block-32 weight is the exact product code * scale, handed to
the bf16 products as that product rounded to the nearest bf16
(`dequant_int8_b32_bf16`); everything else is the exact-as-possible result
the GPU path approximates.

Sources (web pages; cited by title and section):
  [HC]  "Host contract -- RGBA-Image-2.1-Turbo (Core AI port of
        Qwen-Image-2.1-Turbo)": s.1 The graphs, s.4 Sequence layout and RoPE,
        s.5 Noise and pack, s.6 Sampler.
  [K4]  "944 -> 346 ms: optimizing FLUX.2 klein-4B on one TPU v6e chip":
        s.2 The two inference paths (cast points), s.4.3 Pallas flash
        attention, s.4.4 Fused qk-prep kernel, Appendix B (D3 rope relayout,
        D3c qk-prep and the double block's per-stream prep, D4 the double
        blocks' per-stream weight names).
  [GZ]  "gizai:dit" module reference: types Block, Sequence, Modulation;
        functions sinusoids, gluRows, gatedInto, normedInto, prepOf, silu,
        Block.forward, Block.parallel; constants HEAD, QKV/OUT/UP/DOWN,
        POST_ATTN/POST_MLP (sandwich norms).

`quantize_rows_int8` is pinned by a worked example (ties to even, the
largest magnitude to 127, zero rows), the half-step error bound, and
`linear_w8a8` by brute-force integer sums and the error bound of the
activations' rounding.

Readings of points the pages leave open are listed in the repository's
design notes; the ones that shape the arithmetic are restated where used.

Parity status: every function below is pinned by the CPU test-suite
(closed forms, printed examples, invariants, brute force on tiny inputs)
except `block_forward`/`denoise` as a whole, whose composition is pinned
only through its parts, a pure-Python brute-force twin on tiny shapes and
structural invariants (identity when all gates are zero, permutation
equivariance of rows); no page prints a block output.
`parallel_block_forward` is pinned to the sequential block: its update is
the sum of the sequential block's attention-only and MLP-only updates (gate
of the other half zero) under the same shift, scale and gate.
`block_forward_runs` is pinned to it: one run, or equal vectors in every
run, is the block; a run with zero gates keeps its rows.
`post_norm` (a sandwich block's norms) is pinned by closed forms: with
eps 0 each row of a half's update divided by its gate and norm weight has
RMS 1 (RMSNorm) or mean 0 and variance 1 (LayerNorm), and the block is
unchanged when the product's weight is scaled.
`block_forward_cached` is pinned to it: with the cache recorded from the
same rows its updated rows are the block's, the read-only rows stay, and
the read-only rows' own values no longer matter once cached.
`double_block_forward` is pinned to it as well: with the same weights in
both streams it is the sequential block, and with no text rows it is the
sequential block of the image weights.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F64 = np.float64
F32 = np.float32


# ---------------------------------------------------------------------------
# Architecture description
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Arch:
    """Shape of one AdaLN block ([GZ] type Arch: hidden, heads, head, ffn,
    eps, qkEps, finalEps).  `axes` are the rotary axis widths (values per
    axis; [HC] s.4 uses 16, 56, 56 for a 128-wide head).  `norm` is
    "layer" (LayerNorm without affine) or "rms" (RMSNorm times weight)."""

    hidden: int
    heads: int
    head_dim: int
    ffn: int
    axes: tuple = (16, 56, 56)
    eps: float = 1e-6
    qk_eps: float = 1e-6
    final_eps: float = 1e-6
    rope_theta: float = 10000.0
    norm: str = "layer"
    time_dim: int = 256      # sinusoid width ([GZ] sinusoids `dim`)
    latent: int = 64         # latent channels per image token ([HC] s.1)

    def __post_init__(self):
        assert self.hidden == self.heads * self.head_dim
        assert sum(self.axes) == self.head_dim
        assert all(a % 2 == 0 for a in self.axes)


# ---------------------------------------------------------------------------
# [HC] s.4 -- positions and rotary tables
# ---------------------------------------------------------------------------

def positions(L: int, h: int, w: int) -> np.ndarray:
    """3-axis (frame, height, width) positions of the packed [text L | image N]
    sequence, [HC] s.4: text token i -> (i, i, i); image token at row y,
    column x (index y*w + x) -> (L, y - (h - h//2), x - (w - w//2)).
    Returns int64 [L + h*w, 3]."""
    pos = np.zeros((L + h * w, 3), dtype=np.int64)
    for i in range(L):
        pos[i] = (i, i, i)
    for y in range(h):
        for x in range(w):
            pos[L + y * w + x] = (L, y - (h - h // 2), x - (w - w // 2))
    return pos


def rope_inverse_frequencies(d: int, theta: float = 10000.0) -> np.ndarray:
    """Inverse frequencies of one rotary axis of width d, [HC] s.4:
    1 / theta^(j/d) for j = 0, 2, 4, ..., d-2 (d/2 of them), float64."""
    j = np.arange(0, d, 2, dtype=F64)
    return 1.0 / np.power(F64(theta), j / F64(d))


def rope_tables(pos: np.ndarray, axes=(16, 56, 56), theta: float = 10000.0):
    """Per-token rotary cos/sin, [HC] s.4: for each axis a, the angles
    pos[:, a] * inv_a (outer product), and a token's row is the three axes'
    rows concatenated in axis order (8 + 28 + 28 = 64 values for a 128 head).
    The pages' tables are fp32; here the angle and its cos/sin are taken in
    float64 and rounded once to fp32.  Returns (cos, sin) float32 [S, sum/2]."""
    cols_c, cols_s = [], []
    for a, d in enumerate(axes):
        ang = np.outer(pos[:, a].astype(F64), rope_inverse_frequencies(d, theta))
        cols_c.append(np.cos(ang))
        cols_s.append(np.sin(ang))
    return (np.concatenate(cols_c, axis=1).astype(F32),
            np.concatenate(cols_s, axis=1).astype(F32))


def rope_apply(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (v[..., 2p], v[..., 2p+1]) by the angle whose
    cos/sin are cos[..., p], sin[..., p]: (a, b) -> (a cos - b sin,
    a sin + b cos).  This is the complex product with torch.polar's unit
    phasors ([HC] s.4), which [K4] Appendix B (D3) writes as
    cos2*x + sin2*pair_swap(x).  v [..., S, 2P]; cos, sin [S, P]."""
    a = v[..., 0::2]
    b = v[..., 1::2]
    c = cos.astype(F64)
    s = sin.astype(F64)
    out = np.empty(v.shape, dtype=F64)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# ---------------------------------------------------------------------------
# [GZ] sinusoids, silu; time MLP and modulation
# ---------------------------------------------------------------------------

def silu(x: np.ndarray) -> np.ndarray:
    """silu(x) = x * sigmoid(x) ([GZ] silu)."""
    x = np.asarray(x, dtype=F64)
    return x / (1.0 + np.exp(-x))


def sinusoids(times, dim: int = 256) -> np.ndarray:
    """[GZ] sinusoids: rows [cos | sin] of each time times the dim/2
    frequencies 10000^(-i/(dim/2)), i = 0 .. dim/2-1.  float64 [T, dim]."""
    times = np.atleast_1d(np.asarray(times, dtype=F64))
    half = dim // 2
    freqs = np.power(F64(10000.0), -np.arange(half, dtype=F64) / F64(half))
    ang = np.outer(times, freqs)
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def timestep_embedding(t: float, dim: int = 256) -> np.ndarray:
    """The DiT's time input t is timesteps/1000 ([HC] s.6); the embedding is
    taken of 1000*t ([K4] s.2 lists the 1000*t scaling among its cast points;
    here it is kept in float64).  Returns [dim]."""
    return sinusoids([1000.0 * float(t)], dim)[0]


def linear(x: np.ndarray, w) -> np.ndarray:
    """x W^T with W stored [out, in] ([GZ] Block: linears [out, in]).  An
    Int8Rows weight takes x's rows through INT8 too (linear_w8a8)."""
    if isinstance(w, Int8Rows):
        return linear_w8a8(x, w)
    return np.asarray(x, dtype=F64) @ np.asarray(w, dtype=F64).T


# ---------------------------------------------------------------------------
# W8A8 linears ([GZ] linear and quantizedOf: a linear with INT8 weights takes
# x's rows as INT8 with one scale a row, and the product is the integer dot
# product times x's scale and W's; [K4] Appendix B, D4: symmetric weights
# with one absmax/127 scale per output row, activations quantized per token
# at each call, int8 x int8 -> int32, then an fp32 dequantisation)
# ---------------------------------------------------------------------------

@dataclass
class Int8Rows:
    """A linear's weights as INT8 rows q [out, in] and one float32 scale per
    row s [out]: W = q * s[:, None].  rotated: the rows are stored in
    ConvRot's basis ([GZ] Block.quantized, Block.dequantized, comfyInt8Rows:
    rotated by the regular Hadamard of 256), so the product's input rows are
    rotated the same way before they are quantized (convrot), and the weights
    of the unrotated input are (q * s) R per group of 256 inputs."""

    q: np.ndarray
    s: np.ndarray
    rotated: bool = False


def hadamard(n: int = 256) -> np.ndarray:
    """The regular Hadamard matrix of order n (a power of two) in its own
    (Sylvester) order, H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]], scaled by
    1/sqrt(n) so that it is orthogonal.  float64 [n, n]."""
    assert n >= 1 and n & (n - 1) == 0
    h = np.ones((1, 1), dtype=F64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h / math.sqrt(n)


def convrot(x, group: int = 256) -> np.ndarray:
    """ConvRot's rotation of the product's input rows ([GZ] linearInto,
    Block.dequantized: each 256 inputs x are taken to y = R x with R the
    regular Hadamard of 256): every consecutive group of 256 values of the
    last axis times R (symmetric, so the row form y = x R^T is x R), in
    float64.  The last axis must be a multiple of 256."""
    x = np.asarray(x, dtype=F64)
    k = x.shape[-1]
    assert k % group == 0
    r = hadamard(group)
    return (x.reshape(x.shape[:-1] + (k // group, group)) @ r.T).reshape(x.shape)


def quantize_rows_int8(x):
    """Symmetric INT8 codes of each row of x over one scale a row:
    s = max|x| / 127 and q = x / s rounded to nearest, ties to even, so
    |q| <= 127 and the largest magnitude maps to +-127; an all-zero row has
    s = 0 and q = 0.  Where floating point decides an integer both sides
    decide in one precision; the pages fix none, so it is the kernels'
    float32: x is taken to float32, inv = 127 / amax and q = rint(x * inv),
    s = amax / 127, each a correctly rounded float32 operation.  Returns
    (q int8 [..., K], s float32 [...])."""
    x = np.asarray(x, dtype=F32)
    amax = np.abs(x).max(axis=-1)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, F32(127) / amax, F32(0)).astype(F32)
    q = np.clip(np.rint(x * inv[..., None]), -127, 127).astype(np.int8)
    return q, (amax / F32(127)).astype(F32)


class _RowSlicer:
    """Row ranges of a weight, float or Int8Rows (its scales go along)."""

    def __init__(self, w):
        self.w = w

    def __getitem__(self, sl):
        if isinstance(self.w, Int8Rows):
            return Int8Rows(q=np.asarray(self.w.q)[sl], s=np.asarray(self.w.s)[sl], rotated=self.w.rotated)
        return np.asarray(self.w, F64)[sl]


def linear_w8a8(x, w: Int8Rows) -> np.ndarray:
    """x W^T with x's rows quantized by quantize_rows_int8 (after ConvRot's
    rotation when the weights are rotated: the rotated rows are rounded once
    to float32, the precision the quantization decides in): the exact
    integer dot products times x's row scale and W's row scale, in float64.
    The integer sums are taken by a float64 matrix product: every product
    of two codes and every partial sum is an integer of magnitude below
    K * 127^2 < 2^53, so each float64 addition is exact in any order."""
    if w.rotated:
        x = convrot(x).astype(F32)
    q, s = quantize_rows_int8(x)
    wq = np.asarray(w.q)
    assert q.shape[-1] * 127 * 127 < 2 ** 53
    acc = q.astype(F64) @ wq.astype(F64).T
    return acc * np.asarray(s, F64)[..., None] * np.asarray(w.s, F64)[None, :]


def time_vector(t: float, w_t1: np.ndarray, w_t2: np.ndarray, dim: int = 256):
    """Conditioning vector vec = W_t2 silu(W_t1 temb(t)), no biases.  The
    time MLP's two linears are the Arch fields timeHidden/timeDim of [GZ];
    the modulations depend on t through vec ([K4] Appendix B, D2)."""
    temb = timestep_embedding(t, dim)
    return linear(silu(linear(temb[None, :], w_t1)), w_t2)[0]


def modulation(vec: np.ndarray, w_mod: np.ndarray, chunks: int = 6):
    """mod = W_mod silu(vec), split into `chunks` rows of `hidden`
    ([GZ] Modulation: shift, scale, gate of the attention, then of the MLP).
    Returns float64 [chunks, hidden]."""
    m = linear(silu(vec)[None, :], w_mod)[0]
    return m.reshape(chunks, -1)


# ---------------------------------------------------------------------------
# Norms ([GZ] normedInto, Block.parallel "modulated LayerNorm")
# ---------------------------------------------------------------------------

def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) per row, biased variance, no affine."""
    x = np.asarray(x, dtype=F64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def rms_norm(x: np.ndarray, w, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w per row."""
    x = np.asarray(x, dtype=F64)
    r = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return r if w is None else r * np.asarray(w, dtype=F64)


def modulated_norm(x, shift, scale, arch: Arch, norm_w=None, eps=None):
    """norm(x) * (1 + scale) + shift, the AdaLN modulated norm a block's
    linears take ([GZ] normedInto)."""
    eps = arch.eps if eps is None else eps
    if arch.norm == "layer":
        n = layer_norm(x, eps)
    elif arch.norm == "rms":
        n = rms_norm(x, norm_w, eps)
    else:
        raise ValueError(arch.norm)
    return n * (1.0 + np.asarray(scale, F64)) + np.asarray(shift, F64)


# ---------------------------------------------------------------------------
# Attention ([K4] s.4.3; [GZ] Sequence: full attention over all rows)
# ---------------------------------------------------------------------------

def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax with the row max subtracted first."""
    s = np.asarray(s, dtype=F64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention(q, k, v, scale=None):
    """o = softmax(q k^T * scale) v per head, no mask: every row attends to
    every row ([K4] s.4.3: DiT attention is full; 1/sqrt(d) applied to the
    scores).  q, k, v [H, S, d] -> o [H, S, d]."""
    q = np.asarray(q, F64)
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=F64)
    for h in range(q.shape[0]):
        p = softmax_rows((q[h] @ k[h].T) * scale)
        out[h] = p @ v[h]
    return out


def swiglu_interleaved(u: np.ndarray) -> np.ndarray:
    """UP's output columns hold gate j at 2j and up j at 2j+1 ([GZ] gluRows);
    SwiGLU is silu(gate) * up ([GZ] Block)."""
    u = np.asarray(u, F64)
    return silu(u[..., 0::2]) * u[..., 1::2]


def heads_of(cols: np.ndarray, heads: int, head_dim: int) -> np.ndarray:
    """[S, heads*head_dim] -> [heads, S, head_dim]; head j = columns
    j*head_dim .. (j+1)*head_dim."""
    S = cols.shape[0]
    return cols.reshape(S, heads, head_dim).transpose(1, 0, 2)


def head_prep(qk: np.ndarray, w, eps: float, cos, sin) -> np.ndarray:
    """[GZ] prepOf: each head over its RMS times the head-norm weight, then
    the rotary turn with the sequence's cos/sin rows ([K4] s.4.4 keeps the
    same order: QK-RMSNorm, then rope).  qk [H, S, d]."""
    n = rms_norm(qk, w, eps)
    return rope_apply(n, cos, sin)


# ---------------------------------------------------------------------------
# [GZ] Block.forward
# ---------------------------------------------------------------------------

@dataclass
class BlockWeights:
    """One block's weights as float values (bf16 values in practice).
    w_qkv [3*H*d, D] (all queries, all keys, all values; [GZ] weightAt),
    w_out [D, H*d], w_up [2F, D] (gate/up interleaved, [GZ] gluRows),
    w_down [D, F], w_mod [6D, D]; q_norm, k_norm [d]; norm1, norm2 [D]
    (RMS variant only); post_attn, post_mlp [D]: a sandwich block's norm
    weights after the attention and after the MLP ([GZ] POST_ATTN,
    POST_MLP), None for a block without them."""

    w_qkv: np.ndarray
    w_out: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    w_mod: np.ndarray
    q_norm: np.ndarray
    k_norm: np.ndarray
    norm1: np.ndarray = None
    norm2: np.ndarray = None
    post_attn: np.ndarray = None
    post_mlp: np.ndarray = None


def post_norm(y, w, arch: Arch):
    """A sandwich block's norm of a product's output rows, taken before the
    gate ([GZ] POST_ATTN, POST_MLP: a sandwich block norms its attention and
    MLP outputs before their gates; a block without the weights adds the
    gated outputs as they are).  The norm is the block's own kind (the
    arch's LayerNorm or RMSNorm, its eps) times the weight w; w None leaves
    y as it is."""
    if w is None:
        return y
    if arch.norm == "rms":
        return rms_norm(y, w, arch.eps)
    if arch.norm == "layer":
        return layer_norm(y, arch.eps) * np.asarray(w, F64)
    raise ValueError(arch.norm)


def _no_sandwich(bw: BlockWeights, form: str):
    if bw.post_attn is not None or bw.post_mlp is not None:
        raise ValueError(f"sandwich norms belong to the sequential block, not the {form}")


def block_forward(x, bw: BlockWeights, vec, cos, sin, arch: Arch,
                  keep: bool = False):
    """One AdaLN block over x [S, D] ([GZ] Block.forward): x + gate_a *
    attention(modulated norm of x), then the same with the SwiGLU MLP.
    Returns the new rows (float64) and, with keep=True, a dict of the
    intermediates (mod, h, q, k, v after prep, o, x1, h2, a)."""
    x = np.asarray(x, F64)
    S, D = x.shape
    H, d = arch.heads, arch.head_dim
    m = modulation(vec, bw.w_mod, 6)
    shift_a, scale_a, gate_a, shift_m, scale_m, gate_m = m
    # attention half
    h = modulated_norm(x, shift_a, scale_a, arch, bw.norm1)
    qkv = linear(h, bw.w_qkv)
    q = heads_of(qkv[:, 0:H * d], H, d)
    k = heads_of(qkv[:, H * d:2 * H * d], H, d)
    v = heads_of(qkv[:, 2 * H * d:3 * H * d], H, d)
    q = head_prep(q, bw.q_norm, arch.qk_eps, cos, sin)
    k = head_prep(k, bw.k_norm, arch.qk_eps, cos, sin)
    o = attention(q, k, v).transpose(1, 0, 2).reshape(S, H * d)
    x1 = x + gate_a * post_norm(linear(o, bw.w_out), bw.post_attn, arch)   # [GZ] gatedInto
    # MLP half
    h2 = modulated_norm(x1, shift_m, scale_m, arch, bw.norm2)
    a = swiglu_interleaved(linear(h2, bw.w_up))
    y = x1 + gate_m * post_norm(linear(a, bw.w_down), bw.post_mlp, arch)
    if not keep:
        return y
    return y, dict(mod=m, h=h, q=q, k=k, v=v, o=o, x1=x1, h2=h2, a=a)


def block_forward_rows(x, bw: BlockWeights, vec, cos, sin, arch: Arch, rows):
    """Block output for the selected rows only (same arithmetic as
    block_forward): keys and values need every row, everything after the
    attention is per row.  Used to check sampled rows at sizes where the
    full oracle is too slow.  Returns (y[rows], o[rows], x1[rows], a[rows])."""
    x = np.asarray(x, F64)
    rows = np.asarray(rows)
    H, d = arch.heads, arch.head_dim
    m = modulation(vec, bw.w_mod, 6)
    shift_a, scale_a, gate_a, shift_m, scale_m, gate_m = m
    h = modulated_norm(x, shift_a, scale_a, arch, bw.norm1)
    wq = _RowSlicer(bw.w_qkv)
    q = heads_of(linear(h[rows], wq[0:H * d]), H, d)
    k = heads_of(linear(h, wq[H * d:2 * H * d]), H, d)
    v = heads_of(linear(h, wq[2 * H * d:]), H, d)
    q = head_prep(q, bw.q_norm, arch.qk_eps, cos[rows], sin[rows])
    k = head_prep(k, bw.k_norm, arch.qk_eps, cos, sin)
    o = attention(q, k, v).transpose(1, 0, 2).reshape(len(rows), H * d)
    x1 = x[rows] + gate_a * post_norm(linear(o, bw.w_out), bw.post_attn, arch)
    h2 = modulated_norm(x1, shift_m, scale_m, arch, bw.norm2)
    a = swiglu_interleaved(linear(h2, bw.w_up))
    y = x1 + gate_m * post_norm(linear(a, bw.w_down), bw.post_mlp, arch)
    return y, o, x1, a


def _modulation_per_row(vecs, w_mod, runs, S: int):
    """Per-row shift/scale/gate vectors [6, S, D] for (first, end, row) runs
    that tile rows [0, S) in order ([GZ] Sequence runs)."""
    mods = [modulation(v, w_mod, 6) for v in np.asarray(vecs, F64)]
    per_row = np.empty((6, S, mods[0].shape[1]))
    end = 0
    for r0, r1, m in runs:                  # contiguous, in order, covering [0, S)
        if r0 != end or r1 <= r0:
            raise ValueError(f"runs must tile the rows in order: {runs}")
        per_row[:, r0:r1] = mods[m][:, None, :]
        end = r1
    if end != S:
        raise ValueError(f"runs end at {end}, not {S}")
    return mods, per_row


def block_forward_runs(x, bw: BlockWeights, vecs, runs, cos, sin, arch: Arch,
                       keep: bool = False):
    """The block with several modulation rows ([GZ] Sequence: map gives each
    row its modulation row; Modulation holds [modulation rows, hidden]
    shift/scale/gate; runsOf/gatedInto: (first, end, row) runs of rows that
    share one).  vecs [R, D] are the conditioning vectors of the R
    modulation rows; runs lists (first, end, row) covering rows [0, S) in
    order.  Every row takes the norm shifts/scales and gates of its run's
    modulation row; the products and the joint attention are unchanged."""
    x = np.asarray(x, F64)
    S, D = x.shape
    H, d = arch.heads, arch.head_dim
    mods, per_row = _modulation_per_row(vecs, bw.w_mod, runs, S)
    shift_a, scale_a, gate_a, shift_m, scale_m, gate_m = per_row
    h = modulated_norm(x, shift_a, scale_a, arch, bw.norm1)
    qkv = linear(h, bw.w_qkv)
    q = head_prep(heads_of(qkv[:, 0:H * d], H, d), bw.q_norm, arch.qk_eps, cos, sin)
    k = head_prep(heads_of(qkv[:, H * d:2 * H * d], H, d), bw.k_norm, arch.qk_eps, cos, sin)
    v = heads_of(qkv[:, 2 * H * d:3 * H * d], H, d)
    o = attention(q, k, v).transpose(1, 0, 2).reshape(S, H * d)
    x1 = x + gate_a * post_norm(linear(o, bw.w_out), bw.post_attn, arch)
    h2 = modulated_norm(x1, shift_m, scale_m, arch, bw.norm2)
    a = swiglu_interleaved(linear(h2, bw.w_up))
    y = x1 + gate_m * post_norm(linear(a, bw.w_down), bw.post_mlp, arch)
    if not keep:
        return y
    return y, dict(mods=np.array(mods), h=h, q=q, k=k, v=v, o=o, x1=x1, h2=h2, a=a)


def block_forward_runs_rows(x, bw: BlockWeights, vecs, runs, cos, sin, arch: Arch, rows):
    """block_forward_runs for the selected rows only (keys and values need
    every row, everything after the attention is per row).  Returns
    (y[rows], o[rows], a[rows])."""
    x = np.asarray(x, F64)
    S = x.shape[0]
    rows = np.asarray(rows)
    H, d = arch.heads, arch.head_dim
    _, per_row = _modulation_per_row(vecs, bw.w_mod, runs, S)
    shift_a, scale_a, gate_a, shift_m, scale_m, gate_m = per_row
    h = modulated_norm(x, shift_a, scale_a, arch, bw.norm1)
    wq = _RowSlicer(bw.w_qkv)
    q = heads_of(linear(h[rows], wq[0:H * d]), H, d)
    k = heads_of(linear(h, wq[H * d:2 * H * d]), H, d)
    v = heads_of(linear(h, wq[2 * H * d:]), H, d)
    q = head_prep(q, bw.q_norm, arch.qk_eps, cos[rows], sin[rows])
    k = head_prep(k, bw.k_norm, arch.qk_eps, cos, sin)
    o = attention(q, k, v).transpose(1, 0, 2).reshape(len(rows), H * d)
    x1 = x[rows] + gate_a[rows] * post_norm(linear(o, bw.w_out), bw.post_attn, arch)
    h2 = modulated_norm(x1, shift_m[rows], scale_m[rows], arch, bw.norm2)
    a = swiglu_interleaved(linear(h2, bw.w_up))
    y = x1 + gate_m[rows] * post_norm(linear(a, bw.w_down), bw.post_mlp, arch)
    return y, o, a


def reference_kv(x, bw: BlockWeights, vec, cos, sin, arch: Arch, first: int):
    """The keys and values (after the head norm and rotary) of rows
    [first, S) as the block computes them over x ([GZ] RefSlot: a recording
    step keeps the reference rows' keys and values).  Returns (k, v), each
    [H, S - first, d]."""
    _, ref = block_forward(x, bw, vec, cos, sin, arch, keep=True)
    return ref["k"][:, first:], ref["v"][:, first:]


def block_forward_cached(x, bw: BlockWeights, vec, cos, sin, arch: Arch, first: int, k_ref, v_ref):
    """The block over the first rows only ([GZ] Sequence.active: rows
    [0, first) are updated, rows [first, S) are read only, with the same
    positions and modulation; RefSlot: the read-only rows' keys and values
    come from a recording step, k_ref and v_ref [H, S - first, d]).  The
    queries are rows [0, first); the keys and values are the first rows'
    own followed by the cached ones.  Rows [first, S) are returned as they
    are."""
    x = np.asarray(x, F64)
    S, D = x.shape
    H, d = arch.heads, arch.head_dim
    shift_a, scale_a, gate_a, shift_m, scale_m, gate_m = modulation(vec, bw.w_mod, 6)
    xa = x[:first]
    h = modulated_norm(xa, shift_a, scale_a, arch, bw.norm1)
    qkv = linear(h, bw.w_qkv)
    q = head_prep(heads_of(qkv[:, 0:H * d], H, d), bw.q_norm, arch.qk_eps, cos[:first], sin[:first])
    k = head_prep(heads_of(qkv[:, H * d:2 * H * d], H, d), bw.k_norm, arch.qk_eps, cos[:first], sin[:first])
    v = heads_of(qkv[:, 2 * H * d:3 * H * d], H, d)
    k = np.concatenate([k, np.asarray(k_ref, F64)], axis=1)
    v = np.concatenate([v, np.asarray(v_ref, F64)], axis=1)
    o = attention(q, k, v).transpose(1, 0, 2).reshape(first, H * d)
    x1 = xa + gate_a * post_norm(linear(o, bw.w_out), bw.post_attn, arch)
    h2 = modulated_norm(x1, shift_m, scale_m, arch, bw.norm2)
    a = swiglu_interleaved(linear(h2, bw.w_up))
    y = x.copy()
    y[:first] = x1 + gate_m * post_norm(linear(a, bw.w_down), bw.post_mlp, arch)
    return y


def parallel_block_forward(x, bw: BlockWeights, vec, cos, sin, arch: Arch,
                           keep: bool = False):
    """The parallel block ([GZ] Block.parallel): one modulated norm feeds
    both the attention and the SwiGLU MLP, and one gate scales their sum:
    x + gate * (attention(h) W_out^T + swiglu(h W_up^T) W_down^T) with
    h = norm(x) (1 + scale) + shift.  The modulation has three rows
    (shift, scale, gate; w_mod [3D, D]); UP's rows are gate/up interleaved
    as in the sequential block.  Returns the new rows (float64) and, with
    keep=True, the intermediates (mod, h, q, k, v after prep, o, a)."""
    x = np.asarray(x, F64)
    _no_sandwich(bw, "parallel block")
    S, D = x.shape
    H, d = arch.heads, arch.head_dim
    m = modulation(vec, bw.w_mod, 3)
    shift, scale, gate = m
    h = modulated_norm(x, shift, scale, arch, bw.norm1)
    qkv = linear(h, bw.w_qkv)
    q = head_prep(heads_of(qkv[:, 0:H * d], H, d), bw.q_norm, arch.qk_eps, cos, sin)
    k = head_prep(heads_of(qkv[:, H * d:2 * H * d], H, d), bw.k_norm, arch.qk_eps, cos, sin)
    v = heads_of(qkv[:, 2 * H * d:3 * H * d], H, d)
    o = attention(q, k, v).transpose(1, 0, 2).reshape(S, H * d)
    a = swiglu_interleaved(linear(h, bw.w_up))
    y = x + gate * (linear(o, bw.w_out) + linear(a, bw.w_down))
    if not keep:
        return y
    return y, dict(mod=m, h=h, q=q, k=k, v=v, o=o, a=a)


def parallel_block_forward_rows(x, bw: BlockWeights, vec, cos, sin, arch: Arch, rows):
    """Parallel-block output for the selected rows only (same arithmetic as
    parallel_block_forward; keys and values need every row).  Returns
    (y[rows], o[rows], a[rows])."""
    x = np.asarray(x, F64)
    _no_sandwich(bw, "parallel block")
    rows = np.asarray(rows)
    H, d = arch.heads, arch.head_dim
    shift, scale, gate = modulation(vec, bw.w_mod, 3)
    h = modulated_norm(x, shift, scale, arch, bw.norm1)
    wq = _RowSlicer(bw.w_qkv)
    q = heads_of(linear(h[rows], wq[0:H * d]), H, d)
    k = heads_of(linear(h, wq[H * d:2 * H * d]), H, d)
    v = heads_of(linear(h, wq[2 * H * d:]), H, d)
    q = head_prep(q, bw.q_norm, arch.qk_eps, cos[rows], sin[rows])
    k = head_prep(k, bw.k_norm, arch.qk_eps, cos, sin)
    o = attention(q, k, v).transpose(1, 0, 2).reshape(len(rows), H * d)
    a = swiglu_interleaved(linear(h[rows], bw.w_up))
    y = x[rows] + gate * (linear(o, bw.w_out) + linear(a, bw.w_down))
    return y, o, a


def double_block_forward(x, bw_txt: BlockWeights, bw_img: BlockWeights, vec, cos, sin,
                         arch: Arch, L: int, keep: bool = False):
    """The double-stream block ([K4] Appendix B, D3c wiring and the D4 key
    names: text and image streams with their own attention and MLP weights,
    joint attention over both): rows [0, L) are the text stream, rows [L, S)
    the image stream.  Each stream takes its own six modulation rows, norms,
    QKV product and head prep (q/k norms, rotary with its rows of the joint
    table); the attention runs over all S rows, text rows first; each
    stream's output, norms and MLP use that stream's weights (each stream is
    the sequential block's arithmetic on its own rows, with the attention
    shared).  Returns the new rows (float64) and, with keep=True, the
    intermediates (h, q, k, v after prep, o, x1, a) over all rows."""
    x = np.asarray(x, F64)
    _no_sandwich(bw_txt, "double-stream block")
    _no_sandwich(bw_img, "double-stream block")
    S, D = x.shape
    H, d = arch.heads, arch.head_dim
    streams = ((bw_txt, slice(0, L)), (bw_img, slice(L, S)))
    mods, hs, qs, ks, vs = [], [], [], [], []
    for bw, r in streams:
        m = modulation(vec, bw.w_mod, 6)
        mods.append(m)
        h = modulated_norm(x[r], m[0], m[1], arch, bw.norm1)
        qkv = linear(h, bw.w_qkv)
        qs.append(head_prep(heads_of(qkv[:, 0:H * d], H, d), bw.q_norm, arch.qk_eps, cos[r], sin[r]))
        ks.append(head_prep(heads_of(qkv[:, H * d:2 * H * d], H, d), bw.k_norm, arch.qk_eps, cos[r], sin[r]))
        vs.append(heads_of(qkv[:, 2 * H * d:3 * H * d], H, d))
        hs.append(h)
    q = np.concatenate(qs, axis=1)
    k = np.concatenate(ks, axis=1)
    v = np.concatenate(vs, axis=1)
    o = attention(q, k, v).transpose(1, 0, 2).reshape(S, H * d)
    y = np.empty_like(x)
    x1s, as_ = [], []
    for (bw, r), m in zip(streams, mods):
        shift_a, scale_a, gate_a, shift_m, scale_m, gate_m = m
        x1 = x[r] + gate_a * linear(o[r], bw.w_out)
        h2 = modulated_norm(x1, shift_m, scale_m, arch, bw.norm2)
        a = swiglu_interleaved(linear(h2, bw.w_up))
        y[r] = x1 + gate_m * linear(a, bw.w_down)
        x1s.append(x1)
        as_.append(a)
    if not keep:
        return y
    return y, dict(h=np.concatenate(hs), q=q, k=k, v=v, o=o, x1=np.concatenate(x1s),
                   a=np.concatenate(as_))


# ---------------------------------------------------------------------------
# [HC] s.1 int8lin weights: one bf16 scale per block of 32
# ---------------------------------------------------------------------------

def bf16_rne(x) -> np.ndarray:
    """The bf16 value nearest to each float32 value of x, ties to the even
    significand (round to nearest even).  Written as the choice between the
    two bf16 neighbours of x -- its float32 bit pattern with the low 16 bits
    cleared, and the next bf16 away from zero -- whichever is nearer, the
    one with an even last significand bit on a tie.  Finite inputs.
    Returns float32."""
    x = np.asarray(x, F32)
    u = x.view(np.uint32)
    lo_bits = u & np.uint32(0xFFFF0000)
    hi_bits = lo_bits + np.uint32(0x10000)
    lo = lo_bits.view(F32).astype(F64)
    hi = hi_bits.view(F32).astype(F64)
    xv = x.astype(F64)
    d_lo, d_hi = np.abs(xv - lo), np.abs(hi - xv)
    lo_even = ((lo_bits >> np.uint32(16)) & np.uint32(1)) == 0
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & lo_even)
    return np.where(take_lo, lo, hi).astype(F32)


def dequant_int8_b32(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W[o, k] = q[o, k] * s[o, k // 32] ([HC] s.1: symmetric int8, one scale
    per block of 32 along the input axis).  With |q| <= 127 (7 bits) and a
    bf16 scale (8 significant bits) the product has at most 15 significant
    bits, so it is exact in float32.  q int8 [out, in]; s float [out, in/32].
    Returns float32 [out, in]."""
    q = np.asarray(q)
    s = np.asarray(s, F32)
    out, inn = q.shape
    assert inn % 32 == 0 and s.shape == (out, inn // 32)
    return q.astype(F32) * np.repeat(s, 32, axis=1)


def dequant_int8_b32_bf16(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The int8 block-32 weight as the bf16 products take it: the exact
    product q * s rounded to the nearest bf16, ties to even.  [HC] s.1 has
    the int8 weights dequantised inside the graph and the products computed
    in bf16; the exact fp32 product needs up to 15 significant bits, so a
    bf16 operand is its rounding (the reading taken is round to nearest
    even).  Returns float32 [out, in] of bf16 values."""
    return bf16_rne(dequant_int8_b32(q, s))


# ---------------------------------------------------------------------------
# [HC] s.6 -- Euler update and sigma grid
# ---------------------------------------------------------------------------

def euler_step(x: np.ndarray, v: np.ndarray, sigma, sigma_next) -> np.ndarray:
    """x + (sigma_next - sigma) * v, all in fp32 as [HC] s.6 writes it
    (a fp32 difference, a fp32 product, a fp32 sum: three roundings)."""
    x = np.asarray(x, F32)
    v = np.asarray(v, F32)
    dt = F32(F32(sigma_next) - F32(sigma))
    return (x + (dt * v).astype(F32)).astype(F32)


def sigma_grid(steps: int) -> np.ndarray:
    """Sigmas from 1 to 0 in `steps` equal steps, `steps + 1` fp32 values (the
    terminal 0 appended as in [HC] s.6); the DiT time input is t = sigma."""
    return np.linspace(1.0, 0.0, steps + 1).astype(F32)


def sigma_schedule(sample_sigmas, shift: float = 1.0):
    """The sampler's grid ([HC] s.6, FlowMatch Euler with a fixed grid): the
    given sigmas in fp32, shifted as shift*s / (1 + (shift - 1)*s), the
    timesteps s*1000 and the DiT time input t = timesteps/1000, every step a
    float32 operation; the grid closed by a terminal 0.  Returns
    (sigmas [n + 1], t [n]), float32."""
    s = np.asarray(sample_sigmas, F32)
    sh = F32(shift)
    s = (sh * s) / (F32(1) + (sh - F32(1)) * s)
    t = (s * F32(1000)) / F32(1000)
    return np.append(s, F32(0)).astype(F32), t.astype(F32)


# ---------------------------------------------------------------------------
# The whole DiT ([HC] s.1 DiT graph: img_tokens, txt_feats, timestep -> vel)
# ---------------------------------------------------------------------------

@dataclass
class ModelWeights:
    """w_t1 [D, time_dim], w_t2 [D, D] (time MLP); w_in [D, latent] (image
    tokens in); w_txt [D, text_dim] (text features in); w_fmod [2D, D]
    (final shift, scale); w_final [latent, D]; blocks: list of BlockWeights."""

    w_t1: np.ndarray
    w_t2: np.ndarray
    w_in: np.ndarray
    w_txt: np.ndarray
    w_fmod: np.ndarray
    w_final: np.ndarray
    blocks: list = field(default_factory=list)


def text_rows(ctx_feats, mw: ModelWeights) -> np.ndarray:
    """Text rows of the sequence, txt = ctx W_txt^T: step-invariant, computed
    once per image ([K4] Appendix B, D2 hoists it out of the Euler loop)."""
    return linear(ctx_feats, mw.w_txt)


def velocity(x_lat, txt, mw: ModelWeights, cos, sin, t, arch: Arch):
    """One DiT evaluation: seq = [txt ; x_lat W_in^T]; every block in turn;
    final modulated norm of the image rows with (shift, scale) =
    W_fmod silu(vec); v = that times W_final^T.  Returns float64 [N, latent]."""
    L = txt.shape[0]
    vec = time_vector(t, mw.w_t1, mw.w_t2, arch.time_dim)
    seq = np.concatenate([np.asarray(txt, F64), linear(x_lat, mw.w_in)], axis=0)
    for bw in mw.blocks:
        seq = block_forward(seq, bw, vec, cos, sin, arch)
    shift_f, scale_f = modulation(vec, mw.w_fmod, 2)
    img = seq[L:]
    hf = layer_norm(img, arch.final_eps) * (1.0 + scale_f) + shift_f
    return linear(hf, mw.w_final)


def denoise(x_lat, ctx_feats, mw: ModelWeights, cos, sin, sigmas, arch: Arch,
            keep_velocities: bool = False):
    """The few-step Euler flow-matching loop ([HC] s.6): for each i, the
    DiT's time input t = (sigma_i * 1000) / 1000 (the timestep, divided again,
    in fp32), vel = DiT(x, t), x = x + (sigma_{i+1} - sigma_i) vel in fp32.
    The DiT's velocity is handed to the fp32 update as fp32 (its graph
    boundary is fp32, [HC] s.1)."""
    txt = text_rows(ctx_feats, mw)
    x = np.asarray(x_lat, F32)
    vels = []
    for i in range(len(sigmas) - 1):
        t = (F32(sigmas[i]) * F32(1000)) / F32(1000)
        vel = velocity(x, txt, mw, cos, sin, float(t), arch).astype(F32)
        vels.append(vel)
        x = euler_step(x, vel, sigmas[i], sigmas[i + 1])
    return (x, vels) if keep_velocities else x


# ---------------------------------------------------------------------------
# FLOP accounting (algorithmic: 2*M*N*K per product, 4*H*S^2*d attention)
# ---------------------------------------------------------------------------

def block_flops(S: int, arch: Arch, chunks: int = 6) -> int:
    """Algorithmic FLOPs of one block over S rows: 2mnk per product, 4 H S^2 d
    for the attention, the modulation GEMV (6 rows of modulation for the
    sequential block, 3 for the parallel one)."""
    D, F, H, d = arch.hidden, arch.ffn, arch.heads, arch.head_dim
    lin = 2 * S * D * (3 * H * d) + 2 * S * (H * d) * D + 2 * S * D * (2 * F) + 2 * S * F * D
    att = 4 * H * S * S * d
    gemv = 2 * (chunks * D) * D
    return lin + att + gemv
