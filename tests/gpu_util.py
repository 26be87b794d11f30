"""Helpers shared by the GPU parity tests: device setup, comparisons and the
oracle <-> device marshalling of one block's inputs."""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from diffusion_transformer_amd import lib as L   # noqa: E402  (raises if libdit.so is missing)
from diffusion_transformer_amd import synth      # noqa: E402
import oracle as O                               # noqa: E402

# The tolerance every floating-point result is held to against the oracle:
# relative L2 error <= 2e-2 and max abs error <= 5e-2.
REL = 2e-2
ABS = 5e-2


# Max-abs bound of a block's outputs at workloads whose values are large (the
# int8 block-32 weights, codes up to 127 times scales ~0.01, are ~30x larger
# than N(0, 0.02) and the block's outputs reach ~1e4, where a fixed 5e-2 is
# below the bf16 resolution).  The GPU and the oracle take the same operands
# (the int8 weights as their bf16 roundings); the GPU stores the block's
# intermediates in bf16 (h, q, k, v, the probabilities P, o, h2, a), each
# rounding at most 2^-9 of the value's magnitude, and a product passes a
# relative perturbation of its inputs to its outputs with gain about 1 (a
# sum of K terms with independent rounding errors grows as sqrt(K), like the
# sum itself).  The longest chain of such roundings into an output element
# is four (P, o in the attention half; h2, a in the MLP half), so an element
# may deviate by at most 4 * 2^-9 = 2^-7 of the output's scale, which the
# reference's largest magnitude bounds from above.
BLOCK_MAXREL = 2.0 ** -7


def block_abs(ref):
    """max-abs bound: ABS, or BLOCK_MAXREL of the reference's largest
    magnitude where that is larger."""
    return max(ABS, BLOCK_MAXREL * float(np.abs(ref).max()))


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def np_of(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def compare(name, got, ref, rel=REL, abs_=ABS, bf16_stored=False):
    """rel-L2 <= rel and max-abs <= abs_.  For an intermediate the GPU stores
    in bf16 (bf16_stored=True) the max-abs bound is at least one bf16 unit in
    the last place at the reference's largest magnitude (2^-7 relative): the
    storage rounding alone reaches half of that."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if bf16_stored and ref.size:
        abs_ = max(abs_, float(np.abs(ref).max()) * 2.0 ** -7)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = got - ref
    den = np.linalg.norm(ref)
    r = np.linalg.norm(err) / den if den > 0 else np.linalg.norm(err)
    m = np.abs(err).max() if err.size else 0.0
    mr = float(np.abs(ref).max()) if ref.size else 0.0
    say(f"{name}: rel_l2={r:.3e} max_abs={m:.3e} (|ref|max={mr:.3g}, max_abs/|ref|max={m / mr if mr else 0:.2e})")
    assert r <= rel, f"{name}: relative L2 {r:.3e} > {rel}"
    assert m <= abs_, f"{name}: max abs {m:.3e} > {abs_}"
    return r, m


def arch_pair(sh, norm="layer"):
    la = L.make_arch(hidden=sh.hidden, heads=sh.heads, head_dim=sh.head_dim, ffn=sh.ffn,
                     axes=sh.axes, norm=L.NORM_RMS if norm == "rms" else L.NORM_LAYER,
                     time_dim=sh.time_dim, latent=sh.latent, text_dim=sh.text_dim)
    oa = O.Arch(sh.hidden, sh.heads, sh.head_dim, sh.ffn, axes=sh.axes, norm=norm,
                time_dim=sh.time_dim, latent=sh.latent)
    return la, oa


def oracle_block(bw: dict, rotated: bool = False) -> "O.BlockWeights":
    """The oracle's view of synth.block_weights' dict: int8 block-32 weights
    become the bf16 operands the products take (the exact code * scale
    rounded to nearest even, oracle.dequant_int8_b32_bf16), so the parity of
    the block measures its arithmetic, as with bf16 weights."""
    def lin(n):
        if "q_" + n in bw:
            return O.dequant_int8_b32_bf16(bw["q_" + n], bw["s_" + n])
        if "q8_" + n in bw:
            return O.Int8Rows(q=bw["q8_" + n], s=bw["s8_" + n], rotated=rotated)
        return bw[n]
    return O.BlockWeights(w_qkv=lin("w_qkv"), w_out=lin("w_out"), w_up=lin("w_up"),
                          w_down=lin("w_down"), w_mod=bw["w_mod"], q_norm=bw["q_norm"],
                          k_norm=bw["k_norm"], norm1=bw.get("norm1"), norm2=bw.get("norm2"),
                          post_attn=bw.get("post_attn"), post_mlp=bw.get("post_mlp"))


class GpuSeq:
    """Positions, rotary tables and the time vector made by the library."""

    def __init__(self, ctx, sh, t, w_t1, w_t2):
        S = sh.S
        self.pos = torch.empty((S, 3), dtype=torch.int32, device="cuda")
        self.cos = torch.empty((S, sh.head_dim // 2), dtype=torch.float32, device="cuda")
        self.sin = torch.empty_like(self.cos)
        ctx.positions(sh.L, sh.h, sh.w, self.pos)
        ctx.rope_tables(self.pos, S, self.cos, self.sin)
        self.vec = torch.empty(sh.hidden, dtype=torch.float32, device="cuda")
        self.w_t1 = L.dev_bf16(w_t1)
        self.w_t2 = L.dev_bf16(w_t2)
        ctx.time_vector(self.w_t1, self.w_t2, float(t), self.vec)


def rel_l2(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)
