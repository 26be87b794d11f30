"""ctypes binding of libdit (include/dit.h).

Argument marshalling only: every entry point here checks that its torch
tensors have the dtype, device and layout the C ABI expects, passes their
device pointers and the current HIP stream, and raises DitError on a non-OK
status.  All compute runs in the library's HIP kernels.  There is no CPU
fallback: if libdit.so is missing, importing this module raises.
"""

from __future__ import annotations

import ctypes as C

import numpy as np
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdit.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "dit.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libdit.so not found at {LIB_PATH}; build it with "
                      "`python -m diffusion_transformer_amd.build` (needs hipcc)")
_lib = C.CDLL(LIB_PATH)

OK, EINVAL, ERANGE, ENOMEM, EDEVICE, EUNSUPPORTED = 0, -1, -2, -3, -4, -5
STAGES = ("mod", "norm1", "qkv", "attn", "out", "norm2", "up", "down", "time", "img_in", "final",
          "euler", "txt_in", "par_in", "par_out", "post", "quant", "qk_prep", "dequant")
W_BF16, W_INT8_B32, W_INT8_ROW, W_INT8_ROT = 0, 1, 2, 3
NORM_LAYER, NORM_RMS = 0, 1
_NAMES = {0: "DIT_OK", -1: "DIT_EINVAL", -2: "DIT_ERANGE", -3: "DIT_ENOMEM", -4: "DIT_EDEVICE",
          -5: "DIT_EUNSUPPORTED"}


class DitError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_NAMES.get(status, status)}: {message}")
        self.status = status


class Arch(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn", C.c_int32), ("axes", C.c_int32 * 3), ("eps", C.c_float),
                ("qk_eps", C.c_float), ("final_eps", C.c_float), ("rope_theta", C.c_float),
                ("norm", C.c_int32), ("time_dim", C.c_int32), ("latent", C.c_int32),
                ("text_dim", C.c_int32)]


class Block(C.Structure):
    _fields_ = [("wtype", C.c_int32), ("w", C.c_void_p * 4), ("scale", C.c_void_p * 4),
                ("norm_w", C.c_void_p * 4), ("w_mod", C.c_void_p), ("post_w", C.c_void_p * 2)]


class Model(C.Structure):
    _fields_ = [("n_blocks", C.c_int32), ("blocks", C.POINTER(Block)), ("w_t1", C.c_void_p),
                ("w_t2", C.c_void_p), ("w_in", C.c_void_p), ("w_txt", C.c_void_p),
                ("w_fmod", C.c_void_p), ("w_final", C.c_void_p)]


_P = C.c_void_p
_SIGS = {
    "dit_ctx_create": (C.c_int, [C.POINTER(C.c_void_p), C.c_int, _P, C.POINTER(Arch), C.c_int]),
    "dit_ctx_destroy": (None, [_P]),
    "dit_ctx_set_stream": (C.c_int, [_P, _P]),
    "dit_last_error": (C.c_char_p, [_P]),
    "dit_version": (C.c_char_p, []),
    "dit_positions": (C.c_int, [_P, C.c_int, C.c_int, C.c_int, _P]),
    "dit_rope_tables": (C.c_int, [_P, _P, C.c_int, _P, _P]),
    "dit_time_vector": (C.c_int, [_P, _P, _P, C.c_float, _P]),
    "dit_time_vector_noalloc": (C.c_int, [_P, C.c_int, C.c_int, _P, _P, C.c_float, _P]),
    "dit_modulation": (C.c_int, [_P, _P, C.c_int, _P, _P]),
    "dit_modulated_norm": (C.c_int, [_P, _P, C.c_int, _P, _P, _P, C.c_float, _P]),
    "dit_linear": (C.c_int, [_P, _P, _P, _P, C.c_int, C.c_int, C.c_int, C.c_int, _P]),
    "dit_quantize_rows": (C.c_int, [_P, _P, C.c_int, C.c_int, _P, _P]),
    "dit_convrot_quantize_rows": (C.c_int, [_P, _P, C.c_int, C.c_int, _P, _P]),
    "dit_sigma_schedule": (C.c_int, [_P, C.c_int, C.c_float, _P, _P]),
    "dit_modulated_norm_int8": (C.c_int, [_P, _P, C.c_int, _P, _P, _P, C.c_float, _P, _P]),
    "dit_linear_w8a8": (C.c_int, [_P, _P, _P, _P, _P, C.c_int, C.c_int, C.c_int, _P]),
    "dit_attention": (C.c_int, [_P, _P, _P, _P, C.c_int, C.c_int, _P]),
    "dit_qk_prep": (C.c_int, [_P, _P, C.c_int, _P, _P, _P, _P, _P, _P, _P]),
    "dit_set_qk_prep": (C.c_int, [_P, C.c_int]),
    "dit_set_int8_products": (C.c_int, [_P, C.c_int]),
    "dit_block_forward": (C.c_int, [_P, C.POINTER(Block), _P, _P, _P, _P, C.c_int, C.c_int]),
    "dit_parallel_block_forward": (C.c_int, [_P, C.POINTER(Block), _P, _P, _P, _P, C.c_int, C.c_int]),
    "dit_double_block_forward": (C.c_int, [_P, C.POINTER(Block), C.POINTER(Block), _P, _P, _P, _P, C.c_int,
                                           C.c_int]),
    "dit_block_forward_cached": (C.c_int, [_P, C.POINTER(Block), _P, _P, _P, _P, C.c_int, C.c_int, C.c_int, _P,
                                           C.c_int]),
    "dit_block_forward_runs": (C.c_int, [_P, C.POINTER(Block), _P, _P, C.c_int, _P, C.c_int, _P, _P, C.c_int,
                                         C.c_int]),
    "dit_prologue": (C.c_int, [_P, C.POINTER(Model), _P, C.c_int, _P]),
    "dit_denoise_step": (C.c_int, [_P, C.POINTER(Model), _P, _P, _P, _P, C.c_int, C.c_int,
                                   C.c_float, C.c_float, _P]),
    "dit_euler_step": (C.c_int, [_P, _P, _P, C.c_int64, C.c_float, C.c_float]),
    "dit_plan_schedule": (C.c_int, [_P, C.POINTER(Model), _P, C.c_int]),
    "dit_dequant_int8_b32": (C.c_int, [_P, _P, _P, C.c_int, C.c_int, _P]),
    "dit_debug_copy": (C.c_int, [_P, C.c_int, _P, C.c_int64]),
    "dit_timing_enable": (C.c_int, [_P, C.c_int]),
    "dit_timing_read": (C.c_int, [_P, C.POINTER(C.c_double), C.POINTER(C.c_int64)]),
}
for _n, (_r, _a) in _SIGS.items():
    _f = getattr(_lib, _n)
    _f.restype = _r
    _f.argtypes = _a


def raw():
    """The loaded ctypes library (for ABI tests)."""
    return _lib


def header_functions() -> list:
    """Names of the functions include/dit.h declares."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dit_\w+)\s*\(", txt, re.M)))


def version() -> str:
    return _lib.dit_version().decode()


def last_error(ctx_ptr=None) -> str:
    return _lib.dit_last_error(ctx_ptr).decode()


def sigma_schedule(sample_sigmas, shift: float = 1.0):
    """The sampler's grid from dit_sigma_schedule: (sigmas [n + 1], t [n]) float32."""
    g = np.ascontiguousarray(np.asarray(sample_sigmas, dtype=np.float32))
    n = len(g)
    sig = np.empty(n + 1, np.float32)
    t = np.empty(n, np.float32)
    st = _lib.dit_sigma_schedule(g.ctypes.data_as(C.c_void_p), n, float(shift), sig.ctypes.data_as(C.c_void_p),
                                 t.ctypes.data_as(C.c_void_p))
    if st != OK:
        raise DitError(st, last_error(None))
    return sig, t


def make_arch(hidden=3072, heads=24, head_dim=128, ffn=12288, axes=(16, 56, 56), eps=1e-6,
              qk_eps=1e-6, final_eps=1e-6, rope_theta=10000.0, norm=NORM_LAYER, time_dim=256,
              latent=64, text_dim=4096) -> Arch:
    a = Arch()
    a.hidden, a.heads, a.head_dim, a.ffn = hidden, heads, head_dim, ffn
    a.axes[0], a.axes[1], a.axes[2] = axes
    a.eps, a.qk_eps, a.final_eps, a.rope_theta = eps, qk_eps, final_eps, rope_theta
    a.norm, a.time_dim, a.latent, a.text_dim = norm, time_dim, latent, text_dim
    return a


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def time_vector_noalloc(hidden, time_dim, w_t1, w_t2, t, vec):
    """dit_time_vector_noalloc on torch's current device and stream (no
    context; the library allocates nothing)."""
    st = _lib.dit_time_vector_noalloc(_stream(), int(hidden), int(time_dim), _ptr(w_t1, torch.bfloat16, "w_t1"),
                                      _ptr(w_t2, torch.bfloat16, "w_t2"), float(t), _ptr(vec, torch.float32, "vec"))
    if st != OK:
        raise DitError(st, last_error(None))


class Context:
    """A libdit context on one device, enqueuing on torch's current stream."""

    def __init__(self, arch: Arch, max_rows: int, device: int = 0):
        self.arch = arch
        self.max_rows = max_rows
        self.device = device
        h = C.c_void_p()
        with torch.cuda.device(device):
            st = _lib.dit_ctx_create(C.byref(h), device, _stream(), C.byref(arch), max_rows)
        if st != OK:
            raise DitError(st, last_error(None))
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None):
            torch.cuda.synchronize(self.device)
            _lib.dit_ctx_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            if getattr(self, "_h", None):
                _lib.dit_ctx_destroy(self._h)
                self._h = None
        except Exception:
            pass

    def _call(self, name, *args):
        _lib.dit_ctx_set_stream(self._h, _stream())
        st = getattr(_lib, name)(self._h, *args)
        if st != OK:
            raise DitError(st, last_error(self._h))

    # ---- entry points -----------------------------------------------------
    def positions(self, L, h, w, pos):
        self._call("dit_positions", L, h, w, _ptr(pos, torch.int32, "pos"))

    def rope_tables(self, pos, S, cos, sin):
        self._call("dit_rope_tables", _ptr(pos, torch.int32, "pos"), S,
                   _ptr(cos, torch.float32, "cos"), _ptr(sin, torch.float32, "sin"))

    def time_vector(self, w_t1, w_t2, t, vec):
        self._call("dit_time_vector", _ptr(w_t1, torch.bfloat16, "w_t1"),
                   _ptr(w_t2, torch.bfloat16, "w_t2"), float(t), _ptr(vec, torch.float32, "vec"))

    def modulation(self, w_mod, chunks, vec, mod):
        self._call("dit_modulation", _ptr(w_mod, torch.bfloat16, "w_mod"), chunks,
                   _ptr(vec, torch.float32, "vec"), _ptr(mod, torch.float32, "mod"))

    def modulated_norm(self, x, rows, shift, scale, norm_w, eps, out):
        self._call("dit_modulated_norm", _ptr(x, torch.float32, "x"), rows,
                   _ptr(shift, torch.float32, "shift"), _ptr(scale, torch.float32, "scale"),
                   _ptr(norm_w, torch.float32, "norm_w"), float(eps),
                   _ptr(out, torch.bfloat16, "out"))

    def linear(self, a, w, scale, M, N, K, out):
        wtype = W_INT8_B32 if w.dtype == torch.int8 else W_BF16
        self._call("dit_linear", _ptr(a, torch.bfloat16, "a"), _ptr(w, None, "w"),
                   _ptr(scale, torch.bfloat16, "scale"), wtype, M, N, K,
                   _ptr(out, torch.float32, "out"))

    def quantize_rows(self, x, rows, K, q, s):
        self._call("dit_quantize_rows", _ptr(x, torch.bfloat16, "x"), rows, K, _ptr(q, torch.int8, "q"),
                   _ptr(s, torch.float32, "s"))

    def convrot_quantize_rows(self, x, rows, K, q, s):
        self._call("dit_convrot_quantize_rows", _ptr(x, torch.bfloat16, "x"), rows, K, _ptr(q, torch.int8, "q"),
                   _ptr(s, torch.float32, "s"))

    def modulated_norm_int8(self, x, rows, shift, scale, norm_w, eps, q, s):
        self._call("dit_modulated_norm_int8", _ptr(x, torch.float32, "x"), rows,
                   _ptr(shift, torch.float32, "shift"), _ptr(scale, torch.float32, "scale"),
                   _ptr(norm_w, torch.float32, "norm_w"), float(eps), _ptr(q, torch.int8, "q"),
                   _ptr(s, torch.float32, "s"))

    def linear_w8a8(self, a, a_scale, w, w_scale, M, N, K, out):
        self._call("dit_linear_w8a8", _ptr(a, torch.int8, "a"), _ptr(a_scale, torch.float32, "a_scale"),
                   _ptr(w, torch.int8, "w"), _ptr(w_scale, torch.float32, "w_scale"), M, N, K,
                   _ptr(out, torch.float32, "out"))

    def qk_prep(self, qkv, S, q_norm, k_norm, cos, sin, q, k, vt):
        self._call("dit_qk_prep", _ptr(qkv, torch.bfloat16, "qkv"), S, _ptr(q_norm, torch.float32, "q_norm"),
                   _ptr(k_norm, torch.float32, "k_norm"), _ptr(cos, torch.float32, "cos"), _ptr(sin, torch.float32, "sin"),
                   _ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"), _ptr(vt, torch.bfloat16, "vt"))

    def set_qk_prep(self, fused: bool):
        self._call("dit_set_qk_prep", 1 if fused else 0)

    def set_int8_products(self, in_product: bool):
        """int8 block-32 weights: converted inside the product (True) or by
        a dequantisation pass into scratch first (False, the default)."""
        self._call("dit_set_int8_products", 1 if in_product else 0)

    def attention(self, q, k, vt, heads, S, o):
        self._call("dit_attention", _ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"),
                   _ptr(vt, torch.bfloat16, "vt"), heads, S, _ptr(o, torch.bfloat16, "o"))

    def block_forward(self, block: "BlockWeights", x, vec, cos, sin, L, N):
        self._call("dit_block_forward", C.byref(block.struct), _ptr(x, torch.float32, "x"),
                   _ptr(vec, torch.float32, "vec"), _ptr(cos, torch.float32, "cos"),
                   _ptr(sin, torch.float32, "sin"), L, N)

    def parallel_block_forward(self, block: "BlockWeights", x, vec, cos, sin, L, N):
        """The parallel block ([GZ] Block.parallel); block.w_mod is [3D, D]."""
        self._call("dit_parallel_block_forward", C.byref(block.struct), _ptr(x, torch.float32, "x"),
                   _ptr(vec, torch.float32, "vec"), _ptr(cos, torch.float32, "cos"),
                   _ptr(sin, torch.float32, "sin"), L, N)

    def block_forward_runs(self, block: "BlockWeights", x, vecs, runs, cos, sin, L, N):
        """The block with modulation rows vecs [R, D] over runs [(first, end, row), ...]."""
        r = np.ascontiguousarray(np.asarray(runs, dtype=np.int32).reshape(-1, 3))
        self._call("dit_block_forward_runs", C.byref(block.struct), _ptr(x, torch.float32, "x"),
                   _ptr(vecs, torch.float32, "vecs"), int(vecs.shape[0]), r.ctypes.data_as(C.c_void_p), len(r),
                   _ptr(cos, torch.float32, "cos"), _ptr(sin, torch.float32, "sin"), L, N)

    def block_forward_cached(self, block: "BlockWeights", x, vec, cos, sin, L, N, first, slot, record):
        """The block with reference rows [first, L+N) whose keys and values live in slot (bf16)."""
        self._call("dit_block_forward_cached", C.byref(block.struct), _ptr(x, torch.float32, "x"),
                   _ptr(vec, torch.float32, "vec"), _ptr(cos, torch.float32, "cos"), _ptr(sin, torch.float32, "sin"),
                   L, N, int(first), _ptr(slot, torch.bfloat16, "slot"), 1 if record else 0)

    def double_block_forward(self, txt: "BlockWeights", img: "BlockWeights", x, vec, cos, sin, L, N):
        """The double-stream block: rows [0, L) take `txt`, the rest `img`."""
        self._call("dit_double_block_forward", C.byref(txt.struct), C.byref(img.struct),
                   _ptr(x, torch.float32, "x"), _ptr(vec, torch.float32, "vec"),
                   _ptr(cos, torch.float32, "cos"), _ptr(sin, torch.float32, "sin"), L, N)

    def prologue(self, model: "ModelWeights", ctx_feats, L, txt):
        self._call("dit_prologue", C.byref(model.struct), _ptr(ctx_feats, torch.float32, "ctx"),
                   L, _ptr(txt, torch.float32, "txt"))

    def denoise_step(self, model: "ModelWeights", x_lat, txt, cos, sin, L, N, sigma, sigma_next,
                     vel_out=None):
        self._call("dit_denoise_step", C.byref(model.struct), _ptr(x_lat, torch.float32, "x_lat"),
                   _ptr(txt, torch.float32, "txt"), _ptr(cos, torch.float32, "cos"),
                   _ptr(sin, torch.float32, "sin"), L, N, float(sigma), float(sigma_next),
                   _ptr(vel_out, torch.float32, "vel_out"))

    def plan_schedule(self, model: "ModelWeights", sigmas):
        """dit_plan_schedule: the modulation of the steps at the host values
        `sigmas` (float32, compared bit for bit by later steps); an empty
        sequence drops the plan."""
        sg = np.ascontiguousarray(np.asarray(sigmas, dtype=np.float32))
        self._call("dit_plan_schedule", C.byref(model.struct),
                   sg.ctypes.data_as(C.c_void_p) if len(sg) else None, len(sg))

    def euler_step(self, x, v, n, sigma, sigma_next):
        self._call("dit_euler_step", _ptr(x, torch.float32, "x"), _ptr(v, torch.float32, "v"),
                   int(n), float(sigma), float(sigma_next))

    def dequant_int8_b32(self, q, s, out, inn, w_out):
        self._call("dit_dequant_int8_b32", _ptr(q, torch.int8, "q"), _ptr(s, torch.bfloat16, "s"),
                   out, inn, _ptr(w_out, torch.float32, "w_out"))

    def timing(self, on: bool):
        self._call("dit_timing_enable", 1 if on else 0)

    def timing_read(self) -> dict:
        """{stage: (total_ms, launches)} since the last read (synchronises)."""
        ms = (C.c_double * len(STAGES))()
        n = (C.c_int64 * len(STAGES))()
        self._call("dit_timing_read", ms, n)
        return {s: (ms[i], n[i]) for i, s in enumerate(STAGES)}

    def debug_copy(self, which: int, dtype, shape):
        """A fresh device tensor holding workspace buffer `which` (see
        dit_debug_copy), viewed as `shape` of `dtype`."""
        out = torch.empty(shape, dtype=dtype, device=f"cuda:{self.device}")
        self._call("dit_debug_copy", which, out.data_ptr(), out.numel() * out.element_size())
        return out


# ---------------------------------------------------------------------------
# device weights (marshalling of host arrays into device tensors + structs)
# ---------------------------------------------------------------------------

def dev_bf16(a, device="cuda"):
    """float32 values (already bf16-representable) -> device bf16 tensor."""
    return torch.from_numpy(a).to(device=device).to(torch.bfloat16).contiguous()


def dev_f32(a, device="cuda"):
    return torch.from_numpy(a).to(device=device, dtype=torch.float32).contiguous()


class BlockWeights:
    """Device tensors of one block plus the dit_block struct that points at
    them.  `w` holds bf16 [out, in] tensors (or int8 codes with `scale`)."""

    LIN = ("w_qkv", "w_out", "w_up", "w_down")

    def __init__(self, tensors: dict, int8: bool = False, rotated: bool = False):
        self.t = tensors
        self.int8 = int8
        w8a8 = "q8_w_qkv" in tensors
        b = Block()
        b.wtype = (W_INT8_ROT if rotated else W_INT8_ROW) if w8a8 else W_INT8_B32 if int8 else W_BF16
        for i, n in enumerate(self.LIN):
            if w8a8:
                b.w[i] = _ptr(tensors["q8_" + n], torch.int8, "q8_" + n)
                b.scale[i] = _ptr(tensors["s8_" + n], torch.float32, "s8_" + n)
            elif int8:
                b.w[i] = _ptr(tensors["q_" + n], torch.int8, "q_" + n)
                b.scale[i] = _ptr(tensors["s_" + n], torch.bfloat16, "s_" + n)
            else:
                b.w[i] = _ptr(tensors[n], torch.bfloat16, n)
                b.scale[i] = None
        for i, n in enumerate(("norm1", "norm2", "q_norm", "k_norm")):
            b.norm_w[i] = _ptr(tensors.get(n), torch.float32, n)
        b.w_mod = _ptr(tensors["w_mod"], torch.bfloat16, "w_mod")
        for i, n in enumerate(("post_attn", "post_mlp")):
            b.post_w[i] = _ptr(tensors.get(n), torch.float32, n)
        self.struct = b

    @classmethod
    def from_host(cls, bw: dict, device="cuda", rotated: bool = False):
        """From synth.block_weights' dict (float32 values / int8 codes);
        rotated: W8A8 rows in ConvRot's basis (DIT_W_INT8_ROT)."""
        t = {}
        int8 = "q_w_qkv" in bw
        for k, v in bw.items():
            if k.startswith("q_w") or k.startswith("q8_w"):
                t[k] = torch.from_numpy(v).to(device)
            elif k in ("q_norm", "k_norm", "norm1", "norm2", "post_attn", "post_mlp") or k.startswith("s8_w"):
                t[k] = dev_f32(v, device)
            else:
                t[k] = dev_bf16(v, device)
        return cls(t, int8=int8, rotated=rotated)


class ModelWeights:
    TOP = ("w_t1", "w_t2", "w_in", "w_txt", "w_fmod", "w_final")

    def __init__(self, top: dict, blocks: list):
        self.top = top
        self.blocks = blocks
        arr = (Block * max(1, len(blocks)))()
        for i, b in enumerate(blocks):
            arr[i] = b.struct
        self._arr = arr
        m = Model()
        m.n_blocks = len(blocks)
        m.blocks = C.cast(arr, C.POINTER(Block))
        for n in self.TOP:
            setattr(m, n, _ptr(top[n], torch.bfloat16, n))
        self.struct = m

    @classmethod
    def from_host(cls, top: dict, blocks: list, device="cuda"):
        return cls({k: dev_bf16(v, device) for k, v in top.items()},
                   [BlockWeights.from_host(b, device) for b in blocks])
