"""C ABI checks that need no GPU: the library loads, exports every function
include/dit.h declares, and rejects bad arguments before any device work."""

import ctypes as C
import re

import pytest

torch = pytest.importorskip("torch")

try:
    from diffusion_transformer_amd import lib as L
except ImportError as e:          # libdit.so not built
    pytest.skip(f"libdit.so unavailable: {e}", allow_module_level=True)


def test_exports_every_declared_function():
    names = L.header_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L.raw(), n), f"{n} declared in dit.h but not exported"


def test_header_declares_what_binding_calls():
    names = set(L.header_functions())
    assert set(L._SIGS) <= names


def test_exports_are_c_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    syms = set(re.findall(r"\bT (dit_\w+)", out))
    assert set(L.header_functions()) <= syms


def test_version_and_null_context():
    assert "gfx950" in L.version()
    lib = L.raw()
    assert lib.dit_positions(None, 1, 1, 1, None) == L.EINVAL
    assert "NULL" in L.last_error(None)
    assert lib.dit_euler_step(None, None, None, 0, 1.0, 0.0) == L.EINVAL
    assert lib.dit_block_forward(None, None, None, None, None, None, 0, 1) == L.EINVAL
    assert lib.dit_set_qk_prep(None, 1) == L.EINVAL
    assert lib.dit_set_int8_products(None, 0) == L.EINVAL
    assert lib.dit_plan_schedule(None, None, None, 0) == L.EINVAL
    assert lib.dit_ctx_set_stream(None, None) == L.EINVAL
    lib.dit_ctx_destroy(None)      # no-op


def _create(arch, max_rows=128):
    h = C.c_void_p()
    st = L.raw().dit_ctx_create(C.byref(h), 0, None, C.byref(arch), max_rows)
    return st, h


@pytest.mark.parametrize("mut,status", [
    (dict(head_dim=64, hidden=128, heads=2), L.EUNSUPPORTED),
    (dict(hidden=300), L.EINVAL),
    (dict(ffn=1000), L.EUNSUPPORTED),
    (dict(axes=(16, 56, 58)), L.EINVAL),
    (dict(axes=(15, 57, 56)), L.EINVAL),
    (dict(norm=7), L.EINVAL),
    (dict(eps=0.0), L.EINVAL),
    (dict(latent=48), L.EINVAL),
])
def test_ctx_create_rejects_bad_arch_before_device(mut, status):
    kw = dict(hidden=256, heads=2, ffn=1024)
    kw.update(mut)
    st, h = _create(L.make_arch(**kw))
    assert st == status, L.last_error(None)
    assert not h.value


def test_ctx_create_rejects_bad_rows():
    st, h = _create(L.make_arch(hidden=256, heads=2, ffn=1024), max_rows=0)
    assert st == L.ERANGE
    st, h = _create(L.make_arch(hidden=256, heads=2, ffn=1024), max_rows=70000)
    assert st == L.ERANGE


def test_ctx_create_without_gpu_reports_device():
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, h = _create(L.make_arch(hidden=256, heads=2, ffn=1024))
    assert st == L.EDEVICE
    assert not h.value


def test_struct_layouts_match_the_header(tmp_path):
    # compile a host-only probe of the header with the system C compiler and
    # compare sizes and field offsets with the binding's ctypes structures
    import os
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    fields = {"dit_arch": L.Arch, "dit_block": L.Block, "dit_model": L.Model}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "dit.h"', "int main(void) {"]
    for cname, ct in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in ct._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run([cc, "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    for line in filter(None, out):
        cname, what, val = line.split()
        ct = fields[cname]
        got = C.sizeof(ct) if what == "size" else getattr(ct, what).offset
        assert got == int(val), f"{cname}.{what}: binding {got}, header {val}"
