"""The allocation-free entry point (dit_time_vector_noalloc) against the
context entry point it varies (dit_time_vector): bit for bit, on two calls
in a row whose second is smaller, and against the oracle."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from gpu_util import L, O, compare, np_of, say, synth, torch  # noqa: E402


def _weights(hidden, time_dim, seed):
    w1 = synth.bf16_round(synth.normal((hidden, time_dim), seed, 0.02))
    w2 = synth.bf16_round(synth.normal((hidden, hidden), seed + 1, 0.02))
    return w1, w2


def _with_context(hidden, time_dim, w1, w2, t):
    ctx = L.Context(L.make_arch(hidden=hidden, heads=hidden // 128, ffn=4 * hidden, time_dim=time_dim), max_rows=64)
    vec = torch.empty(hidden, dtype=torch.float32, device="cuda")
    ctx.time_vector(L.dev_bf16(w1), L.dev_bf16(w2), t, vec)
    torch.cuda.synchronize()
    ctx.close()
    return np_of(vec)


def test_noalloc_time_vector_matches_the_context_entry_point():
    cases = [(3072, 256, 0.8125, 31), (256, 128, 0.25, 32)]     # the second call is smaller
    got = []
    for hidden, time_dim, t, seed in cases:
        say("time vector noalloc", hidden, time_dim, t)
        w1, w2 = _weights(hidden, time_dim, seed)
        vec = torch.full((hidden,), float("nan"), dtype=torch.float32, device="cuda")
        L.time_vector_noalloc(hidden, time_dim, L.dev_bf16(w1), L.dev_bf16(w2), t, vec)
        torch.cuda.synchronize()
        got.append((np_of(vec), hidden, time_dim, t, w1, w2))
    for v, hidden, time_dim, t, w1, w2 in got:
        ref = _with_context(hidden, time_dim, w1, w2, t)
        assert (v.view(np.uint32) == ref.view(np.uint32)).all(), "differs from dit_time_vector"
        compare(f"vec-{hidden}", v, O.time_vector(t, w1, w2, time_dim), rel=1e-4, abs_=1e-4)


def test_noalloc_time_vector_rejects_sizes_beyond_its_array():
    w = torch.zeros((8, 8), dtype=torch.bfloat16, device="cuda")
    vec = torch.zeros(8192, dtype=torch.float32, device="cuda")
    for hidden, time_dim in [(8192, 256), (256, 8200), (0, 256), (260, 256)]:
        with pytest.raises(L.DitError) as e:
            L.time_vector_noalloc(hidden, time_dim, w, w, 0.5, vec)
        assert e.value.status == L.ERANGE
