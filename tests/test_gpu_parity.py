"""GPU parity: every entry point of libdit against the CPU oracle, on seeded
inputs from diffusion_transformer_amd.synth.

Integer and index work (positions, rotary tables, int8 dequantisation, the
Euler update, the zero-gate identity) must match bit for bit; floating point
is held to relative L2 <= 2e-2 and max abs <= 5e-2 (tighter where the kernel
does exact-input fp32 arithmetic only).  Shapes cover several tiles on every
grid axis, ragged tails and the full 1024-px block.
"""

import contextlib
import ctypes as C

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from gpu_util import (L, O, REL, ABS, GpuSeq, arch_pair, block_abs, compare, np_of, oracle_block,  # noqa: E402
                      rel_l2, say, synth, torch)


@pytest.fixture(scope="module")
def ctx_tiny():
    sh = synth.SHAPES["tiny"]
    la, _ = arch_pair(sh)
    c = L.Context(la, max_rows=4608)
    yield c
    c.close()


@pytest.fixture(scope="module")
def ctx_big():
    sh = synth.SHAPES["s4608"]
    la, _ = arch_pair(sh)
    c = L.Context(la, max_rows=4608)
    yield c
    c.close()


@contextlib.contextmanager
def int8_products(ctx, in_product):
    """int8 block-32 weights converted inside the products (True) or by the
    dequantisation pass (False, the default) for the body of the block."""
    ctx.set_int8_products(bool(in_product))
    try:
        yield
    finally:
        ctx.set_int8_products(False)


# the int8 block-32 workload in both conversion placements
BLOCK_FORMS = [("s4608", False), ("s4608_int8", False), ("s4608_int8", True)]


# --------------------------------------------------------------- positions, rope

@pytest.mark.parametrize("Lh", [(8, 8, 8), (512, 64, 64), (64, 32, 32), (0, 3, 5), (7, 16, 16), (1, 1, 1),
                                (5, 9, 13)])
def test_positions_and_rope_tables_bit_exact(ctx_big, Lh):
    Ln, h, w = Lh
    S = Ln + h * w
    say("positions/rope", Lh)
    pos = torch.empty((S, 3), dtype=torch.int32, device="cuda")
    ctx_big.positions(Ln, h, w, pos)
    cs = torch.empty((S, 64), dtype=torch.float32, device="cuda")
    sn = torch.empty_like(cs)
    ctx_big.rope_tables(pos, S, cs, sn)
    torch.cuda.synchronize()
    ref = O.positions(Ln, h, w)
    assert (np_of(pos) == ref).all()
    rc, rs = O.rope_tables(ref, (16, 56, 56))
    gc, gs = np_of(cs), np_of(sn)
    bad = int((gc != rc).sum() + (gs != rs).sum())
    assert bad == 0, f"{bad} table entries differ"


# --------------------------------------------------------------- small steps

@pytest.mark.parametrize("name", ["tiny", "w4096", "s4608"])
def test_time_vector_and_modulation(ctx_tiny, ctx_big, name):
    # w4096: inputs wider than 3072 (the GEMV's other register layout)
    case = synth.block_case(name)
    sh = case["shape"]
    ctx = {"tiny": ctx_tiny, "s4608": ctx_big}.get(name) or L.Context(arch_pair(sh)[0], max_rows=sh.S)
    say("time_vector/modulation", name)
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    vref = O.time_vector(float(case["t"]), case["w_t1"], case["w_t2"], sh.time_dim)
    torch.cuda.synchronize()
    compare("vec", np_of(seq.vec), vref, rel=1e-4, abs_=1e-4)
    wm = L.dev_bf16(case["block"]["w_mod"])
    mod = torch.empty(6 * sh.hidden, dtype=torch.float32, device="cuda")
    ctx.modulation(wm, 6, seq.vec, mod)
    torch.cuda.synchronize()
    mref = O.modulation(vref, case["block"]["w_mod"], 6).reshape(-1)
    compare("mod", np_of(mod), mref, rel=1e-4, abs_=1e-4)


@pytest.mark.parametrize("norm", ["layer", "rms"])
@pytest.mark.parametrize("rows,D", [(72, 256), (4608, 3072), (5, 3072), (72, 4096)])
def test_modulated_norm(norm, rows, D):
    sh = synth.Shape("n", D, D // 128, 128, 1024, 0, 1, rows, seed=0)
    la, oa = arch_pair(sh, norm)
    ctx = L.Context(la, max_rows=max(rows, 64))
    say("modulated_norm", norm, rows, D)
    x = synth.normal((rows, D), seed=rows + D, std=2.0, mean=0.5)
    shift = synth.normal(D, seed=rows + D + 1, std=0.3)
    scale = synth.normal(D, seed=rows + D + 2, std=0.3)
    nw = synth.normal(D, seed=rows + D + 3, std=0.1, mean=1.0)
    out = torch.empty((rows, D), dtype=torch.bfloat16, device="cuda")
    ctx.modulated_norm(L.dev_f32(x), rows, L.dev_f32(shift), L.dev_f32(scale),
                       L.dev_f32(nw) if norm == "rms" else None, 1e-6, out)
    torch.cuda.synchronize()
    ref = O.modulated_norm(x, shift, scale, oa, nw if norm == "rms" else None)
    compare("h", np_of(out), ref, bf16_stored=True)
    # bf16 output: within one bf16 rounding (2^-8 relative) plus fp32 noise
    assert np.abs(np_of(out) - ref).max() <= np.abs(ref).max() * 2 ** -8 + 1e-5
    ctx.close()


# --------------------------------------------------------------- products

@pytest.mark.parametrize("M,N,K", [(72, 256, 256), (1088, 3072, 3072), (4608, 64, 3072), (4096, 3072, 64),
                                   (333, 768, 1024), (1, 128, 128), (4608, 9216, 3072), (4608, 2048, 128),
                                   (4608, 3072, 12288)])
@pytest.mark.parametrize("w8", [False, "pass", "in_product"])
def test_linear(ctx_big, M, N, K, w8):
    say("linear", M, N, K, f"int8 ({w8})" if w8 else "bf16")
    rng = np.random.default_rng(M * 7 + N + K)
    a = synth.bf16_round(synth.normal((M, K), seed=M * 7 + N + K))
    if w8:
        # the products take code * scale rounded to the nearest bf16 (ties to
        # even): against those operands the int8 product is held to the bf16
        # product's bound, which a truncating or otherwise misrounded
        # dequantisation exceeds (its weights differ by up to 2^-8 relative)
        q, s = synth.int8_weight(rng, N, K)
        wref = O.dequant_int8_b32_bf16(q, s)
        w_dev, s_dev = torch.from_numpy(q).cuda(), L.dev_bf16(s)
    else:
        wref = synth.bf16_round(synth.normal((N, K), seed=M + N * 3 + K, std=0.05))
        w_dev, s_dev = L.dev_bf16(wref), None
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    with int8_products(ctx_big, w8 == "in_product"):
        ctx_big.linear(L.dev_bf16(a), w_dev, s_dev, M, N, K, out)
        torch.cuda.synchronize()
    rows = np.arange(M) if M * N * K <= 2 ** 33 else synth.rows_sample(M, 300)
    ref = O.linear(a[rows], wref)
    got = np_of(out)[rows]
    # exact bf16 products, fp32 accumulation: only the summation order differs
    r, m = compare("linear-int8" if w8 else "linear-bf16", got, ref, rel=1e-5,
                   abs_=1e-3 * max(1.0, np.abs(ref).max()))
    if w8:
        # the exact (unrounded) weights are measurably further away: the
        # bound above pins the rounding itself
        far = O.linear(a[rows], O.dequant_int8_b32(q, s))
        assert rel_l2(got, far) > 4 * max(r, 1e-7), "the product's weights are not the rounded ones"


def test_dequant_bit_exact(ctx_big):
    rng = np.random.default_rng(44)
    for out_, in_ in [(3, 32), (96, 3072), (7, 12288)]:
        q, s = synth.int8_weight(rng, out_, in_)
        w = torch.empty((out_, in_), dtype=torch.float32, device="cuda")
        ctx_big.dequant_int8_b32(torch.from_numpy(q).cuda(), L.dev_bf16(s), out_, in_, w)
        torch.cuda.synchronize()
        assert (np_of(w) == O.dequant_int8_b32(q, s)).all()


@pytest.mark.parametrize("n", [0, 1, 1001, 4096 * 64])
def test_euler_bit_exact(ctx_big, n):
    x = synth.normal(max(n, 1), seed=n)[:n]
    v = synth.normal(max(n, 1), seed=n + 1)[:n]
    sig = O.sigma_grid(4)
    xd = L.dev_f32(x.copy()) if n else torch.empty(0, device="cuda")
    vd = L.dev_f32(v) if n else torch.empty(0, device="cuda")
    ref = x.copy()
    for i in range(4):
        if n:
            ctx_big.euler_step(xd, vd, n, float(sig[i]), float(sig[i + 1]))
        ref = O.euler_step(ref, v, sig[i], sig[i + 1])
    torch.cuda.synchronize()
    if n:
        assert (np_of(xd) == ref).all()


# --------------------------------------------------------------- attention

def _attn_inputs(H, S, seed, peak=1.0):
    q = synth.bf16_round(synth.normal((H, S, 128), seed=seed, std=peak))
    k = synth.bf16_round(synth.normal((H, S, 128), seed=seed + 1))
    v = synth.bf16_round(synth.normal((H, S, 128), seed=seed + 2))
    return q, k, v


def _run_attention(ctx, q, k, v):
    H, S, _ = q.shape
    Sp = (S + 63) // 64 * 64
    vt = np.zeros((H, 128, Sp), np.float32)
    vt[:, :, S:] = np.nan                      # padding must never be read into the result
    vt[:, :, :S] = v.transpose(0, 2, 1)
    o = torch.empty((S, H * 128), dtype=torch.bfloat16, device="cuda")
    vt_dev = torch.from_numpy(vt).cuda().to(torch.bfloat16)
    ctx.attention(L.dev_bf16(q), L.dev_bf16(k), vt_dev, H, S, o)
    torch.cuda.synchronize()
    return np_of(o)


@pytest.mark.parametrize("H,S,peak", [(2, 1, 1.0), (2, 7, 1.0), (2, 64, 1.0), (2, 72, 1.0), (3, 200, 3.0),
                                      (24, 1088, 1.0), (2, 4608, 2.0)])
def test_attention(ctx_big, H, S, peak):
    say("attention", H, S, peak)
    q, k, v = _attn_inputs(H, S, H * 1000 + S, peak)
    got = _run_attention(ctx_big, q, k, v)
    rows = np.arange(S) if S <= 1088 else synth.rows_sample(S, 200)
    ref = O.attention(q[:, rows], k, v).transpose(1, 0, 2).reshape(len(rows), H * 128)
    compare("attention", got[rows], ref, bf16_stored=True)


@pytest.mark.parametrize("S", [1, 5, 16, 17, 63, 65, 127, 128, 129, 191, 192, 193, 255, 257, 321])
def test_attention_tile_boundaries(ctx_big, S):
    """Key counts on and around the 64-key tiles: one to six tiles, full or
    with a ragged last tile, so that every form of the per-wave pipeline
    runs (the first tile's scores in the prologue, the inner tiles, the
    masked tile before the last, the last tile's products) and the padding
    of the last value tile (NaN here) is never read; down to one key and
    query, fewer than one 16-row matrix block."""
    H = 3
    say("attention tile boundaries", H, S)
    q, k, v = _attn_inputs(H, S, 7000 + S, 2.0)
    got = _run_attention(ctx_big, q, k, v)
    ref = O.attention(q, k, v).transpose(1, 0, 2).reshape(S, H * 128)
    assert np.isfinite(got).all()
    compare(f"attention-S{S}", got, ref, bf16_stored=True)


def test_attention_degenerate_keys(ctx_big):
    # all keys equal -> every output row is the mean of the values
    H, S = 2, 150
    q, k, v = _attn_inputs(H, S, 5)
    k[:] = k[:, :1]
    got = _run_attention(ctx_big, q, k, v)
    ref = np.repeat(v.mean(axis=1, keepdims=True), S, axis=1).transpose(1, 0, 2).reshape(S, H * 128)
    compare("attention-equal-keys", got, ref, bf16_stored=True)


def test_attention_large_logits(ctx_big):
    """Scores of hundreds of nats, with the first key tile far below the
    best keys for half the queries and far above them for the other half:
    the running maximum then moves by hundreds (base-2 units) in both
    directions across the queries of one wave.  The output must stay finite
    and match the oracle (each row is essentially the mean of its best keys'
    values)."""
    H, S = 2, 300
    rng = np.random.default_rng(77)
    u = np.where(rng.random(128) < 0.5, -1.0, 1.0).astype(np.float32)
    sign = np.where(np.arange(S) % 2 == 0, 1.0, -1.0).astype(np.float32)[:, None]
    q = synth.bf16_round(np.broadcast_to(10.0 * sign * u, (H, S, 128)) + rng.standard_normal((H, S, 128)).astype(np.float32))
    k = rng.standard_normal((H, S, 128)).astype(np.float32)
    k[:, :64] += -3.0 * u                    # first key tile: -340 nats for even queries, +340 for odd
    k[:, 200:210] += 3.0 * u                 # ten keys 64+ tiles later: the reverse
    k = synth.bf16_round(k)
    v = synth.bf16_round(rng.standard_normal((H, S, 128)).astype(np.float32))
    say("attention large logits", H, S)
    got = _run_attention(ctx_big, q, k, v)
    ref = O.attention(q, k, v).transpose(1, 0, 2).reshape(S, H * 128)
    assert np.isfinite(got).all()
    compare("attention-large-logits", got, ref, bf16_stored=True)


# --------------------------------------------------------------- block forward

def _block_gpu(ctx, case, norm="layer"):
    sh = case["shape"]
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    x = L.dev_f32(case["x"])
    ctx.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    torch.cuda.synchronize()
    return x, seq, bw


def _oracle_inputs(case, oa):
    sh = case["shape"]
    pos = O.positions(sh.L, sh.h, sh.w)
    cs, sn = O.rope_tables(pos, sh.axes)
    vec = O.time_vector(float(case["t"]), case["w_t1"], case["w_t2"], sh.time_dim)
    return cs, sn, vec


def _intermediates(ctx, sh, S):
    D, H, F = sh.hidden, sh.heads, sh.ffn
    Sp = (S + 63) // 64 * 64
    return dict(
        mod=np_of(ctx.debug_copy(0, torch.float32, (6, D))),
        h=np_of(ctx.debug_copy(1, torch.bfloat16, (S, D))),
        q=np_of(ctx.debug_copy(2, torch.bfloat16, (H, S, 128))),
        k=np_of(ctx.debug_copy(3, torch.bfloat16, (H, S, 128))),
        v=np_of(ctx.debug_copy(4, torch.bfloat16, (H, 128, Sp)))[:, :, :S].transpose(0, 2, 1),
        o=np_of(ctx.debug_copy(5, torch.bfloat16, (S, D))),
        h2=np_of(ctx.debug_copy(6, torch.bfloat16, (S, D))),
        a=np_of(ctx.debug_copy(7, torch.bfloat16, (S, F))),
    )


@pytest.mark.parametrize("name,norm,norm_std", [("tiny", "layer", 0.0), ("tiny", "rms", 0.1),
                                                 ("t_img", "layer", 0.0), ("t_one", "rms", 0.1),
                                                 ("t_few", "layer", 0.0), ("m640", "rms", 0.1),
                                                 ("w4096", "layer", 0.0),
                                                 ("s1088", "layer", 0.0), ("r1077", "rms", 0.1)])
def test_block_full_parity(name, norm, norm_std):
    # r1077: 77 text + 25 x 40 image rows, ragged against the 64-key
    # attention tiles and the 256-row product tiles at the full width;
    # t_img, t_one, t_few: no text rows, a single row, five rows
    case = synth.block_case(name, norm_std=norm_std, rms=(norm == "rms"))
    sh = case["shape"]
    la, oa = arch_pair(sh, norm)
    ctx = L.Context(la, max_rows=sh.S)
    say("block", name, norm, "S =", sh.S)
    x, _, _ = _block_gpu(ctx, case, norm)
    got = np_of(x)
    inter = _intermediates(ctx, sh, sh.S)
    cs, sn, vec = _oracle_inputs(case, oa)
    y, ref = O.block_forward(case["x"], oracle_block(case["block"]), vec, cs, sn, oa, keep=True)
    compare(f"{name}/mod", inter["mod"], ref["mod"], rel=1e-4, abs_=1e-4)
    for k in ("h", "q", "k", "v", "o", "h2", "a"):   # x1 is updated in place: checked through y
        compare(f"{name}/{k}", inter[k], ref[k], bf16_stored=True)
    compare(f"{name}/y", got, y)
    compare(f"{name}/delta", got - case["x"], y - case["x"])
    ctx.close()


def test_arm_switches_reject_other_values(ctx_tiny):
    for fn in ("dit_set_qk_prep", "dit_set_int8_products"):
        for v in (-1, 2):
            assert getattr(L.raw(), fn)(ctx_tiny.handle, v) == L.EINVAL
    assert L.raw().dit_set_int8_products(ctx_tiny.handle, 0) == L.OK


@pytest.mark.parametrize("name", ["tiny", "t_one", "t_few", "m640", "w4096", "s1088", "r1077"])
@pytest.mark.parametrize("in_product", [False, True])
def test_block_int8_full_parity(name, in_product):
    """int8 block-32 weights in the sequential block, every row and
    intermediate against the oracle.  A block with other int8 weights runs
    first on the same context, not waited for: the dequantised copies of the
    second block's weights (scratch shared by all calls, the later weights
    converted on the context's second stream) must not mix with the
    first's."""
    case = synth.block_case(name)
    sh = case["shape"]
    case["block"] = synth.block_weights(np.random.default_rng(sh.seed + 50), sh, int8=True)
    other = synth.block_weights(np.random.default_rng(sh.seed + 51), sh, int8=True)
    la, oa = arch_pair(sh)
    ctx = L.Context(la, max_rows=sh.S)
    ctx.set_int8_products(in_product)
    say("block int8", name, "in product" if in_product else "dequantisation pass", "S =", sh.S)
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    bo, bw = L.BlockWeights.from_host(other), L.BlockWeights.from_host(case["block"])
    x0, x = L.dev_f32(case["x"]), L.dev_f32(case["x"])
    ctx.block_forward(bo, x0, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    ctx.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    torch.cuda.synchronize()
    got = np_of(x)
    inter = _intermediates(ctx, sh, sh.S)
    cs, sn, vec = _oracle_inputs(case, oa)
    y, ref = O.block_forward(case["x"], oracle_block(case["block"]), vec, cs, sn, oa, keep=True)
    for k in ("h", "q", "k", "v", "o", "h2", "a"):
        compare(f"{name}-int8/{k}", inter[k], ref[k], abs_=block_abs(ref[k]), bf16_stored=True)
    compare(f"{name}-int8/y", got, y, abs_=block_abs(y))
    d = y - case["x"]
    compare(f"{name}-int8/delta", got - case["x"], d, abs_=block_abs(d))
    ctx.close()


@pytest.mark.parametrize("name,in_product", BLOCK_FORMS)
def test_block_full_size_sampled_rows(ctx_big, name, in_product):
    case = synth.block_case(name)
    sh = case["shape"]
    _, oa = arch_pair(sh)
    say("block", name, "S =", sh.S, "int8 in product" if in_product else "")
    with int8_products(ctx_big, in_product):
        x, _, _ = _block_gpu(ctx_big, case)
    got = np_of(x)
    inter = _intermediates(ctx_big, sh, sh.S)
    cs, sn, vec = _oracle_inputs(case, oa)
    rows = synth.rows_sample(sh.S, 48, L=sh.L)
    y, o, x1, a = O.block_forward_rows(case["x"], oracle_block(case["block"]), vec, cs, sn, oa, rows)
    sc = (lambda r: block_abs(r)) if sh.int8 else (lambda r: ABS)
    compare(f"{name}/o", inter["o"][rows], o, abs_=sc(o), bf16_stored=True)
    compare(f"{name}/a", inter["a"][rows], a, abs_=sc(a), bf16_stored=True)
    compare(f"{name}/y", got[rows], y, abs_=sc(y))
    d = y - case["x"][rows]
    compare(f"{name}/delta", got[rows] - case["x"][rows], d, abs_=sc(d))


def test_block_zero_modulation_is_identity(ctx_tiny):
    case = synth.block_case("tiny")
    case["block"]["w_mod"][:] = 0.0
    x, _, _ = _block_gpu(ctx_tiny, case)
    assert (np_of(x) == case["x"]).all()


@pytest.mark.parametrize("name", ["tiny", "s1088"])
def test_block_rotary_special_tables_bit_exact(name):
    """The rotation inside the QKV product's epilogue with special tables
    (tiny: the register epilogue; 512 px: the LDS-staged one): with cos = 0,
    sin = 1 every pair (a, b) of q and k must come out as (-b, a) of the
    cos = 1, sin = 0 run bit for bit; with the quarter turn at one (row,
    pair) only, that pair alone moves.  The identity run is the oracle's
    head norm (no rotation)."""
    case = synth.block_case(name)
    sh = case["shape"]
    la, oa = arch_pair(sh)
    ctx = L.Context(la, max_rows=sh.S)
    S, H = sh.S, sh.heads
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    say("rotary special tables", name)

    def qk_with(cs, sn):
        x = L.dev_f32(case["x"])
        ctx.block_forward(bw, x, seq.vec, L.dev_f32(cs), L.dev_f32(sn), sh.L, sh.N)
        q = ctx.debug_copy(2, torch.bfloat16, (H, S, 128)).view(torch.int16).cpu().numpy()
        k = ctx.debug_copy(3, torch.bfloat16, (H, S, 128)).view(torch.int16).cpu().numpy()
        torch.cuda.synchronize()
        return q, k

    one, zero = np.ones((S, 64), np.float32), np.zeros((S, 64), np.float32)
    q_id, k_id = qk_with(one, zero)
    q_qt, k_qt = qk_with(zero, one)
    r_s, p_s = S // 2 + 1, 41
    c1, s1 = one.copy(), zero.copy()
    c1[r_s, p_s], s1[r_s, p_s] = 0.0, 1.0
    q_oh, k_oh = qk_with(c1, s1)

    def turned(t):           # (a, b) -> (-b, a) on bf16 bit patterns
        out = t.copy()
        out[..., 0::2] = t[..., 1::2] ^ np.int16(-0x8000)
        out[..., 1::2] = t[..., 0::2]
        return out

    for nm, idt, qt, oh in (("q", q_id, q_qt, q_oh), ("k", k_id, k_qt, k_oh)):
        assert (qt == turned(idt)).all(), f"{nm}: quarter turn is not (-b, a) of the identity run"
        want = idt.copy()
        want[:, r_s, 2 * p_s:2 * p_s + 2] = turned(idt)[:, r_s, 2 * p_s:2 * p_s + 2]
        assert (oh == want).all(), f"{nm}: a one-hot angle moved more than its pair"
        assert (oh[:, r_s, 2 * p_s:2 * p_s + 2] != idt[:, r_s, 2 * p_s:2 * p_s + 2]).any()
    # the identity run against the oracle's head norm with no rotation
    cs, sn, vec = _oracle_inputs(case, oa)
    _, ref = O.block_forward(case["x"], oracle_block(case["block"]), vec, one, zero, oa, keep=True)
    as_f = lambda t: (t.astype(np.int32).astype(np.uint32) << 16).view(np.float32)
    compare(f"{name}/q-identity", as_f(q_id), ref["q"], bf16_stored=True)
    compare(f"{name}/k-identity", as_f(k_id), ref["k"], bf16_stored=True)
    ctx.close()


@pytest.mark.parametrize("name", ["s4608", "s4608_int8"])
def test_block_forward_repeats_bit_identical(ctx_big, name):
    """The same block on the same rows, three times in a row: every kernel
    (the attention's per-wave pipeline, the products' tile schedules, the
    int8 dequantisation on the second stream) gives the same bits."""
    case = synth.block_case(name)
    sh = case["shape"]
    seq = GpuSeq(ctx_big, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    say("block repeats", name)
    outs = []
    for _ in range(3):
        x = L.dev_f32(case["x"])
        ctx_big.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
        outs.append(x)
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("kind", ["bf16", "int8", "w8a8"])
def test_block_independent_of_earlier_calls(ctx_big, kind):
    """One context runs blocks of different lengths in turn (the full
    1024-px sequence, ragged ones, a single row); every result equals the
    same call on a fresh context bit for bit, so nothing a call leaves in
    the workspace (padding of the transposed values, rows past S, the
    dequantised weights, the INT8 rows of W8A8 products) reaches a later
    one."""
    case = synth.block_case({"bf16": "s1088", "int8": "s4608_int8", "w8a8": "s4608_w8a8"}[kind])
    base = case["shape"]
    bw = L.BlockWeights.from_host(case["block"])
    shapes = [(512, 64, 64), (77, 25, 40), (0, 1, 1), (3, 1, 2), (64, 32, 32), (5, 9, 13)]
    for k, (Ln, h, w) in enumerate(shapes):
        sh = synth.Shape("seq", base.hidden, base.heads, 128, base.ffn, Ln, h, w, seed=100 + k)
        say("independent of earlier calls", kind, sh.L, sh.N)
        x0 = synth.normal((sh.S, sh.hidden), seed=100 + k)
        outs = []
        for fresh in (False, True):
            ctx = L.Context(L.make_arch(), max_rows=4608) if fresh else ctx_big
            seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
            x = L.dev_f32(x0)
            ctx.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
            torch.cuda.synchronize()
            outs.append(x)
            if fresh:
                ctx.close()
        assert torch.equal(outs[0], outs[1]), (Ln, h, w)


def test_block_rejects_bad_rows(ctx_tiny):
    case = synth.block_case("tiny")
    sh = case["shape"]
    seq = GpuSeq(ctx_tiny, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    x = L.dev_f32(case["x"])
    for Ln, N in [(513, 8), (8, 0), (8, 4097), (-1, 8)]:
        with pytest.raises(L.DitError) as e:
            ctx_tiny.block_forward(bw, x, seq.vec, seq.cos, seq.sin, Ln, N)
        assert e.value.status == L.ERANGE


def _shifted(t, elems):
    """A contiguous view of t's storage starting `elems` elements later (so
    misaligned by elems * itemsize bytes), same shape: the allocation gets
    one extra row to hold it."""
    flat = torch.empty(t.numel() + 64, dtype=t.dtype, device=t.device)
    flat[elems:elems + t.numel()].copy_(t.reshape(-1))
    return flat[elems:elems + t.numel()].view(t.shape)


@pytest.mark.parametrize("what", ["w_qkv", "q_w_down", "s_w_up", "w_mod", "k_norm", "x"])
def test_block_rejects_misaligned_pointers(ctx_tiny, what):
    """Weights and x the kernels read in 16-byte pieces (block-32 scales in
    4-byte ones) are refused with DIT_EINVAL before any launch."""
    case = synth.block_case("tiny")
    sh = case["shape"]
    seq = GpuSeq(ctx_tiny, sh, case["t"], case["w_t1"], case["w_t2"])
    blk = case["block"]
    if what in ("q_w_down", "s_w_up"):
        blk = synth.block_weights(np.random.default_rng(7), sh, int8=True)
    bw = L.BlockWeights.from_host(blk)
    x = L.dev_f32(case["x"])
    if what == "x":
        x = _shifted(x, 2)
    else:
        t = dict(bw.t)
        t[what] = _shifted(t[what], 1)
        bw = L.BlockWeights(t, int8=bw.int8)
    x0 = x.clone()
    with pytest.raises(L.DitError) as e:
        ctx_tiny.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    assert e.value.status == L.EINVAL
    assert "aligned" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(x, x0)


def test_linear_rejects_misaligned_weights(ctx_tiny):
    rng = np.random.default_rng(3)
    a = L.dev_bf16(rng.standard_normal((64, 128)).astype(np.float32))
    w = L.dev_bf16(rng.standard_normal((64, 128)).astype(np.float32))
    out = torch.empty(64, 64, dtype=torch.float32, device="cuda")
    ctx_tiny.linear(a, w, None, 64, 64, 128, out)          # aligned: accepted
    for bad in (dict(a=_shifted(a, 4)), dict(w=_shifted(w, 2)), dict(out=_shifted(out, 1))):
        args = dict(a=a, w=w, out=out)
        args.update(bad)
        with pytest.raises(L.DitError) as e:
            ctx_tiny.linear(args["a"], args["w"], None, 64, 64, 128, args["out"])
        assert e.value.status == L.EINVAL


# --------------------------------------------------------------- unfused q/k/v prep (B arm)

@pytest.mark.parametrize("name", ["tiny", "s1088", "s4608"])
def test_qk_prep_standalone(ctx_big, name):
    """The prep pass on a stored bf16 projection: q and k against the
    oracle's head norm and rotation, vt the exact transpose of the values,
    and the rotation's special tables bit for bit."""
    sh = synth.SHAPES[name]
    S, H = sh.S, sh.heads
    la, _ = arch_pair(sh)
    ctx = ctx_big if name != "tiny" else L.Context(la, max_rows=S)
    rng = np.random.default_rng(S + H)
    qkv = synth.bf16_round(rng.standard_normal((S, 3 * H * 128)).astype(np.float32) * np.float32(2.0))
    qn = synth.bf16_round(1.0 + 0.1 * rng.standard_normal(128).astype(np.float32))
    kn = synth.bf16_round(1.0 + 0.1 * rng.standard_normal(128).astype(np.float32))
    pos = O.positions(sh.L, sh.h, sh.w)
    cs, sn = O.rope_tables(pos, sh.axes)
    Sp = (S + 63) // 64 * 64
    say("qk prep", name, S, H)

    def run(c, s_):
        q = torch.empty((H, S, 128), dtype=torch.bfloat16, device="cuda")
        k = torch.empty_like(q)
        vt = torch.zeros((H, 128, Sp), dtype=torch.bfloat16, device="cuda")
        ctx.qk_prep(L.dev_bf16(qkv), S, L.dev_f32(qn), L.dev_f32(kn), L.dev_f32(c), L.dev_f32(s_), q, k, vt)
        torch.cuda.synchronize()
        return q, k, vt

    q, k, vt = run(cs, sn)
    heads = lambda cols: O.heads_of(cols, H, 128)
    rows = np.arange(S) if S <= 1088 else synth.rows_sample(S, 200)
    qr = O.head_prep(heads(qkv[rows, :H * 128]), qn, 1e-6, cs[rows], sn[rows])
    kr = O.head_prep(heads(qkv[rows, H * 128:2 * H * 128]), kn, 1e-6, cs[rows], sn[rows])
    compare(f"{name}/q", np_of(q)[:, rows], qr, bf16_stored=True)
    compare(f"{name}/k", np_of(k)[:, rows], kr, bf16_stored=True)
    v = heads(qkv[:, 2 * H * 128:])
    assert (np_of(vt)[:, :, :S] == v.transpose(0, 2, 1)).all()
    one, zero = np.ones_like(cs), np.zeros_like(cs)
    bits = lambda t: t.view(torch.int16).cpu().numpy()
    qi, ki, _ = run(one, zero)
    qt, kt, _ = run(zero, one)
    for a, b in ((bits(qi), bits(qt)), (bits(ki), bits(kt))):
        assert (b[..., 0::2] == (a[..., 1::2] ^ np.int16(-0x8000))).all() and (b[..., 1::2] == a[..., 0::2]).all()
    if ctx is not ctx_big:
        ctx.close()


@pytest.mark.parametrize("name", ["tiny", "s1088", "s4608"])
def test_block_unfused_qk_prep(ctx_big, name):
    """The block with the q/k/v prep as a pass of its own (the B arm): its
    intermediates and output against the oracle, and the stage timers show
    which arm ran."""
    case = synth.block_case(name)
    sh = case["shape"]
    la, oa = arch_pair(sh)
    ctx = ctx_big if name == "s4608" else L.Context(la, max_rows=sh.S)
    say("block, unfused qk prep", name)
    ctx.set_qk_prep(False)
    try:
        ctx.timing(True)
        x, _, _ = _block_gpu(ctx, case)
        tm = ctx.timing_read()
        ctx.timing(False)
    finally:
        ctx.set_qk_prep(True)
    assert tm["qk_prep"][1] == 1, "the prep pass did not run"
    got = np_of(x)
    cs, sn, vec = _oracle_inputs(case, oa)
    if sh.S <= 1088:
        inter = _intermediates(ctx, sh, sh.S)
        y, ref = O.block_forward(case["x"], oracle_block(case["block"]), vec, cs, sn, oa, keep=True)
        for kk in ("q", "k", "v", "o", "a"):
            compare(f"{name}/{kk}", inter[kk], ref[kk], bf16_stored=True)
        compare(f"{name}/y", got, y)
        compare(f"{name}/delta", got - case["x"], y - case["x"])
    else:
        rows = synth.rows_sample(sh.S, 48, L=sh.L)
        y, o, x1, a = O.block_forward_rows(case["x"], oracle_block(case["block"]), vec, cs, sn, oa, rows)
        compare(f"{name}/y", got[rows], y)
        compare(f"{name}/delta", got[rows] - case["x"][rows], y - case["x"][rows])
    # the fused arm (the default) runs no prep pass
    ctx.timing(True)
    _block_gpu(ctx, case)
    tm = ctx.timing_read()
    ctx.timing(False)
    assert tm["qk_prep"][1] == 0
    if ctx is not ctx_big:
        ctx.close()


# --------------------------------------------------------------- parallel block

def _parallel_case(name, **kw):
    case = synth.block_case(name, **kw)
    D = case["shape"].hidden
    case["block"]["w_mod"] = np.ascontiguousarray(case["block"]["w_mod"][:3 * D])   # shift, scale, gate
    return case


def _parallel_gpu(ctx, case):
    sh = case["shape"]
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    x = L.dev_f32(case["x"])
    ctx.parallel_block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    torch.cuda.synchronize()
    return x


@pytest.mark.parametrize("name,norm,norm_std", [("tiny", "layer", 0.0), ("tiny", "rms", 0.1),
                                                 ("t_one", "layer", 0.0), ("t_few", "rms", 0.1),
                                                 ("m640", "layer", 0.0), ("w4096", "rms", 0.1),
                                                 ("s1088", "layer", 0.0), ("r1077", "layer", 0.0)])
def test_parallel_block_full_parity(name, norm, norm_std):
    # below the ping-pong sizes: the four-product form
    case = _parallel_case(name, norm_std=norm_std, rms=(norm == "rms"))
    sh = case["shape"]
    la, oa = arch_pair(sh, norm)
    ctx = L.Context(la, max_rows=sh.S)
    say("parallel block", name, norm, "S =", sh.S)
    got = np_of(_parallel_gpu(ctx, case))
    D, F = sh.hidden, sh.ffn
    cs, sn, vec = _oracle_inputs(case, oa)
    y, ref = O.parallel_block_forward(case["x"], oracle_block(case["block"]), vec, cs, sn, oa, keep=True)
    compare(f"{name}/mod", np_of(ctx.debug_copy(0, torch.float32, (3, D))), ref["mod"], rel=1e-4, abs_=1e-4)
    compare(f"{name}/h", np_of(ctx.debug_copy(1, torch.bfloat16, (sh.S, D))), ref["h"], bf16_stored=True)
    compare(f"{name}/o", np_of(ctx.debug_copy(5, torch.bfloat16, (sh.S, D))), ref["o"], bf16_stored=True)
    compare(f"{name}/a", np_of(ctx.debug_copy(7, torch.bfloat16, (sh.S, F))), ref["a"], bf16_stored=True)
    compare(f"{name}/y", got, y)
    compare(f"{name}/delta", got - case["x"], y - case["x"])
    ctx.close()


@pytest.mark.parametrize("name,in_product", BLOCK_FORMS)
def test_parallel_block_full_size_sampled_rows(ctx_big, name, in_product):
    # s4608 runs the two fused products ([QKV | UP] with both epilogues,
    # [OUT | DOWN] over the concatenated rows), with int8 weights on their
    # dequantised copies; int8 weights converted inside the products: the four
    case = _parallel_case(name)
    sh = case["shape"]
    _, oa = arch_pair(sh)
    D, F = sh.hidden, sh.ffn
    say("parallel block", name, "S =", sh.S, "int8 in product" if in_product else "")
    with int8_products(ctx_big, in_product):
        got = np_of(_parallel_gpu(ctx_big, case))
    if in_product:
        o_got = np_of(ctx_big.debug_copy(5, torch.bfloat16, (sh.S, D)))
        a_got = np_of(ctx_big.debug_copy(7, torch.bfloat16, (sh.S, F)))
    else:
        oa_got = np_of(ctx_big.debug_copy(8, torch.bfloat16, (sh.S, D + F)))
        o_got, a_got = oa_got[:, :D], oa_got[:, D:]
    cs, sn, vec = _oracle_inputs(case, oa)
    rows = synth.rows_sample(sh.S, 48, L=sh.L)
    y, o, a = O.parallel_block_forward_rows(case["x"], oracle_block(case["block"]), vec, cs, sn, oa, rows)
    sc = (lambda r: block_abs(r)) if sh.int8 else (lambda r: ABS)
    compare(f"{name}/o", o_got[rows], o, abs_=sc(o), bf16_stored=True)
    compare(f"{name}/a", a_got[rows], a, abs_=sc(a), bf16_stored=True)
    compare(f"{name}/y", got[rows], y, abs_=sc(y))
    d = y - case["x"][rows]
    compare(f"{name}/delta", got[rows] - case["x"][rows], d, abs_=sc(d))


@pytest.mark.parametrize("name", ["tiny", "s4608"])
def test_parallel_block_zero_gate_is_identity(ctx_tiny, ctx_big, name):
    case = _parallel_case(name)
    D = case["shape"].hidden
    case["block"]["w_mod"][2 * D:] = 0.0
    x = _parallel_gpu(ctx_tiny if name == "tiny" else ctx_big, case)
    assert (np_of(x) == case["x"]).all()


# --------------------------------------------------------------- double-stream block

def _double_case(name):
    # the image stream takes the workload's block, the text stream a second
    # draw of the same shapes (another seed)
    case = synth.block_case(name)
    other = synth.block_case(name, seed=case["shape"].seed + 100)
    case["txt_block"] = other["block"]
    return case


def _double_gpu(ctx, case):
    sh = case["shape"]
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    bt = L.BlockWeights.from_host(case["txt_block"])
    bi = L.BlockWeights.from_host(case["block"])
    x = L.dev_f32(case["x"])
    ctx.double_block_forward(bt, bi, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    torch.cuda.synchronize()
    return x


@pytest.mark.parametrize("name,in_product", [("tiny", False), ("t_img", False), ("t_few", False), ("m640", False),
                                             ("w4096", False),
                                             ("s1088", False),
                                             ("r1077", False), ("s4608", False),
                                             ("s4608_int8", False), ("s4608_int8", True)])
def test_double_block_full_parity(ctx_big, name, in_product):
    case = _double_case(name)
    sh = case["shape"]
    la, oa = arch_pair(sh)
    ctx = ctx_big if name.startswith("s4608") else L.Context(la, max_rows=sh.S)
    say("double block", name, "L =", sh.L, "N =", sh.N, "int8 in product" if in_product else "")
    with int8_products(ctx, in_product):
        got = np_of(_double_gpu(ctx, case))
    D, F, H = sh.hidden, sh.ffn, sh.heads
    S, Sp = sh.S, (sh.S + 63) // 64 * 64
    cs, sn, vec = _oracle_inputs(case, oa)
    y, ref = O.double_block_forward(case["x"], oracle_block(case["txt_block"]), oracle_block(case["block"]),
                                    vec, cs, sn, oa, sh.L, keep=True)
    mods = np_of(ctx.debug_copy(0, torch.float32, (12, D)))
    compare(f"{name}/mod-txt", mods[:6], O.modulation(vec, case["txt_block"]["w_mod"], 6), rel=1e-4, abs_=1e-4)
    compare(f"{name}/mod-img", mods[6:], O.modulation(vec, case["block"]["w_mod"], 6), rel=1e-4, abs_=1e-4)
    compare(f"{name}/h", np_of(ctx.debug_copy(1, torch.bfloat16, (S, D))), ref["h"], bf16_stored=True)
    compare(f"{name}/q", np_of(ctx.debug_copy(2, torch.bfloat16, (H, S, 128))), ref["q"], bf16_stored=True)
    compare(f"{name}/k", np_of(ctx.debug_copy(3, torch.bfloat16, (H, S, 128))), ref["k"], bf16_stored=True)
    v = np_of(ctx.debug_copy(4, torch.bfloat16, (H, 128, Sp)))[:, :, :S].transpose(0, 2, 1)
    # int8 weights: tolerance relative to the reference's largest magnitude
    sc = (lambda r: block_abs(r)) if sh.int8 else (lambda r: ABS)
    compare(f"{name}/v", v, ref["v"], abs_=sc(ref["v"]), bf16_stored=True)
    compare(f"{name}/o", np_of(ctx.debug_copy(5, torch.bfloat16, (S, D))), ref["o"], abs_=sc(ref["o"]), bf16_stored=True)
    compare(f"{name}/a", np_of(ctx.debug_copy(7, torch.bfloat16, (S, F))), ref["a"], abs_=sc(ref["a"]), bf16_stored=True)
    compare(f"{name}/y", got, y, abs_=sc(y))
    d = y - case["x"]
    compare(f"{name}/delta", got - case["x"], d, abs_=sc(d))
    if ctx is not ctx_big:
        ctx.close()


def test_double_block_zero_modulation_is_identity(ctx_tiny):
    case = _double_case("tiny")
    case["block"]["w_mod"][:] = 0.0
    case["txt_block"]["w_mod"][:] = 0.0
    assert (np_of(_double_gpu(ctx_tiny, case)) == case["x"]).all()



# --------------------------------------------------------------- modulation runs

def _runs_case(name, R):
    # R conditioning vectors drawn at the time vector's scale (its values
    # have a standard deviation of about 0.13 at hidden 3072)
    case = synth.block_case(name)
    sh = case["shape"]
    case["vecs"] = synth.normal((R, sh.hidden), seed=sh.seed + 200, std=0.13)
    return case


def _runs_gpu(ctx, case, runs, vecs=None):
    sh = case["shape"]
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    x = L.dev_f32(case["x"])
    v = L.dev_f32(case["vecs"] if vecs is None else vecs)
    ctx.block_forward_runs(bw, x, v, runs, seq.cos, seq.sin, sh.L, sh.N)
    torch.cuda.synchronize()
    return x


def _runs_of(name, sh):
    # text rows on one modulation row, the image rows split raggedly over
    # two others (three runs: the OUT/DOWN launches pair two runs, then one)
    if name == "s4608":
        return [(0, sh.L, 1), (sh.L, sh.S, 0)]
    cut = sh.L + (5 if name == "tiny" else 517)
    return [(0, sh.L, 2), (sh.L, cut, 0), (cut, sh.S, 1)]


@pytest.mark.parametrize("name", ["tiny", "s1088"])
def test_block_runs_full_parity(ctx_tiny, name):
    case = _runs_case(name, 3)
    sh = case["shape"]
    la, oa = arch_pair(sh)
    ctx = ctx_tiny if name == "tiny" else L.Context(la, max_rows=sh.S)
    runs = _runs_of(name, sh)
    say("block runs", name, runs)
    got = np_of(_runs_gpu(ctx, case, runs))
    D, F, H = sh.hidden, sh.ffn, sh.heads
    S, Sp = sh.S, (sh.S + 63) // 64 * 64
    cs, sn, _ = _oracle_inputs(case, oa)
    y, ref = O.block_forward_runs(case["x"], oracle_block(case["block"]), case["vecs"], runs, cs, sn, oa, keep=True)
    mods = np_of(ctx.debug_copy(0, torch.float32, (3, 6, D)))
    compare(f"{name}/mods", mods, ref["mods"], rel=1e-4, abs_=1e-4)
    compare(f"{name}/h", np_of(ctx.debug_copy(1, torch.bfloat16, (S, D))), ref["h"], bf16_stored=True)
    compare(f"{name}/q", np_of(ctx.debug_copy(2, torch.bfloat16, (H, S, 128))), ref["q"], bf16_stored=True)
    compare(f"{name}/k", np_of(ctx.debug_copy(3, torch.bfloat16, (H, S, 128))), ref["k"], bf16_stored=True)
    v = np_of(ctx.debug_copy(4, torch.bfloat16, (H, 128, Sp)))[:, :, :S].transpose(0, 2, 1)
    compare(f"{name}/v", v, ref["v"], bf16_stored=True)
    compare(f"{name}/o", np_of(ctx.debug_copy(5, torch.bfloat16, (S, D))), ref["o"], bf16_stored=True)
    compare(f"{name}/h2", np_of(ctx.debug_copy(6, torch.bfloat16, (S, D))), ref["h2"], bf16_stored=True)
    compare(f"{name}/a", np_of(ctx.debug_copy(7, torch.bfloat16, (S, F))), ref["a"], bf16_stored=True)
    compare(f"{name}/y", got, y)
    compare(f"{name}/delta", got - case["x"], y - case["x"])
    if ctx is not ctx_tiny:
        ctx.close()


def test_block_runs_full_size_sampled_rows(ctx_big):
    case = _runs_case("s4608", 2)
    sh = case["shape"]
    _, oa = arch_pair(sh)
    D, F = sh.hidden, sh.ffn
    runs = _runs_of("s4608", sh)
    say("block runs s4608", runs)
    got = np_of(_runs_gpu(ctx_big, case, runs))
    o_got = np_of(ctx_big.debug_copy(5, torch.bfloat16, (sh.S, D)))
    a_got = np_of(ctx_big.debug_copy(7, torch.bfloat16, (sh.S, F)))
    cs, sn, _ = _oracle_inputs(case, oa)
    rows = synth.rows_sample(sh.S, 48, L=sh.L)
    y, o, a = O.block_forward_runs_rows(case["x"], oracle_block(case["block"]), case["vecs"], runs, cs, sn, oa, rows)
    compare("s4608/o", o_got[rows], o, bf16_stored=True)
    compare("s4608/a", a_got[rows], a, bf16_stored=True)
    compare("s4608/y", got[rows], y)
    compare("s4608/delta", got[rows] - case["x"][rows], y - case["x"][rows])


@pytest.mark.parametrize("name", ["tiny", "s4608"])
def test_block_runs_equal_vectors_are_the_block_bit_exact(ctx_tiny, ctx_big, name):
    # every row's arithmetic is the single-vector block's, in the same
    # kernels (the text and image runs of the 4608-row block share one
    # launch of each gated product), so the rows agree to the bit
    case = synth.block_case(name)
    sh = case["shape"]
    ctx = ctx_tiny if name == "tiny" else ctx_big
    ref, seq, _ = _block_gpu(ctx, case)
    vec = np_of(seq.vec).reshape(1, -1)
    runs = [(0, sh.L, 1), (sh.L, sh.S, 0)] if name == "s4608" else [(0, 3, 1), (3, sh.S, 0)]
    say("block runs equal vectors", name, runs)
    got = _runs_gpu(ctx, case, runs, vecs=np.concatenate([vec, vec]))
    assert torch.equal(got, ref)


def test_block_runs_zero_gates_is_identity(ctx_tiny):
    case = _runs_case("tiny", 3)
    D = case["shape"].hidden
    case["block"]["w_mod"][2 * D:3 * D] = 0.0
    case["block"]["w_mod"][5 * D:] = 0.0
    assert (np_of(_runs_gpu(ctx_tiny, case, _runs_of("tiny", case["shape"]))) == case["x"]).all()


def test_block_runs_rejects_bad_runs(ctx_tiny):
    case = _runs_case("tiny", 2)
    sh = case["shape"]
    for runs in ([(0, 3, 0), (4, sh.S, 1)], [(0, 3, 0), (3, sh.S, 2)], [(0, 3, 0)], [(1, sh.S, 0)],
                 [(0, 0, 0), (0, sh.S, 1)]):
        with pytest.raises(RuntimeError):
            _runs_gpu(ctx_tiny, case, runs)


# --------------------------------------------------------------- sandwich norms

@pytest.mark.parametrize("name,norm,norm_std", [("tiny", "layer", 0.0), ("tiny", "rms", 0.1),
                                                 ("s1088", "layer", 0.0), ("s1088", "rms", 0.1),
                                                 ("t_few", "layer", 0.0), ("r1077", "rms", 0.1)])
def test_sandwich_block_full_parity(name, norm, norm_std):
    case = synth.block_case(name, norm_std=norm_std, rms=(norm == "rms"), sandwich=True)
    sh = case["shape"]
    la, oa = arch_pair(sh, norm)
    ctx = L.Context(la, max_rows=sh.S)
    say("sandwich block", name, norm, "S =", sh.S)
    x, _, _ = _block_gpu(ctx, case, norm)
    got = np_of(x)
    inter = _intermediates(ctx, sh, sh.S)
    cs, sn, vec = _oracle_inputs(case, oa)
    y, ref = O.block_forward(case["x"], oracle_block(case["block"]), vec, cs, sn, oa, keep=True)
    for k in ("h", "o", "h2", "a"):   # h2 follows the attention half's post norm
        compare(f"{name}/{k}", inter[k], ref[k], bf16_stored=True)
    compare(f"{name}/y", got, y)
    compare(f"{name}/delta", got - case["x"], y - case["x"])
    ctx.close()


@pytest.mark.parametrize("name,in_product", BLOCK_FORMS)
def test_sandwich_block_full_size_sampled_rows(ctx_big, name, in_product):
    case = synth.block_case(name, sandwich=True)
    sh = case["shape"]
    _, oa = arch_pair(sh)
    say("sandwich block", name, "S =", sh.S, "int8 in product" if in_product else "")
    with int8_products(ctx_big, in_product):
        x, _, _ = _block_gpu(ctx_big, case)
    got = np_of(x)
    inter = _intermediates(ctx_big, sh, sh.S)
    cs, sn, vec = _oracle_inputs(case, oa)
    rows = synth.rows_sample(sh.S, 48, L=sh.L)
    y, o, x1, a = O.block_forward_rows(case["x"], oracle_block(case["block"]), vec, cs, sn, oa, rows)
    # int8 weights: tolerance relative to the reference's largest magnitude
    sc = (lambda r: block_abs(r)) if sh.int8 else (lambda r: ABS)
    compare(f"{name}/o", inter["o"][rows], o, abs_=sc(o), bf16_stored=True)
    compare(f"{name}/a", inter["a"][rows], a, abs_=sc(a), bf16_stored=True)
    compare(f"{name}/y", got[rows], y, abs_=sc(y))
    d = y - case["x"][rows]
    compare(f"{name}/delta", got[rows] - case["x"][rows], d, abs_=sc(d))


def test_sandwich_block_runs_parity(ctx_tiny):
    case = synth.block_case("tiny", sandwich=True)
    sh = case["shape"]
    case["vecs"] = synth.normal((3, sh.hidden), seed=sh.seed + 200, std=0.13)
    _, oa = arch_pair(sh)
    runs = _runs_of("tiny", sh)
    say("sandwich block runs", runs)
    got = np_of(_runs_gpu(ctx_tiny, case, runs))
    cs, sn, _ = _oracle_inputs(case, oa)
    y = O.block_forward_runs(case["x"], oracle_block(case["block"]), case["vecs"], runs, cs, sn, oa)
    compare("tiny/y", got, y)
    compare("tiny/delta", got - case["x"], y - case["x"])


def test_sandwich_block_zero_gates_is_identity(ctx_tiny):
    case = synth.block_case("tiny", sandwich=True)
    D = case["shape"].hidden
    case["block"]["w_mod"][2 * D:3 * D] = 0.0
    case["block"]["w_mod"][5 * D:] = 0.0
    x, _, _ = _block_gpu(ctx_tiny, case)
    assert (np_of(x) == case["x"]).all()


def test_sandwich_weights_rejected_where_not_taken(ctx_tiny):
    case = synth.block_case("tiny", sandwich=True)
    sh = case["shape"]
    seq = GpuSeq(ctx_tiny, sh, case["t"], case["w_t1"], case["w_t2"])
    x = L.dev_f32(case["x"])
    one = dict(case["block"])
    del one["post_mlp"]
    with pytest.raises(L.DitError) as e:
        ctx_tiny.block_forward(L.BlockWeights.from_host(one), x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    assert e.value.status == L.EINVAL
    bw = L.BlockWeights.from_host(case["block"])
    with pytest.raises(L.DitError) as e:
        ctx_tiny.double_block_forward(bw, bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    assert e.value.status == L.EINVAL
    pb = dict(case["block"])
    pb["w_mod"] = np.ascontiguousarray(pb["w_mod"][:3 * sh.hidden])
    with pytest.raises(L.DitError) as e:
        ctx_tiny.parallel_block_forward(L.BlockWeights.from_host(pb), x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    assert e.value.status == L.EINVAL
    torch.cuda.synchronize()
    assert (np_of(x) == case["x"]).all()


# --------------------------------------------------------------- W8A8

def _bf16_rows(rows, K, seed):
    # rows at spreads from 1e-3 to 1e3, a zero row and a row of one value
    x = synth.normal((rows, K), seed=seed) * np.float32(10.0) ** np.linspace(-3, 3, rows, dtype=np.float32)[:, None]
    x[1] = 0.0
    x[2] = 0.75
    return synth.bf16_round(x)


@pytest.mark.parametrize("rows,K", [(5, 8), (72, 256), (300, 3072), (4608, 12288), (3, 16384)])
def test_quantize_rows_bit_exact(ctx_tiny, rows, K):
    x = _bf16_rows(rows, K, seed=rows + K)
    q = torch.empty((rows, K), dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    say("quantize rows", rows, K)
    ctx_tiny.quantize_rows(L.dev_bf16(x), rows, K, q, s)
    torch.cuda.synchronize()
    qr, sr = O.quantize_rows_int8(x)
    assert (np_of(s) == sr).all()
    assert (np_of(q) == qr).all()


@pytest.mark.parametrize("rows,K", [(5, 256), (72, 768), (300, 3072), (4608, 12288), (3, 16384)])
def test_convrot_quantize_rows(ctx_tiny, rows, K):
    """ConvRot then INT8 rows: the GPU rotates in fp32 butterflies, the oracle
    takes the plain product with the Hadamard matrix in float64 and rounds it
    once to fp32, so a code may sit one step away where the two roundings
    straddle a half step.  Every GPU code must still be a nearest code of the
    exact rotated value (within its half step and the rotation's rounding),
    and such one-step codes must be rare."""
    x = _bf16_rows(rows, K, seed=rows + K + 7)
    q = torch.empty((rows, K), dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    say("convrot quantize rows", rows, K)
    ctx_tiny.convrot_quantize_rows(L.dev_bf16(x), rows, K, q, s)
    torch.cuda.synchronize()
    y = O.convrot(x)
    qr, sr = O.quantize_rows_int8(y.astype(np.float32))
    qg, sg = np_of(q).astype(np.int64), np_of(s).astype(np.float64)
    amax = np.abs(y).max(axis=1)
    assert np.all(np.abs(sg - sr) <= 1e-6 * sr + 1e-30)
    assert (sg[1] == 0.0) and (qg[1] == 0).all()                                    # zero row
    d = np.abs(qg - qr.astype(np.int64))
    assert d.max() <= 1 and d.sum() <= max(2, 1e-3 * d.size), f"{int(d.sum())} codes differ by one"
    err = np.abs(qg * sg[:, None] - y)
    assert np.all(err <= sg[:, None] * (0.5 + 1e-3) + amax[:, None] * 1e-6)
    # a constant row rotates exactly: each group's first value is 16x it
    assert (qg[2].reshape(-1, 256)[:, 0] == 127).all() and (qg[2].reshape(-1, 256)[:, 1:] == 0).all()


@pytest.mark.parametrize("norm", ["layer", "rms"])
@pytest.mark.parametrize("rows", [72, 4608])
def test_modulated_norm_int8(norm, rows):
    # the codes are taken from the fp32 norm output, which the oracle holds
    # in float64: the integer decisions agree except where the two values
    # straddle a rounding boundary, and there by one step
    D = 3072
    sh = synth.Shape("n", D, D // 128, 128, 1024, 0, 1, rows, seed=0)
    la, oa = arch_pair(sh, norm)
    ctx = L.Context(la, max_rows=rows)
    x = synth.normal((rows, D), seed=rows + 7, std=2.0, mean=0.5)
    shift = synth.normal((D,), seed=1, std=0.3)
    scale = synth.normal((D,), seed=2, std=0.3)
    nw = synth.normal((D,), seed=3, std=0.1, mean=1.0)
    q = torch.empty((rows, D), dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    say("modulated norm int8", norm, rows)
    ctx.modulated_norm_int8(L.dev_f32(x), rows, L.dev_f32(shift), L.dev_f32(scale), L.dev_f32(nw), 1e-6, q, s)
    torch.cuda.synchronize()
    ref = O.modulated_norm(x, shift, scale, oa, nw)
    qr, sr = O.quantize_rows_int8(ref)
    d = np_of(q).astype(int) - qr.astype(int)
    say(f"codes off by one: {np.count_nonzero(d)} of {d.size}")
    assert np.abs(d).max() <= 1 and np.count_nonzero(d) <= d.size * 1e-3
    assert np.allclose(np_of(s), sr, rtol=1e-5, atol=0)
    ctx.close()


@pytest.mark.parametrize("M,N,K", [(72, 256, 128), (300, 768, 256), (4608, 3072, 3072), (4608, 24576, 3072),
                                   (4608, 3072, 12288), (1, 256, 12288)])
def test_linear_w8a8(ctx_big, M, N, K):
    # exact int32 sums times two fp32 scales: three fp32 roundings
    rng = np.random.default_rng(M + N + K)
    a = rng.integers(-127, 128, (M, K), dtype=np.int8)
    w = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sa = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("linear w8a8", M, N, K)
    ctx_big.linear_w8a8(torch.from_numpy(a).cuda(), L.dev_f32(sa), torch.from_numpy(w).cuda(), L.dev_f32(sw),
                        M, N, K, out)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 300 else synth.rows_sample(M, 48)
    # int8 products summed over K <= 12288 stay below 2^53: float64 is exact
    ref = (a[rows].astype(np.float64) @ w.astype(np.float64).T) * sa[rows, None].astype(np.float64) * sw[None, :]
    got = np_of(out)[rows].astype(np.float64)
    assert np.all(np.abs(got - ref) <= 3e-7 * np.abs(ref) + 1e-30)


def _w8a8_gpu(ctx, case, runs=None, rotated=False):
    sh = case["shape"]
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"], rotated=rotated)
    x = L.dev_f32(case["x"])
    if runs is None:
        ctx.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    else:
        ctx.block_forward_runs(bw, x, L.dev_f32(case["vecs"]), runs, seq.cos, seq.sin, sh.L, sh.N)
    torch.cuda.synchronize()
    return x


@pytest.mark.parametrize("name,norm,norm_std,sandwich,rot", [("tiny", "layer", 0.0, False, False),
                                                              ("tiny", "rms", 0.1, False, False),
                                                              ("tiny", "layer", 0.0, True, False),
                                                              ("s1088", "layer", 0.0, False, False),
                                                              ("tiny", "layer", 0.0, False, True),
                                                              ("tiny", "rms", 0.1, True, True),
                                                              ("t_one", "layer", 0.0, False, False),
                                                              ("t_few", "rms", 0.1, True, True),
                                                              ("m640", "layer", 0.0, False, True),
                                                              ("w4096", "rms", 0.1, True, True),
                                                              ("s1088", "layer", 0.0, False, True),
                                                              ("r1077", "rms", 0.1, False, True)])
def test_w8a8_block_full_parity(name, norm, norm_std, sandwich, rot):
    case = synth.block_case(name, norm_std=norm_std, rms=(norm == "rms"), sandwich=sandwich, w8a8=True)
    sh = case["shape"]
    la, oa = arch_pair(sh, norm)
    ctx = L.Context(la, max_rows=sh.S)
    say("w8a8 block", name, norm, "sandwich" if sandwich else "", "convrot" if rot else "", "S =", sh.S)
    got = np_of(_w8a8_gpu(ctx, case, rotated=rot))
    D, F, H = sh.hidden, sh.ffn, sh.heads
    S, Sp = sh.S, (sh.S + 63) // 64 * 64
    cs, sn, vec = _oracle_inputs(case, oa)
    y, ref = O.block_forward(case["x"], oracle_block(case["block"], rotated=rot), vec, cs, sn, oa, keep=True)
    compare(f"{name}/q", np_of(ctx.debug_copy(2, torch.bfloat16, (H, S, 128))), ref["q"], bf16_stored=True)
    compare(f"{name}/k", np_of(ctx.debug_copy(3, torch.bfloat16, (H, S, 128))), ref["k"], bf16_stored=True)
    v = np_of(ctx.debug_copy(4, torch.bfloat16, (H, 128, Sp)))[:, :, :S].transpose(0, 2, 1)
    compare(f"{name}/v", v, ref["v"], bf16_stored=True)
    compare(f"{name}/o", np_of(ctx.debug_copy(5, torch.bfloat16, (S, D))), ref["o"], bf16_stored=True)
    compare(f"{name}/a", np_of(ctx.debug_copy(7, torch.bfloat16, (S, F))), ref["a"], bf16_stored=True)
    compare(f"{name}/y", got, y)
    compare(f"{name}/delta", got - case["x"], y - case["x"])
    ctx.close()


@pytest.mark.parametrize("rot", [False, True])
def test_w8a8_block_full_size_sampled_rows(ctx_big, rot):
    case = synth.block_case("s4608_w8a8")
    sh = case["shape"]
    _, oa = arch_pair(sh)
    D, F = sh.hidden, sh.ffn
    say("w8a8 block s4608", "convrot" if rot else "")
    got = np_of(_w8a8_gpu(ctx_big, case, rotated=rot))
    o_got = np_of(ctx_big.debug_copy(5, torch.bfloat16, (sh.S, D)))
    a_got = np_of(ctx_big.debug_copy(7, torch.bfloat16, (sh.S, F)))
    cs, sn, vec = _oracle_inputs(case, oa)
    rows = synth.rows_sample(sh.S, 48, L=sh.L)
    y, o, x1, a = O.block_forward_rows(case["x"], oracle_block(case["block"], rotated=rot), vec, cs, sn, oa, rows)
    compare("s4608_w8a8/o", o_got[rows], o, bf16_stored=True)
    compare("s4608_w8a8/a", a_got[rows], a, bf16_stored=True)
    compare("s4608_w8a8/y", got[rows], y)
    compare("s4608_w8a8/delta", got[rows] - case["x"][rows], y - case["x"][rows])


def test_w8a8_block_runs_parity(ctx_tiny):
    case = synth.block_case("tiny", w8a8=True)
    sh = case["shape"]
    case["vecs"] = synth.normal((3, sh.hidden), seed=sh.seed + 200, std=0.13)
    _, oa = arch_pair(sh)
    runs = _runs_of("tiny", sh)
    say("w8a8 block runs", runs)
    got = np_of(_w8a8_gpu(ctx_tiny, case, runs))
    cs, sn, _ = _oracle_inputs(case, oa)
    y = O.block_forward_runs(case["x"], oracle_block(case["block"]), case["vecs"], runs, cs, sn, oa)
    compare("tiny/y", got, y)
    compare("tiny/delta", got - case["x"], y - case["x"])


def test_w8a8_weights_rejected_where_not_taken(ctx_tiny):
    case = synth.block_case("tiny", w8a8=True)
    sh = case["shape"]
    seq = GpuSeq(ctx_tiny, sh, case["t"], case["w_t1"], case["w_t2"])
    x = L.dev_f32(case["x"])
    bw = L.BlockWeights.from_host(case["block"])
    with pytest.raises(L.DitError) as e:
        ctx_tiny.double_block_forward(bw, bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    assert e.value.status == L.EINVAL
    pb = dict(case["block"])
    pb["w_mod"] = np.ascontiguousarray(pb["w_mod"][:3 * sh.hidden])
    with pytest.raises(L.DitError) as e:
        ctx_tiny.parallel_block_forward(L.BlockWeights.from_host(pb), x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    assert e.value.status == L.EINVAL


def test_w8a8_wide_ffn_rejected_before_device_work():
    # the SwiGLU rows of a W8A8 block are quantized a row per workgroup, up
    # to 16384 wide: a wider ffn is refused before anything is enqueued, so
    # x is never left half-updated
    sh = synth.Shape("wide", 256, 2, 128, 16640, 8, 4, 4, seed=9, w8a8=True)
    la, _ = arch_pair(sh)
    ctx = L.Context(la, max_rows=64)
    rng = np.random.default_rng(9)
    bw = L.BlockWeights.from_host(synth.block_weights(rng, sh))
    x0 = synth.normal((sh.S, sh.hidden), seed=9)
    x = L.dev_f32(x0)
    seq = GpuSeq(ctx, sh, 0.5, synth.normal((sh.hidden, 256), 1, 0.02), synth.normal((sh.hidden, sh.hidden), 2, 0.02))
    with pytest.raises(L.DitError) as e:
        ctx.block_forward(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    assert e.value.status == L.EUNSUPPORTED
    torch.cuda.synchronize()
    assert (np_of(x) == x0).all()
    ctx.close()



# --------------------------------------------------------------- reference rows (RefSlot)

def _ref_first(name, sh):
    # the reference: the last rows of the image (24, 300 or 1024 of them)
    return sh.S - {"tiny": 24, "s1088": 300, "s4608": 1024}[name]


@pytest.mark.parametrize("name", ["tiny", "s1088"])
def test_cached_block_parity(ctx_tiny, name):
    case = synth.block_case(name)
    sh = case["shape"]
    la, oa = arch_pair(sh)
    ctx = ctx_tiny if name == "tiny" else L.Context(la, max_rows=sh.S)
    first, H, D = _ref_first(name, sh), sh.heads, sh.hidden
    count = sh.S - first
    say("cached block", name, "first =", first)
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    slot = torch.empty(2 * H * count * 128, dtype=torch.bfloat16, device="cuda")
    # recording step: the whole block, then the reference rows' k and v
    x0 = L.dev_f32(case["x"])
    ctx.block_forward_cached(bw, x0, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, True)
    torch.cuda.synchronize()
    cs, sn, vec = _oracle_inputs(case, oa)
    ob = oracle_block(case["block"])
    compare(f"{name}/record y", np_of(x0), O.block_forward(case["x"], ob, vec, cs, sn, oa))
    k_ref, v_ref = O.reference_kv(case["x"], ob, vec, cs, sn, oa, first)
    sl = np_of(slot)
    compare(f"{name}/slot k", sl[:H * count * 128].reshape(H, count, 128), k_ref, bf16_stored=True)
    compare(f"{name}/slot v", sl[H * count * 128:].reshape(H, 128, count).transpose(0, 2, 1), v_ref, bf16_stored=True)
    # a later step: new values in the updated rows, the reference rows as they were
    x1h = case["x"].copy()
    x1h[:first] = synth.normal((first, D), seed=sh.seed + 400)
    x1 = L.dev_f32(x1h)
    ctx.block_forward_cached(bw, x1, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, False)
    torch.cuda.synchronize()
    got = np_of(x1)
    y = O.block_forward_cached(x1h, ob, vec, cs, sn, oa, first, k_ref, v_ref)
    assert (got[first:] == x1h[first:]).all()
    compare(f"{name}/step y", got[:first], y[:first])
    compare(f"{name}/step delta", got[:first] - x1h[:first], y[:first] - x1h[:first])
    if ctx is not ctx_tiny:
        ctx.close()


def test_cached_block_step_on_the_recorded_rows_is_the_block_bit_exact(ctx_big):
    # the same rows after the recording step: the first rows' arithmetic is
    # the whole block's in the same kernels, with the keys and values of the
    # reference rows put back bit for bit
    case = synth.block_case("s4608")
    sh = case["shape"]
    first, H = _ref_first("s4608", sh), sh.heads
    count = sh.S - first
    say("cached block s4608 first =", first)
    seq = GpuSeq(ctx_big, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    slot = torch.empty(2 * H * count * 128, dtype=torch.bfloat16, device="cuda")
    x0 = L.dev_f32(case["x"])
    ctx_big.block_forward_cached(bw, x0, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, True)
    x1 = L.dev_f32(case["x"])
    ctx_big.block_forward_cached(bw, x1, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, False)
    ref = L.dev_f32(case["x"])
    ctx_big.block_forward(bw, ref, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    torch.cuda.synchronize()
    assert torch.equal(x0, ref)
    assert torch.equal(x1[:first], ref[:first])
    assert torch.equal(x1[first:], L.dev_f32(case["x"])[first:])


def test_cached_block_rejects_bad_arguments(ctx_tiny):
    case = synth.block_case("tiny")
    sh = case["shape"]
    seq = GpuSeq(ctx_tiny, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    x = L.dev_f32(case["x"])
    for first, slot in ((0, None), (sh.S + 1, None), (sh.S - 4, None)):
        with pytest.raises(L.DitError):
            ctx_tiny.block_forward_cached(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, False)
    # no reference rows: no slot needed, and the step is the block
    ref = L.dev_f32(case["x"])
    ctx_tiny.block_forward(bw, ref, seq.vec, seq.cos, seq.sin, sh.L, sh.N)
    ctx_tiny.block_forward_cached(bw, x, seq.vec, seq.cos, seq.sin, sh.L, sh.N, sh.S, None, False)
    torch.cuda.synchronize()
    assert torch.equal(x, ref)


def test_block_runs_single_row_runs(ctx_tiny):
    # runs of one row at the start, in the middle and at the end
    case = _runs_case("tiny", 3)
    sh = case["shape"]
    _, oa = arch_pair(sh)
    runs = [(0, 1, 1), (1, 2, 0), (2, 40, 2), (40, 41, 1), (41, sh.S - 1, 0), (sh.S - 1, sh.S, 2)]
    say("block runs", runs)
    got = np_of(_runs_gpu(ctx_tiny, case, runs))
    cs, sn, _ = _oracle_inputs(case, oa)
    y = O.block_forward_runs(case["x"], oracle_block(case["block"]), case["vecs"], runs, cs, sn, oa)
    compare("tiny/y", got, y)
    compare("tiny/delta", got - case["x"], y - case["x"])


@pytest.mark.parametrize("first", [1, 71])
def test_cached_block_one_active_or_one_cached_row(ctx_tiny, first):
    case = synth.block_case("tiny")
    sh = case["shape"]
    _, oa = arch_pair(sh)
    H, count = sh.heads, sh.S - first
    say("cached block tiny first =", first)
    seq = GpuSeq(ctx_tiny, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    slot = torch.empty(2 * H * count * 128, dtype=torch.bfloat16, device="cuda")
    x0 = L.dev_f32(case["x"])
    ctx_tiny.block_forward_cached(bw, x0, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, True)
    x1h = case["x"].copy()
    x1h[:first] = synth.normal((first, sh.hidden), seed=sh.seed + 401)
    x1 = L.dev_f32(x1h)
    ctx_tiny.block_forward_cached(bw, x1, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, False)
    torch.cuda.synchronize()
    cs, sn, vec = _oracle_inputs(case, oa)
    ob = oracle_block(case["block"])
    k_ref, v_ref = O.reference_kv(case["x"], ob, vec, cs, sn, oa, first)
    y = O.block_forward_cached(x1h, ob, vec, cs, sn, oa, first, k_ref, v_ref)
    got = np_of(x1)
    assert (got[first:] == x1h[first:]).all()
    compare("tiny/step y", got[:first], y[:first])
    compare("tiny/step delta", got[:first] - x1h[:first], y[:first] - x1h[:first])


def test_denoise_step_full_size():
    """At the 1024-px DiT's sizes (L=512, N=4096, hidden 3072, two blocks)
    one denoise step equals the same step put together from the library's
    single-step entry points (time vector, text rows and image-in product,
    the blocks, final modulation, norm and product, Euler update), bit for
    bit; and its velocity and updated latent match the oracle's."""
    m = synth.model_case("dit32", blocks=2)
    sh = m["shape"]
    la, _ = arch_pair(sh)
    ctx = L.Context(la, max_rows=sh.S)
    D, lat, S = sh.hidden, sh.latent, sh.S
    say("denoise step parts, S =", S)
    mw = L.ModelWeights.from_host(m["top"], m["blocks"])
    top = mw.top
    pos = torch.empty((S, 3), dtype=torch.int32, device="cuda")
    ctx.positions(sh.L, sh.h, sh.w, pos)
    cs = torch.empty((S, 64), dtype=torch.float32, device="cuda")
    sn = torch.empty_like(cs)
    ctx.rope_tables(pos, S, cs, sn)
    txt = torch.empty((sh.L, D), dtype=torch.float32, device="cuda")
    ctx.prologue(mw, L.dev_f32(m["ctx"]), sh.L, txt)
    sigma, sigma_next = 0.75, 0.5
    x = L.dev_f32(m["x_lat"])
    v = torch.empty((sh.N, lat), dtype=torch.float32, device="cuda")
    ctx.denoise_step(mw, x, txt, cs, sn, sh.L, sh.N, sigma, sigma_next, v)
    # the same step from its parts
    vec = torch.empty(D, dtype=torch.float32, device="cuda")
    t_in = float(O.sigma_schedule([sigma])[1][0])       # ([HC] s.6) (sigma * 1000) / 1000
    ctx.time_vector(top["w_t1"], top["w_t2"], t_in, vec)
    seq = torch.empty((S, D), dtype=torch.float32, device="cuda")
    seq[:sh.L] = txt
    ctx.linear(L.dev_f32(m["x_lat"]).to(torch.bfloat16), top["w_in"], None, sh.N, D, lat, seq[sh.L:])
    for b in mw.blocks:
        ctx.block_forward(b, seq, vec, cs, sn, sh.L, sh.N)
    fmod = torch.empty(2 * D, dtype=torch.float32, device="cuda")
    ctx.modulation(top["w_fmod"], 2, vec, fmod)
    h = torch.empty((sh.N, D), dtype=torch.bfloat16, device="cuda")
    ctx.modulated_norm(seq[sh.L:], sh.N, fmod[:D], fmod[D:], None, la.final_eps, h)
    v2 = torch.empty((sh.N, lat), dtype=torch.float32, device="cuda")
    ctx.linear(h, top["w_final"], None, sh.N, lat, D, v2)
    x2 = L.dev_f32(m["x_lat"])
    ctx.euler_step(x2, v2, sh.N * lat, sigma, sigma_next)
    torch.cuda.synchronize()
    assert torch.equal(v, v2)
    assert torch.equal(x, x2)
    # and the velocity and the updated latent against the oracle (float64,
    # the same two blocks on the host)
    say("denoise step vs oracle velocity, S =", S)
    ow = O.ModelWeights(**m["top"], blocks=[oracle_block(b) for b in m["blocks"]])
    _, oa = arch_pair(sh)
    opos = O.positions(sh.L, sh.h, sh.w)
    ocs, osn = O.rope_tables(opos, sh.axes)
    txt_ref = O.text_rows(m["ctx"], ow)
    compare("txt", np_of(txt), txt_ref)
    vref = O.velocity(m["x_lat"], txt_ref, ow, ocs, osn, t_in, oa)
    compare("vel", np_of(v), vref)
    xref = O.euler_step(m["x_lat"], vref.astype(np.float32), sigma, sigma_next)
    compare("x_next", np_of(x), xref)
    ctx.close()


@pytest.mark.parametrize("norm", ["layer", "rms"])
def test_cached_w8a8_sandwich_block(norm):
    # the cached step, W8A8 weights and sandwich norms together, at 512 px
    case = synth.block_case("s1088", norm_std=0.1 if norm == "rms" else 0.0, rms=(norm == "rms"), sandwich=True,
                            w8a8=True)
    sh = case["shape"]
    la, oa = arch_pair(sh, norm)
    ctx = L.Context(la, max_rows=sh.S)
    first, H, D = _ref_first("s1088", sh), sh.heads, sh.hidden
    count = sh.S - first
    say("cached w8a8 sandwich block", norm, "first =", first)
    seq = GpuSeq(ctx, sh, case["t"], case["w_t1"], case["w_t2"])
    bw = L.BlockWeights.from_host(case["block"])
    slot = torch.empty(2 * H * count * 128, dtype=torch.bfloat16, device="cuda")
    x0 = L.dev_f32(case["x"])
    ctx.block_forward_cached(bw, x0, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, True)
    x1h = case["x"].copy()
    x1h[:first] = synth.normal((first, D), seed=sh.seed + 402)
    x1 = L.dev_f32(x1h)
    ctx.block_forward_cached(bw, x1, seq.vec, seq.cos, seq.sin, sh.L, sh.N, first, slot, False)
    torch.cuda.synchronize()
    cs, sn, vec = _oracle_inputs(case, oa)
    ob = oracle_block(case["block"])
    y0, ref0 = O.block_forward(case["x"], ob, vec, cs, sn, oa, keep=True)
    compare("record y", np_of(x0), y0)
    k_ref, v_ref = ref0["k"][:, first:], ref0["v"][:, first:]      # what reference_kv returns
    y = O.block_forward_cached(x1h, ob, vec, cs, sn, oa, first, k_ref, v_ref)
    got = np_of(x1)
    assert (got[first:] == x1h[first:]).all()
    compare("step y", got[:first], y[:first])
    compare("step delta", got[:first] - x1h[:first], y[:first] - x1h[:first])
    ctx.close()

# --------------------------------------------------------------- sampler grid

@pytest.mark.parametrize("shift", [1.0, 3.0, 0.37])
def test_sigma_schedule_bit_exact(shift):
    # host code of the library: every step one rounded fp32 operation, as
    # the oracle's float32 NumPy steps
    given = [1.0, 0.978453, 0.95418, 0.926626, 0.89508, 0.845148, 0.704534, 0.414568]
    grid = np.concatenate([np.array(given, np.float32), np.linspace(0.9, 0.01, 37, dtype=np.float32)])
    sig, t = L.sigma_schedule(grid, shift)
    rs, rt = O.sigma_schedule(grid, shift)
    assert (sig.view(np.uint32) == rs.view(np.uint32)).all()
    assert (t.view(np.uint32) == rt.view(np.uint32)).all()
    with pytest.raises(L.DitError):
        L.sigma_schedule([1.0, 1.5], shift)
    with pytest.raises(L.DitError):
        L.sigma_schedule(grid, 0.0)

# --------------------------------------------------------------- denoise

def _twin_setup(m):
    sh = m["shape"]
    la, _ = arch_pair(sh)
    ctx = L.Context(la, max_rows=sh.S)
    mw = L.ModelWeights.from_host(m["top"], m["blocks"])
    pos = torch.empty((sh.S, 3), dtype=torch.int32, device="cuda")
    ctx.positions(sh.L, sh.h, sh.w, pos)
    cs = torch.empty((sh.S, 64), dtype=torch.float32, device="cuda")
    sn = torch.empty_like(cs)
    ctx.rope_tables(pos, sh.S, cs, sn)
    txt = torch.empty((sh.L, sh.hidden), dtype=torch.float32, device="cuda")
    if sh.L > 0:
        ctx.prologue(mw, L.dev_f32(m["ctx"]), sh.L, txt)
    return ctx, mw, cs, sn, txt


def _run_steps(ctx, mw, m, cs, sn, txt, sig, steps):
    sh = m["shape"]
    x = L.dev_f32(m["x_lat"])
    vels = []
    for i in steps:
        v = torch.empty((sh.N, sh.latent), dtype=torch.float32, device="cuda")
        ctx.denoise_step(mw, x, txt, cs, sn, sh.L, sh.N, float(sig[i]), float(sig[i + 1]), v)
        vels.append(v)
    torch.cuda.synchronize()
    return x, vels


@pytest.mark.parametrize("name,kw", [("twin", dict(blocks=3, hidden=256, heads=2, ffn=1024, L=8, h=8, w=8,
                                                   text_dim=256)),
                                     ("twin_w8a8", dict(blocks=2, hidden=256, heads=2, ffn=1024, L=8, h=8, w=8,
                                                        text_dim=256, w8a8=True)),
                                     ("wide", dict(blocks=2, hidden=4096, heads=32, ffn=16384, L=8, h=8, w=8,
                                                   text_dim=256)),
                                     ("full", dict(blocks=2))])
def test_planned_schedule_is_the_loop_bit_exact(name, kw):
    """Steps whose modulation rows come from dit_plan_schedule (each
    modulation weight read once for all four steps) equal the unplanned
    steps bit for bit: the whole 4-step loop on a small model, and at the
    1024-px DiT's sizes (two blocks); a plan of the first two sigmas only
    (the other steps compute their own); a plan made for another model's
    weights is not used."""
    m = synth.model_case("dit32", **kw)
    sh = m["shape"]
    ctx, mw, cs, sn, txt = _twin_setup(m)
    say("planned schedule", name, "S =", sh.S)
    sig = O.sigma_grid(4)
    steps = range(4) if name != "full" else range(2)
    x0, v0 = _run_steps(ctx, mw, m, cs, sn, txt, sig, steps)
    ctx.plan_schedule(mw, sig[:4])
    x1, v1 = _run_steps(ctx, mw, m, cs, sn, txt, sig, steps)
    for a, b in zip(v0, v1):
        assert torch.equal(a, b)
    assert torch.equal(x0, x1)
    ctx.plan_schedule(mw, sig[:2])
    x2, v2 = _run_steps(ctx, mw, m, cs, sn, txt, sig, steps)
    for a, b in zip(v0, v2):
        assert torch.equal(a, b)
    assert torch.equal(x0, x2)
    if name == "twin":
        # another model's weights: its steps ignore this plan
        m2 = synth.model_case("dit32", seed=77, **kw)
        mw2 = L.ModelWeights.from_host(m2["top"], m2["blocks"])
        txt2 = torch.empty_like(txt)
        ctx.prologue(mw2, L.dev_f32(m2["ctx"]), sh.L, txt2)
        ctx.plan_schedule(mw2, [])
        xa, va = _run_steps(ctx, mw2, m2, cs, sn, txt2, sig, steps)
        ctx.plan_schedule(mw, sig[:4])
        xb, vb = _run_steps(ctx, mw2, m2, cs, sn, txt2, sig, steps)
        for a, b in zip(va, vb):
            assert torch.equal(a, b)
        assert torch.equal(xa, xb)
        assert not torch.equal(xa, x0)
    ctx.close()


@pytest.mark.parametrize("steps", [3, 5, 8])
def test_planned_schedule_of_other_lengths(steps):
    """Plans of three steps (the three-vector GEMV) and of more than four
    (the four-vector GEMV in chunks: 4 + 1, 4 + 4) give every step the
    unplanned rows bit for bit."""
    m = synth.model_case("dit32", blocks=2, hidden=256, heads=2, ffn=1024, L=8, h=8, w=8, text_dim=256)
    ctx, mw, cs, sn, txt = _twin_setup(m)
    say("planned schedule of", steps, "steps")
    sig = O.sigma_grid(steps)
    x0, v0 = _run_steps(ctx, mw, m, cs, sn, txt, sig, range(steps))
    ctx.plan_schedule(mw, sig[:steps])
    x1, v1 = _run_steps(ctx, mw, m, cs, sn, txt, sig, range(steps))
    for a, b in zip(v0, v1):
        assert torch.equal(a, b)
    assert torch.equal(x0, x1)
    ctx.close()


def test_planned_schedule_rejects_bad_arguments(ctx_tiny):
    m = synth.model_case("dit32", blocks=1, hidden=256, heads=2, ffn=1024, L=8, h=8, w=8, text_dim=256)
    mw = L.ModelWeights.from_host(m["top"], m["blocks"])
    with pytest.raises(L.DitError) as e:
        ctx_tiny.plan_schedule(mw, np.linspace(1, 0, 65))
    assert e.value.status == L.ERANGE
    with pytest.raises(L.DitError) as e:
        ctx_tiny.plan_schedule(mw, [1.0, float("nan")])
    assert e.value.status == L.ERANGE
    assert L.raw().dit_plan_schedule(ctx_tiny.handle, C.byref(mw.struct), None, 2) == L.EINVAL
    assert L.raw().dit_plan_schedule(None, C.byref(mw.struct), None, 0) == L.EINVAL
    ctx_tiny.plan_schedule(mw, [])


@pytest.mark.parametrize("w8a8,Lh", [(False, (8, 8, 8)), (True, (8, 8, 8)), (False, (0, 4, 4))])
def test_denoise_twin(ctx_tiny, w8a8, Lh):
    """A reduced-width DiT (hidden 256, 2 heads, 3 blocks, 8 text + 8x8 image
    rows, text features 256-d) through the full 4-step loop; bf16 or W8A8
    block weights; and one with no text rows (4x4 image rows only, no
    prologue: the step takes no text)."""
    Ln, h, w = Lh
    m = synth.model_case("dit32", blocks=3, hidden=256, heads=2, ffn=1024, L=Ln, h=h, w=w, text_dim=256, w8a8=w8a8)
    sh = m["shape"]
    la, oa = arch_pair(sh)
    ctx = L.Context(la, max_rows=sh.S)
    say("denoise twin S =", sh.S, "L =", sh.L)
    mw = L.ModelWeights.from_host(m["top"], m["blocks"])
    pos = torch.empty((sh.S, 3), dtype=torch.int32, device="cuda")
    ctx.positions(sh.L, sh.h, sh.w, pos)
    cs = torch.empty((sh.S, 64), dtype=torch.float32, device="cuda")
    sn = torch.empty_like(cs)
    ctx.rope_tables(pos, sh.S, cs, sn)
    txt = torch.empty((sh.L, sh.hidden), dtype=torch.float32, device="cuda")
    if sh.L > 0:
        ctx.prologue(mw, L.dev_f32(m["ctx"]), sh.L, txt)
    x = L.dev_f32(m["x_lat"])
    sig = O.sigma_grid(4)
    vels = []
    for i in range(4):
        v = torch.empty((sh.N, sh.latent), dtype=torch.float32, device="cuda")
        ctx.denoise_step(mw, x, txt, cs, sn, sh.L, sh.N, float(sig[i]), float(sig[i + 1]), v)
        vels.append(v)
    torch.cuda.synchronize()
    ow = O.ModelWeights(**m["top"], blocks=[oracle_block(b) for b in m["blocks"]])
    opos = O.positions(sh.L, sh.h, sh.w)
    ocs, osn = O.rope_tables(opos, sh.axes)
    if sh.L > 0:
        compare("txt", np_of(txt), O.text_rows(m["ctx"], ow))
    xr, vr = O.denoise(m["x_lat"], m["ctx"], ow, ocs, osn, sig, oa, keep_velocities=True)
    compare("vel0", np_of(vels[0]), vr[0])
    for i in range(1, 4):
        compare(f"vel{i}", np_of(vels[i]), vr[i])
    compare("x_final", np_of(x), xr)
    ctx.close()
