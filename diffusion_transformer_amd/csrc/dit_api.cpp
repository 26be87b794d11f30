// libdit C ABI: argument validation, the context and its workspace, and the
// launch sequences of a block forward and a denoise step.
//
// Sources: "gizai:dit" reference (Block.forward, Work, CHUNK, Modulation);
// "Host contract -- RGBA-Image-2.1-Turbo" s.1 (DiT graph boundary and axes),
// s.4 (positions, rotary tables), s.6 (Euler sampler); "944 -> 346 ms:
// optimizing FLUX.2 klein-4B on one TPU v6e chip" s.4.1 (resident weights)
// and Appendix B D2 (text rows and rotary tables hoisted out of the loop).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/dit.h"
#include "kernels.h"

using namespace dit;

struct dit_ctx {
    int device = -1;
    hipStream_t stream = nullptr;
    dit_arch arch{};
    int max_rows = 0;
    int max_rows_pad = 0;
    void *pool = nullptr;
    size_t pool_bytes = 0;
    // workspace ([GZ] Work), carved from one allocation
    float *mod = nullptr, *vec = nullptr, *temb = nullptr, *t1 = nullptr, *fmod = nullptr;
    uint16_t *h = nullptr, *h2 = nullptr, *q = nullptr, *k = nullptr, *vt = nullptr, *o = nullptr,
             *a = nullptr, *latb = nullptr, *ctxb = nullptr;
    // parallel block: [attention output | SwiGLU output] per row, the one A
    // operand of its fused output product
    uint16_t *oa = nullptr;
    // a sandwich block's fp32 product output [S, D]; it shares oa's memory
    // (the sequential and the parallel block never run at once on one
    // context: its calls are ordered on its stream)
    float *yf = nullptr;
    // W8A8 blocks: a product's A rows as INT8 codes [Sx, max(D, F)] and
    // their scales [Sx]
    int8_t *aq = nullptr;
    float *as = nullptr;
    float *seq = nullptr, *vel = nullptr;
    size_t bytes[9] = {};
    // QK-norm + rotary inside the QKV product's epilogue (true), or the
    // product's bf16 projection and then the separate prep pass
    bool qk_fused = true;
    // int8 block-32 weights: converted inside the product (true), or by a
    // pass into wdq (two slots of wdq_slot bf16 values, allocated on first
    // use) before a bf16 product
    bool int8_in_product = false;
    uint16_t *wdq = nullptr;
    // a second stream of the context (default priority) on which the
    // sequential block dequantises its later weights while the first
    // products run; the events order it against the context's stream
    hipStream_t side = nullptr;
    hipEvent_t ev_fork = nullptr, ev_ready[4] = {};
    // a planned schedule (dit_plan_schedule): the time vectors [n][D], every
    // block's modulation rows [n][blocks][6D] and the final layer's [n][2D]
    // for the sigmas plan_sig, computed from the weights named in plan_keys
    // (time MLP, final modulation, each block's modulation weight)
    float *plan_mem = nullptr, *plan_vec = nullptr, *plan_mod = nullptr, *plan_fmod = nullptr;
    size_t plan_bytes = 0;
    int plan_n = 0;
    std::vector<float> plan_sig;
    std::vector<const void *> plan_keys;
    std::string err;
    // stage timing
    bool timing = false;
    struct Rec {
        int stage;
        hipEvent_t a, b;
    };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> spare;
};

namespace {

// modulation rows the workspace holds (six vectors of D each): the runs
// form of the block takes at most this many conditioning vectors; the
// double-stream block uses two
constexpr int kMaxModRows = 8;

thread_local std::string g_err;

// a block's bf16 block-32 weight scales (DIT_W_INT8_B32)
inline const uint16_t *bscale(const dit_block *b, int i) { return static_cast<const uint16_t *>(b->scale[i]); }

dit_status fail(dit_ctx *c, dit_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (c)
        c->err = buf;
    else
        g_err = buf;
    return s;
}

dit_status check_launch(dit_ctx *c, hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(c, DIT_EDEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
    return DIT_OK;
}

}  // namespace

// The last-error text of calls that take no context (dit_last_error(NULL)),
// for the entry points defined in other sources of the library.
void dit_set_global_error(const char *msg) { g_err = msg; }

namespace {

#define DIT_TRY(expr)                      \
    do {                                   \
        dit_status _s = (expr);            \
        if (_s != DIT_OK) return _s;       \
    } while (0)

#define DIT_LAUNCH(c, expr, what) DIT_TRY(check_launch((c), (expr), (what)))

int round_up(int a, int b) { return (a + b - 1) / b * b; }

hipEvent_t take_event(dit_ctx *c) {
    if (!c->spare.empty()) {
        hipEvent_t e = c->spare.back();
        c->spare.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Brackets one launch stage with HIP events when timing is enabled.
struct Stage {
    dit_ctx *c;
    int stage;
    hipEvent_t a = nullptr;
    hipStream_t hs;
    Stage(dit_ctx *ctx, int s, hipStream_t on = nullptr) : c(ctx), stage(s), hs(on ? on : ctx->stream) {
        if (!c->timing) return;
        a = take_event(c);
        if (a) hipEventRecord(a, hs);
    }
    ~Stage() {
        if (!a) return;
        hipEvent_t b = take_event(c);
        if (!b) {
            c->spare.push_back(a);
            return;
        }
        hipEventRecord(b, hs);
        c->recs.push_back({stage, a, b});
    }
};

void drop_records(dit_ctx *c) {
    for (auto &r : c->recs) {
        c->spare.push_back(r.a);
        c->spare.push_back(r.b);
    }
    c->recs.clear();
}

dit_status validate_arch(const dit_arch *a) {
    if (!a) return fail(nullptr, DIT_EINVAL, "arch is NULL");
    if (a->head_dim != 128) return fail(nullptr, DIT_EUNSUPPORTED, "head_dim %d: only 128 is supported", a->head_dim);
    if (a->heads < 1 || a->hidden != a->heads * a->head_dim)
        return fail(nullptr, DIT_EINVAL, "hidden %d != heads %d * head_dim %d", a->hidden, a->heads, a->head_dim);
    if (a->hidden % 256 || a->hidden > 4096)
        return fail(nullptr, DIT_EUNSUPPORTED, "hidden %d: must be a multiple of 256, at most 4096", a->hidden);
    if (a->ffn < 256 || a->ffn % 256 || a->ffn > 65536)
        return fail(nullptr, DIT_EUNSUPPORTED, "ffn %d: must be a multiple of 256 in 256..65536", a->ffn);
    if (a->axes[0] < 0 || a->axes[1] < 0 || a->axes[2] < 0 || a->axes[0] % 2 || a->axes[1] % 2 ||
        a->axes[2] % 2 || a->axes[0] + a->axes[1] + a->axes[2] != a->head_dim)
        return fail(nullptr, DIT_EINVAL, "rotary axes %d+%d+%d must be even and sum to head_dim", a->axes[0],
                    a->axes[1], a->axes[2]);
    if (!(a->eps > 0) || !(a->qk_eps > 0) || !(a->final_eps > 0) || !(a->rope_theta > 0))
        return fail(nullptr, DIT_EINVAL, "eps and rope_theta must be positive");
    if (a->norm != DIT_NORM_LAYER && a->norm != DIT_NORM_RMS) return fail(nullptr, DIT_EINVAL, "unknown norm %d", a->norm);
    if (a->time_dim < 2 || a->time_dim % 8 || a->time_dim > 4096)
        return fail(nullptr, DIT_EINVAL, "time_dim %d: must be a multiple of 8 in 8..4096", a->time_dim);
    if (a->latent < 64 || a->latent % 64 || a->latent > 4096)
        return fail(nullptr, DIT_EINVAL, "latent %d: must be a multiple of 64", a->latent);
    if (a->text_dim < 64 || a->text_dim % 64 || a->text_dim > 65536)
        return fail(nullptr, DIT_EINVAL, "text_dim %d: must be a multiple of 64", a->text_dim);
    return DIT_OK;
}

dit_status check_ctx(dit_ctx *c) {
    if (!c) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (c->device < 0 || !c->pool) return fail(c, DIT_EDEVICE, "context has no device");
    if (hipSetDevice(c->device) != hipSuccess) return fail(c, DIT_EDEVICE, "hipSetDevice(%d) failed", c->device);
    return DIT_OK;
}

// `sequential`: whether the form is a sequential one, which alone takes a
// sandwich block's post norms and W8A8 weights; the others reject them.
bool aligned_to(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
dit_status check_block(dit_ctx *c, const dit_block *b, bool parallel = false, bool sequential = false) {
    if (!b) return fail(c, DIT_EINVAL, "block is NULL");
    if (b->wtype != DIT_W_BF16 && b->wtype != DIT_W_INT8_B32 && b->wtype != DIT_W_INT8_ROW &&
        b->wtype != DIT_W_INT8_ROT)
        return fail(c, DIT_EINVAL, "unknown wtype %d", b->wtype);
    const bool w8a8 = b->wtype == DIT_W_INT8_ROW || b->wtype == DIT_W_INT8_ROT;
    if (w8a8 && !sequential)
        return fail(c, DIT_EINVAL, "W8A8 weights are taken by the sequential block forms only");
    // the SwiGLU rows of a W8A8 block are quantized one row per workgroup,
    // at most 16384 wide; refused here, before the attention half updates x
    if (w8a8 && c->arch.ffn > 16384)
        return fail(c, DIT_EUNSUPPORTED, "W8A8 blocks take ffn up to 16384 (arch ffn %d)", c->arch.ffn);
    // the products and the GEMV read weights in 16-byte pieces, scales in
    // 4-byte ones
    for (int i = 0; i < 4; ++i) {
        if (!b->w[i]) return fail(c, DIT_EINVAL, "block weight w[%d] is NULL", i);
        if (b->wtype != DIT_W_BF16 && !b->scale[i]) return fail(c, DIT_EINVAL, "int8 weight %d has no scales", i);
        if (b->wtype == DIT_W_BF16 && b->scale[i]) return fail(c, DIT_EINVAL, "bf16 weight %d given scales", i);
        if (!aligned_to(b->w[i], 16) || !aligned_to(b->scale[i], 4))
            return fail(c, DIT_EINVAL, "weight %d: w must be 16-byte and scale 4-byte aligned", i);
    }
    if (!b->w_mod) return fail(c, DIT_EINVAL, "block w_mod is NULL");
    if (!aligned_to(b->w_mod, 16)) return fail(c, DIT_EINVAL, "block w_mod must be 16-byte aligned");
    if (!b->norm_w[2] || !b->norm_w[3]) return fail(c, DIT_EINVAL, "head-norm weights are NULL");
    for (int i = 0; i < 4; ++i)
        if (!aligned_to(b->norm_w[i], 16) || (i < 2 && !aligned_to(b->post_w[i], 16)))
            return fail(c, DIT_EINVAL, "norm and post-norm weights must be 16-byte aligned");
    if (c->arch.norm == DIT_NORM_RMS && (!b->norm_w[0] || (!parallel && !b->norm_w[1])))
        return fail(c, DIT_EINVAL, parallel ? "RMSNorm needs norm weight NORM1" : "RMSNorm needs norm weights NORM1 and NORM2");
    if (!b->post_w[0] != !b->post_w[1])
        return fail(c, DIT_EINVAL, "a sandwich block needs both post-norm weights (POST_ATTN and POST_MLP)");
    if (b->post_w[0] && !sequential)
        return fail(c, DIT_EINVAL, "sandwich norms are taken by the sequential block forms only");
    return DIT_OK;
}

// The weight operand of product w of block b (N outputs, K inputs) as the
// product launch takes it: bf16 weights as they are; int8 block-32 weights
// either as codes and scales (converted inside the product) or, by default,
// dequantised first into the context's scratch: two sets (the double-stream
// block's streams) of one slot per block weight, each of that weight's size.
struct WeightArg {
    const void *w;
    const uint16_t *scale;
    bool w8;
};
size_t wdq_elems(const dit_ctx *c, int w) {
    const size_t D = c->arch.hidden, F = c->arch.ffn;
    const size_t n[4] = {3 * D * D, D * D, 2 * F * D, F * D};
    return n[w];
}
uint16_t *wdq_slot(const dit_ctx *c, int set, int w) {
    size_t off = set * (wdq_elems(c, 0) + wdq_elems(c, 1) + wdq_elems(c, 2) + wdq_elems(c, 3));
    for (int i = 0; i < w; ++i) off += wdq_elems(c, i);
    return c->wdq + off;
}
dit_status ensure_wdq(dit_ctx *c) {
    if (c->wdq) return DIT_OK;
    const size_t n = 2 * (wdq_elems(c, 0) + wdq_elems(c, 1) + wdq_elems(c, 2) + wdq_elems(c, 3));
    void *p = nullptr;
    if (hipMalloc(&p, n * sizeof(uint16_t)) != hipSuccess)
        return fail(c, DIT_ENOMEM, "int8 dequantisation scratch (%zu bytes) failed", n * sizeof(uint16_t));
    c->wdq = static_cast<uint16_t *>(p);
    return DIT_OK;
}
dit_status ensure_side(dit_ctx *c) {
    if (c->side) return DIT_OK;
    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess)
        return fail(c, DIT_EDEVICE, "creating the dequantisation stream failed");
    bool ok = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) == hipSuccess;
    for (hipEvent_t &e : c->ev_ready) ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
    c->side = s;
    return ok ? DIT_OK : fail(c, DIT_EDEVICE, "creating the dequantisation events failed");
}
// Dequantises int8 codes wp (N x K, block-32 scales, 16-byte aligned) into
// dst of cap values on stream hs when the context takes that path and they
// fit; otherwise the codes themselves.
dit_status weight_arg_of(dit_ctx *c, const void *wp, const uint16_t *scale, bool int8, int N, int K, uint16_t *dst,
                         size_t cap, hipStream_t hs, WeightArg *out) {
    *out = WeightArg{wp, nullptr, false};
    if (!int8) return DIT_OK;
    if (c->int8_in_product || static_cast<size_t>(N) * K > cap) {
        *out = WeightArg{wp, scale, true};
        return DIT_OK;
    }
    {
        Stage t(c, DIT_ST_DEQUANT, hs);
        DIT_LAUNCH(c, launch_dequant_bf16(static_cast<const int8_t *>(wp), scale, N, K, dst, hs), "int8 dequantisation");
    }
    *out = WeightArg{dst, nullptr, false};
    return DIT_OK;
}
dit_status weight_arg(dit_ctx *c, const dit_block *b, int w, int N, int K, int set, WeightArg *out) {
    const bool int8 = b->wtype == DIT_W_INT8_B32;
    if (int8 && !c->int8_in_product) DIT_TRY(ensure_wdq(c));
    return weight_arg_of(c, b->w[w], bscale(b, w), int8, N, K, int8 && c->wdq ? wdq_slot(c, set, w) : nullptr,
                         int8 && c->wdq ? wdq_elems(c, w) : 0, c->stream, out);
}

dit_status check_rows(dit_ctx *c, int L, int N) {
    if (L < 0 || L > 512) return fail(c, DIT_ERANGE, "L = %d outside 0..512", L);
    if (N < 1 || N > 4096) return fail(c, DIT_ERANGE, "N = %d outside 1..4096", N);
    if (L + N > c->max_rows) return fail(c, DIT_ERANGE, "L + N = %d exceeds max_rows %d", L + N, c->max_rows);
    return DIT_OK;
}

// The parallel block's launch sequence ([GZ] Block.parallel; validated
// arguments): modulation (shift, scale, gate), one modulated norm, then for
// bf16 weights at ping-pong sizes one product over [QKV | UP] (head-norm +
// rotary epilogue on the QKV columns, SwiGLU on the rest, written beside the
// attention output) and one gated-residual product over [o | a] with
// [W_out | W_down] (k < D from W_out, the rest from W_down); otherwise the
// same as four products.
dit_status parallel_block_forward(dit_ctx *c, const dit_block *b, float *x, const float *vec, const float *cs,
                                  const float *sn, int S) {
    const dit_arch &A = c->arch;
    const int D = A.hidden, F = A.ffn, H = A.heads;
    const int Sp = round_up(S, 64);
    const bool w8 = b->wtype == DIT_W_INT8_B32;
    const bool rms = A.norm == DIT_NORM_RMS;
    hipStream_t st = c->stream;
    float *mod = c->mod;

    {
        Stage t(c, DIT_ST_MOD);
        DIT_LAUNCH(c, launch_gemv(b->w_mod, vec, 3 * D, D, true, mod, st), "modulation");
    }
    {
        Stage t(c, DIT_ST_NORM1);
        DIT_LAUNCH(c, launch_modnorm(x, S, D, mod, mod + D, b->norm_w[0], rms, A.eps, c->h, st), "norm");
    }
    GemmEpi e{};
    e.kind = EPI_QKV;
    e.q = c->q;
    e.k = c->k;
    e.vt = c->vt;
    e.heads = H;
    e.ldv = Sp;
    e.qn = b->norm_w[2];
    e.kn = b->norm_w[3];
    e.cos = cs;
    e.sin = sn;
    e.qk_eps = A.qk_eps;
    GemmEpi fin = e;
    fin.kind = EPI_QKV_SWIGLU;
    fin.w2 = static_cast<const uint16_t *>(b->w[2]);
    fin.n_split = 3 * D;
    fin.act = c->oa + D;
    fin.ld_act = D + F;
    GemmEpi g{};
    g.kind = EPI_GATE_RES;
    g.out = x;
    g.ldo = D;
    g.gate = mod + 2 * D;
    GemmEpi gk = g;
    gk.w2 = static_cast<const uint16_t *>(b->w[3]);
    gk.k_split = D;
    // the fused pair of products takes bf16 weights: bf16 blocks, and int8
    // block-32 blocks dequantised by a pass first
    const bool dq = !c->int8_in_product;
    const bool fused = (!w8 || dq) && gemm_pingpong_ok(S, 3 * D + 2 * F, D, false, fin, true) &&
                       gemm_pingpong_ok(S, D, D + F, false, gk, true);
    WeightArg wa{}, wb{};
    if (fused) {
        DIT_TRY(weight_arg(c, b, 0, 3 * D, D, 0, &wa));
        DIT_TRY(weight_arg(c, b, 2, 2 * F, D, 0, &wb));
        fin.w2 = static_cast<const uint16_t *>(wb.w);
        {
            Stage t(c, DIT_ST_PAR_IN);
            DIT_LAUNCH(c, launch_gemm(c->h, wa.w, nullptr, false, S, 3 * D + 2 * F, D, fin, st, true), "qkv+up");
        }
        {
            Stage t(c, DIT_ST_ATTN);
            DIT_LAUNCH(c, launch_attention(c->q, c->k, c->vt, H, S, Sp, c->oa, D + F, st), "attention");
        }
        DIT_TRY(weight_arg(c, b, 1, D, D, 0, &wa));
        DIT_TRY(weight_arg(c, b, 3, D, F, 0, &wb));
        gk.w2 = static_cast<const uint16_t *>(wb.w);
        {
            Stage t(c, DIT_ST_PAR_OUT);
            DIT_LAUNCH(c, launch_gemm(c->oa, wa.w, nullptr, false, S, D, D + F, gk, st, true), "out+down");
        }
        return DIT_OK;
    }
    DIT_TRY(weight_arg(c, b, 0, 3 * D, D, 0, &wa));
    {
        Stage t(c, DIT_ST_QKV);
        DIT_LAUNCH(c, launch_gemm(c->h, wa.w, wa.scale, wa.w8, S, 3 * D, D, e, st, true), "qkv");
    }
    GemmEpi u{};
    u.kind = EPI_SWIGLU;
    u.act = c->a;
    DIT_TRY(weight_arg(c, b, 2, 2 * F, D, 0, &wa));
    {
        Stage t(c, DIT_ST_UP);
        DIT_LAUNCH(c, launch_gemm(c->h, wa.w, wa.scale, wa.w8, S, 2 * F, D, u, st, true), "up");
    }
    {
        Stage t(c, DIT_ST_ATTN);
        DIT_LAUNCH(c, launch_attention(c->q, c->k, c->vt, H, S, Sp, c->o, D, st), "attention");
    }
    DIT_TRY(weight_arg(c, b, 1, D, D, 0, &wa));
    {
        Stage t(c, DIT_ST_OUT);
        DIT_LAUNCH(c, launch_gemm(c->o, wa.w, wa.scale, wa.w8, S, D, D, g, st, true), "out");
    }
    DIT_TRY(weight_arg(c, b, 3, D, F, 0, &wa));
    {
        Stage t(c, DIT_ST_DOWN);
        DIT_LAUNCH(c, launch_gemm(c->a, wa.w, wa.scale, wa.w8, S, D, F, g, st, true), "down");
    }
    return DIT_OK;
}

// The double-stream block's launch sequence ([K4] Appendix B, double blocks;
// validated arguments): rows [0, L) take the text stream's weights and
// modulation, rows [L, S) the image stream's; each product runs once per
// stream over its rows (the image stream's from row L of the operands; QKV
// writes q, k and vt at the stream's row offset), the attention once over
// all rows.  The modulation buffer holds the text stream's six rows, then
// the image stream's.
dit_status double_block_forward(dit_ctx *c, const dit_block *bt, const dit_block *bi, float *x, const float *vec,
                                const float *cs, const float *sn, int L, int N) {
    const dit_arch &A = c->arch;
    const int D = A.hidden, F = A.ffn, H = A.heads;
    const int S = L + N, Sp = round_up(S, 64);
    const bool rms = A.norm == DIT_NORM_RMS;
    hipStream_t st = c->stream;
    struct Stream {
        const dit_block *b;
        int r0, rows;
        float *mod;
    };
    const Stream sts[2] = {{bt, 0, L, c->mod}, {bi, L, N, c->mod + 6 * D}};
    for (const Stream &t : sts) {
        Stage tm(c, DIT_ST_MOD);
        DIT_LAUNCH(c, launch_gemv(t.b->w_mod, vec, 6 * D, D, true, t.mod, st), "modulation");
    }
    for (const Stream &t : sts) {
        if (!t.rows) continue;
        Stage tm(c, DIT_ST_NORM1);
        DIT_LAUNCH(c, launch_modnorm(x + int64_t(t.r0) * D, t.rows, D, t.mod, t.mod + D, t.b->norm_w[0], rms, A.eps,
                                     c->h + int64_t(t.r0) * D, st),
                   "norm1");
    }
    // one launch per product for both streams (image tiles first) when both
    // take the ping-pong kernel with the same weight type; streams with
    // different weight types: two launches
    const bool mixed = bt->wtype != bi->wtype;
    // weights of both streams for product w: image stream in scratch slot 0,
    // text stream in slot 1 (int8 block-32 weights dequantised by a pass)
    WeightArg wgt[2]{};
    auto weights = [&](int w, int n, int k) -> dit_status {
        for (int i = 1; i >= 0; --i)
            if (sts[i].rows) DIT_TRY(weight_arg(c, sts[i].b, w, n, k, 1 - i, &wgt[i]));
        return DIT_OK;
    };
    auto two = [&](int kind, const uint16_t *a_base, int64_t a_ld, const GemmEpi (&ep)[2], int w, int n, int k) {
        const Stream &ti = sts[1], &tt = sts[0];
        (void)w;
        if (mixed || wgt[0].w8 != wgt[1].w8) {
            hipError_t e = hipSuccess;
            for (int i = 1; i >= 0 && e == hipSuccess; --i) {
                const Stream &t = sts[i];
                if (t.rows)
                    e = launch_gemm(a_base + int64_t(t.r0) * a_ld, wgt[i].w, wgt[i].scale, wgt[i].w8, t.rows, n, k, ep[i],
                                    st, true);
            }
            return e;
        }
        (void)kind;
        return launch_gemm2(a_base + int64_t(ti.r0) * a_ld, wgt[1].w, wgt[1].scale, ti.rows, ep[1],
                            a_base + int64_t(tt.r0) * a_ld, wgt[0].w, wgt[0].scale, tt.rows, ep[0], wgt[1].w8, n, k, st);
    };
    {
        GemmEpi e[2]{};
        for (int i = 0; i < 2; ++i) {
            const Stream &t = sts[i];
            e[i].kind = EPI_QKV;
            e[i].q = c->q;
            e[i].k = c->k;
            e[i].vt = c->vt;
            e[i].heads = H;
            e[i].ldv = Sp;
            e[i].qn = t.b->norm_w[2];
            e[i].kn = t.b->norm_w[3];
            e[i].cos = cs + int64_t(t.r0) * 64;
            e[i].sin = sn + int64_t(t.r0) * 64;
            e[i].qk_eps = A.qk_eps;
            e[i].row_base = t.r0;
            e[i].rows_total = S;
        }
        DIT_TRY(weights(0, 3 * D, D));
        Stage tm(c, DIT_ST_QKV);
        DIT_LAUNCH(c, two(EPI_QKV, c->h, D, e, 0, 3 * D, D), "qkv");
    }
    {
        Stage tm(c, DIT_ST_ATTN);
        DIT_LAUNCH(c, launch_attention(c->q, c->k, c->vt, H, S, Sp, c->o, D, st), "attention");
    }
    {
        GemmEpi g[2]{};
        for (int i = 0; i < 2; ++i) {
            g[i].kind = EPI_GATE_RES;
            g[i].out = x + int64_t(sts[i].r0) * D;
            g[i].ldo = D;
            g[i].gate = sts[i].mod + 2 * D;
        }
        DIT_TRY(weights(1, D, D));
        Stage tm(c, DIT_ST_OUT);
        DIT_LAUNCH(c, two(EPI_GATE_RES, c->o, D, g, 1, D, D), "out");
    }
    for (const Stream &t : sts) {
        if (!t.rows) continue;
        Stage tm(c, DIT_ST_NORM2);
        DIT_LAUNCH(c, launch_modnorm(x + int64_t(t.r0) * D, t.rows, D, t.mod + 3 * D, t.mod + 4 * D, t.b->norm_w[1], rms,
                                     A.eps, c->h2 + int64_t(t.r0) * D, st),
                   "norm2");
    }
    {
        GemmEpi u[2]{};
        for (int i = 0; i < 2; ++i) {
            u[i].kind = EPI_SWIGLU;
            u[i].act = c->a + int64_t(sts[i].r0) * F;
        }
        DIT_TRY(weights(2, 2 * F, D));
        Stage tm(c, DIT_ST_UP);
        DIT_LAUNCH(c, two(EPI_SWIGLU, c->h2, D, u, 2, 2 * F, D), "up");
    }
    {
        GemmEpi g[2]{};
        for (int i = 0; i < 2; ++i) {
            g[i].kind = EPI_GATE_RES;
            g[i].out = x + int64_t(sts[i].r0) * D;
            g[i].ldo = D;
            g[i].gate = sts[i].mod + 5 * D;
        }
        DIT_TRY(weights(3, D, F));
        Stage tm(c, DIT_ST_DOWN);
        DIT_LAUNCH(c, two(EPI_GATE_RES, c->a, F, g, 3, D, F), "down");
    }
    return DIT_OK;
}

// The block with several modulation rows over runs of rows ([GZ] Sequence
// map/runs, Modulation, gatedInto: one gated product per run; validated
// arguments, runs[i] = (first, end, row) on the host, tiling [0, S)).  The
// norms run per run with the run's shift and scale; QKV, the attention and
// UP once over all rows; OUT and DOWN per run with the run's gate, two runs
// per launch.
// Keys and values of rows [first, Sk) between the block's q/k/vt buffers
// (head stride Sk, V^T row stride round_up(Sk, 64)) and a RefSlot's rows:
// K [H, count, 128] then V^T [H, 128, count], count = Sk - first; out:
// buffers -> slot (a recording step), else slot -> buffers.
dit_status ref_copy(dit_ctx *c, uint16_t *slot_mut, const uint16_t *slot, int first, int Sk, bool out) {
    const int H = c->arch.heads, count = Sk - first, ldv = round_up(Sk, 64);
    if (count <= 0) return DIT_OK;
    uint16_t *sk = const_cast<uint16_t *>(out ? slot_mut : slot);
    uint16_t *sv = sk + static_cast<size_t>(H) * count * 128;
    uint16_t *bk = c->k + static_cast<size_t>(first) * 128, *bv = c->vt + first;
    const size_t kw = static_cast<size_t>(count) * 256, kp = static_cast<size_t>(Sk) * 256;
    const size_t vw = static_cast<size_t>(count) * 2, vp = static_cast<size_t>(ldv) * 2;
    hipError_t e = out ? hipMemcpy2DAsync(sk, kw, bk, kp, kw, H, hipMemcpyDeviceToDevice, c->stream)
                       : hipMemcpy2DAsync(bk, kp, sk, kw, kw, H, hipMemcpyDeviceToDevice, c->stream);
    if (e == hipSuccess)
        e = out ? hipMemcpy2DAsync(sv, vw, bv, vp, vw, static_cast<size_t>(H) * 128, hipMemcpyDeviceToDevice, c->stream)
                : hipMemcpy2DAsync(bv, vp, sv, vw, vw, static_cast<size_t>(H) * 128, hipMemcpyDeviceToDevice, c->stream);
    if (e != hipSuccess) return fail(c, DIT_EDEVICE, "reference key/value copy: %s", hipGetErrorString(e));
    return DIT_OK;
}

// With Sk > S the rows [S, Sk) are read-only context ([GZ] Sequence.active,
// RefSlot): their keys and values come from `slot` (K [H, Sk - S, 128] then
// V^T [H, 128, Sk - S]), copied in after the QKV product of rows [0, S), and
// the attention's queries are rows [0, S) against all Sk keys.
dit_status block_forward_runs(dit_ctx *c, const dit_block *b, float *x, const float *vecs, int R, const int32_t *runs,
                              int n_runs, const float *cs, const float *sn, int S, int Sk = 0,
                              const uint16_t *slot = nullptr, const float *pre_mod = nullptr) {
    const dit_arch &A = c->arch;
    const int D = A.hidden, F = A.ffn, H = A.heads;
    if (Sk < S) Sk = S;
    const int Sp = round_up(Sk, 64);
    const bool rms = A.norm == DIT_NORM_RMS;
    hipStream_t st = c->stream;
    // the modulation rows: computed here, or given (one vector's six rows,
    // from a planned schedule)
    const float *mod = pre_mod ? pre_mod : c->mod;
    for (int r = 0; r < R && !pre_mod; ++r) {
        Stage t(c, DIT_ST_MOD);
        DIT_LAUNCH(c, launch_gemv(b->w_mod, vecs + int64_t(r) * D, 6 * D, D, true, c->mod + int64_t(r) * 6 * D, st),
                   "modulation");
    }
    // W8A8 (DIT_W_INT8_ROW, DIT_W_INT8_ROT): every product takes its A rows
    // as INT8 codes and a scale a row in aq / as -- from the norms directly,
    // from a quantization pass over o and a; with DIT_W_INT8_ROT each 256
    // values of a row are rotated by the regular Hadamard of 256 first
    const bool q8 = b->wtype == DIT_W_INT8_ROW || b->wtype == DIT_W_INT8_ROT;
    const bool rot = b->wtype == DIT_W_INT8_ROT;
    auto norms = [&](const float *shift_of, int which, uint16_t *out, const float *nw) -> dit_status {
        for (int i = 0; i < n_runs; ++i) {
            const int f = runs[3 * i], e = runs[3 * i + 1], m = runs[3 * i + 2];
            const float *mr = mod + int64_t(m) * 6 * D;
            const float *sh = mr + (shift_of - mod), *sc = sh + D;
            Stage t(c, which);
            if (q8)
                DIT_LAUNCH(c, launch_modnorm_i8(x + int64_t(f) * D, e - f, D, sh, sc, nw, rms, A.eps,
                                                c->aq + int64_t(f) * D, c->as + f, st, rot),
                           "norm");
            else
                DIT_LAUNCH(c, launch_modnorm(x + int64_t(f) * D, e - f, D, sh, sc, nw, rms, A.eps, out + int64_t(f) * D, st),
                           "norm");
        }
        return DIT_OK;
    };
    // the product of weight w over rows [r0, r0 + M) of A (bf16 a with row
    // stride K, or the INT8 rows in aq / as); wa: the weight operand of
    // bf16 and int8 block-32 blocks (weight_arg)
    WeightArg wa{};
    auto product = [&](const uint16_t *a, int r0, int M, int w, int N, int K, const GemmEpi &ep) -> hipError_t {
        if (q8)
            return launch_gemm_w8a8(c->aq + int64_t(r0) * K, c->as + r0, static_cast<const int8_t *>(b->w[w]),
                                    static_cast<const float *>(b->scale[w]), M, N, K, ep, st);
        return launch_gemm(a + int64_t(r0) * K, wa.w, wa.scale, wa.w8, M, N, K, ep, st, true);
    };
    // int8 block-32 weights dequantised by the pass: OUT, UP and DOWN on
    // the second stream, started once the QKV product is done, where they
    // can take compute units the attention's second round of tiles leaves
    // idle; each of those products waits for its own weight
    const bool async_dq = b->wtype == DIT_W_INT8_B32 && !c->int8_in_product;
    auto fork_dequant = [&]() -> dit_status {
        if (!async_dq) return DIT_OK;
        DIT_TRY(ensure_wdq(c));
        DIT_TRY(ensure_side(c));
        if (hipEventRecord(c->ev_fork, st) != hipSuccess || hipStreamWaitEvent(c->side, c->ev_fork, 0) != hipSuccess)
            return fail(c, DIT_EDEVICE, "ordering the dequantisation stream failed");
        const int nk[4][2] = {{3 * D, D}, {D, D}, {2 * F, D}, {D, F}};
        for (int w = 1; w < 4; ++w) {
            {
                Stage t(c, DIT_ST_DEQUANT, c->side);
                DIT_LAUNCH(c, launch_dequant_bf16(static_cast<const int8_t *>(b->w[w]), bscale(b, w), nk[w][0], nk[w][1],
                                                  wdq_slot(c, 0, w), c->side),
                           "int8 dequantisation");
            }
            if (hipEventRecord(c->ev_ready[w], c->side) != hipSuccess)
                return fail(c, DIT_EDEVICE, "recording a dequantised weight failed");
        }
        return DIT_OK;
    };
    auto prep = [&](int w, int N, int K) -> dit_status {
        if (q8) return DIT_OK;
        if (async_dq && w > 0) {
            if (hipStreamWaitEvent(st, c->ev_ready[w], 0) != hipSuccess)
                return fail(c, DIT_EDEVICE, "waiting for a dequantised weight failed");
            wa = WeightArg{wdq_slot(c, 0, w), nullptr, false};
            return DIT_OK;
        }
        return weight_arg(c, b, w, N, K, 0, &wa);
    };
    // OUT / DOWN: x[run] += gate(run) * (a_base[run] W^T), two runs per
    // launch; a sandwich block's product writes its rows in fp32 and the
    // post norm adds them, normed, with the run's gate
    auto gated = [&](const uint16_t *a_base, int lda, int w, int K, int gate_at, int stage,
                     const float *post) -> dit_status {
        if (q8) {
            Stage t(c, DIT_ST_QUANT);
            DIT_LAUNCH(c, launch_quant_rows(a_base, S, K, c->aq, c->as, st, rot), "quantize rows");
        }
        DIT_TRY(prep(w, D, K));
        if (post) {
            GemmEpi f{};
            f.kind = EPI_F32;
            f.out = c->yf;
            f.ldo = D;
            {
                Stage t(c, stage);
                DIT_LAUNCH(c, product(a_base, 0, S, w, D, K, f), "product");
            }
            for (int i = 0; i < n_runs; ++i) {
                const int r0 = runs[3 * i], r1 = runs[3 * i + 1];
                Stage t(c, DIT_ST_POST);
                DIT_LAUNCH(c, launch_post_norm_gate(c->yf + int64_t(r0) * D, r1 - r0, D, post, rms, A.eps,
                                                    mod + int64_t(runs[3 * i + 2]) * 6 * D + gate_at,
                                                    x + int64_t(r0) * D, st),
                           "post norm");
            }
            return DIT_OK;
        }
        if (q8) {
            for (int i = 0; i < n_runs; ++i) {
                const int r0 = runs[3 * i], r1 = runs[3 * i + 1];
                GemmEpi g{};
                g.kind = EPI_GATE_RES;
                g.out = x + int64_t(r0) * D;
                g.ldo = D;
                g.gate = mod + int64_t(runs[3 * i + 2]) * 6 * D + gate_at;
                Stage t(c, stage);
                DIT_LAUNCH(c, product(a_base, r0, r1 - r0, w, D, K, g), "gated product");
            }
            return DIT_OK;
        }
        for (int i = 0; i < n_runs; i += 2) {
            GemmEpi g[2]{};
            int f[2] = {0, 0}, rows[2] = {0, 0};
            for (int j = 0; j < 2 && i + j < n_runs; ++j) {
                f[j] = runs[3 * (i + j)];
                rows[j] = runs[3 * (i + j) + 1] - f[j];
                g[j].kind = EPI_GATE_RES;
                g[j].out = x + int64_t(f[j]) * D;
                g[j].ldo = D;
                g[j].gate = mod + int64_t(runs[3 * (i + j) + 2]) * 6 * D + gate_at;
            }
            Stage t(c, stage);
            DIT_LAUNCH(c, launch_gemm2(a_base + int64_t(f[0]) * lda, wa.w, wa.scale, rows[0], g[0],
                                       a_base + int64_t(f[1]) * lda, wa.w, wa.scale, rows[1], g[1], wa.w8, D, K, st),
                       "gated product");
        }
        return DIT_OK;
    };
    DIT_TRY(norms(mod, DIT_ST_NORM1, c->h, b->norm_w[0]));
    GemmEpi e{};
    e.kind = EPI_QKV;
    e.q = c->q;
    e.k = c->k;
    e.vt = c->vt;
    e.heads = H;
    e.ldv = Sp;
    e.qn = b->norm_w[2];
    e.kn = b->norm_w[3];
    e.cos = cs;
    e.sin = sn;
    e.qk_eps = A.qk_eps;
    e.rows_total = Sk;
    DIT_TRY(prep(0, 3 * D, D));
    if (c->qk_fused) {
        Stage t(c, DIT_ST_QKV);
        DIT_LAUNCH(c, product(c->h, 0, S, 0, 3 * D, D, e), "qkv");
    } else {
        // the unfused arm: the projection stored in bf16 (the parallel
        // block's [o | a] buffer, unused by the sequential forms until the
        // sandwich norms' output product), then the q/k/v prep pass
        GemmEpi pe{};
        pe.kind = EPI_BF16;
        pe.act = c->oa;
        pe.ld_act = 3 * D;
        {
            Stage t(c, DIT_ST_QKV);
            DIT_LAUNCH(c, product(c->h, 0, S, 0, 3 * D, D, pe), "qkv");
        }
        Stage t(c, DIT_ST_QK_PREP);
        DIT_LAUNCH(c, launch_qk_prep(c->oa, S, H, Sk, b->norm_w[2], b->norm_w[3], cs, sn, A.qk_eps, c->q, c->k, c->vt, Sp, st),
                   "qk prep");
    }
    // the later weights' dequantisation starts once the QKV product is done:
    // it then shares the compute units with the attention
    DIT_TRY(fork_dequant());
    if (Sk > S) DIT_TRY(ref_copy(c, nullptr, slot, S, Sk, false));
    {
        Stage t(c, DIT_ST_ATTN);
        DIT_LAUNCH(c, launch_attention(c->q, c->k, c->vt, H, Sk, Sp, c->o, D, st, S), "attention");
    }
    DIT_TRY(gated(c->o, D, 1, D, 2 * D, DIT_ST_OUT, b->post_w[0]));
    DIT_TRY(norms(mod + 3 * D, DIT_ST_NORM2, c->h2, b->norm_w[1]));
    GemmEpi u{};
    u.kind = EPI_SWIGLU;
    u.act = c->a;
    DIT_TRY(prep(2, 2 * F, D));
    {
        Stage t(c, DIT_ST_UP);
        DIT_LAUNCH(c, product(c->h2, 0, S, 2, 2 * F, D, u), "up");
    }
    DIT_TRY(gated(c->a, F, 3, F, 5 * D, DIT_ST_DOWN, b->post_w[1]));
    return DIT_OK;
}

// The block forward ([GZ] Block.forward; validated arguments): one run of
// all rows on the one modulation row.
dit_status block_forward(dit_ctx *c, const dit_block *b, float *x, const float *vec, const float *cs,
                         const float *sn, int S, const float *pre_mod = nullptr) {
    const int32_t one[3] = {0, S, 0};
    return block_forward_runs(c, b, x, vec, 1, one, 1, cs, sn, S, 0, nullptr, pre_mod);
}

dit_status time_vector(dit_ctx *c, const uint16_t *w1, const uint16_t *w2, float t, float *vec) {
    const dit_arch &A = c->arch;
    hipStream_t st = c->stream;
    Stage tm(c, DIT_ST_TIME);
    DIT_LAUNCH(c, launch_time_embedding(t, A.time_dim, c->temb, st), "time embedding");
    DIT_LAUNCH(c, launch_gemv(w1, c->temb, A.hidden, A.time_dim, false, c->t1, st), "time mlp 1");
    DIT_LAUNCH(c, launch_gemv(w2, c->t1, A.hidden, A.hidden, true, vec, st), "time mlp 2");
    return DIT_OK;
}

// The DiT's time input for a step at sigma ([HC] s.6): the timestep
// sigma * 1000, divided by 1000 again, each an fp32 operation rounded on its
// own (equal to sigma on grids such as linspace(1, 0, n); after a shift the
// two can differ in the last bit).
#pragma clang fp contract(off)
float dit_time_input(float sigma) {
    const float ts = sigma * 1000.f;
    return ts / 1000.f;
}
#pragma clang fp contract(on)

dit_status check_model(dit_ctx *c, const dit_model *m) {
    if (!m) return fail(c, DIT_EINVAL, "model is NULL");
    if (m->n_blocks < 0 || m->n_blocks > 1024) return fail(c, DIT_ERANGE, "n_blocks %d outside 0..1024", m->n_blocks);
    if (m->n_blocks > 0 && !m->blocks) return fail(c, DIT_EINVAL, "model blocks array is NULL");
    if (!m->w_t1 || !m->w_t2 || !m->w_in || !m->w_txt || !m->w_fmod || !m->w_final)
        return fail(c, DIT_EINVAL, "a model weight pointer is NULL");
    for (int i = 0; i < m->n_blocks; ++i) DIT_TRY(check_block(c, &m->blocks[i], false, true));
    return DIT_OK;
}

// the steps a schedule may plan
constexpr int kMaxPlanSteps = 64;

// the weights a plan's rows are computed from, in a fixed order
std::vector<const void *> plan_keys_of(const dit_model *m) {
    std::vector<const void *> k = {m->w_t1, m->w_t2, m->w_fmod};
    for (int i = 0; i < m->n_blocks; ++i) k.push_back(m->blocks[i].w_mod);
    return k;
}

// the planned step of sigma (the same bits) for this model's weights, or -1
int plan_step(const dit_ctx *c, const dit_model *m, float sigma) {
    if (c->plan_n == 0 || c->plan_keys != plan_keys_of(m)) return -1;
    for (int i = 0; i < c->plan_n; ++i)
        if (std::memcmp(&c->plan_sig[i], &sigma, sizeof(float)) == 0) return i;
    return -1;
}

}  // namespace

extern "C" {

const char *dit_version(void) { return "libdit 0.1 (gfx950)"; }

const char *dit_last_error(const dit_ctx *ctx) {
    if (ctx) return ctx->err.c_str();
    return g_err.c_str();
}

dit_status dit_ctx_create(dit_ctx **out, int device, void *stream, const dit_arch *arch, int max_rows) {
    if (!out) return fail(nullptr, DIT_EINVAL, "out is NULL");
    *out = nullptr;
    DIT_TRY(validate_arch(arch));
    if (max_rows < 1 || max_rows > 65536) return fail(nullptr, DIT_ERANGE, "max_rows %d outside 1..65536", max_rows);
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0)
        return fail(nullptr, DIT_EDEVICE, "no HIP device available");
    if (device < 0 || device >= count) return fail(nullptr, DIT_EDEVICE, "device %d outside 0..%d", device, count - 1);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess)
        return fail(nullptr, DIT_EDEVICE, "cannot query device %d", device);
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(nullptr, DIT_EDEVICE, "device %d is %s; this library is built for gfx950", device, prop.gcnArchName);
    if (hipSetDevice(device) != hipSuccess) return fail(nullptr, DIT_EDEVICE, "hipSetDevice(%d) failed", device);

    dit_ctx *c = new (std::nothrow) dit_ctx();
    if (!c) return fail(nullptr, DIT_ENOMEM, "out of host memory");
    c->device = device;
    c->stream = static_cast<hipStream_t>(stream);
    c->arch = *arch;
    c->max_rows = max_rows;
    c->max_rows_pad = round_up(max_rows, 256);   // whole 256-row product tiles

    const size_t S = c->max_rows_pad, D = arch->hidden, F = arch->ffn, H = arch->heads;
    // h, h2, o, a: one more 256-row tile, read (not used) when the double-
    // stream block runs the image rows as a product starting at row L
    const size_t Sx = S + 256;
    const size_t sizes[] = {
        kMaxModRows * 6 * D * 4, D * 4, size_t(arch->time_dim) * 4, D * 4, 2 * D * 4,  // mod vec temb t1 fmod
        Sx * D * 2, Sx * D * 2,                                        // h h2
        H * S * 128 * 2, H * S * 128 * 2, H * 128 * S * 2,             // q k vt
        Sx * D * 2, Sx * F * 2,                                        // o a
        S * size_t(arch->latent) * 2, S * size_t(arch->text_dim) * 2,  // latb ctxb
        S * D * 4, S * size_t(arch->latent) * 4,                       // seq vel
        S * std::max(std::max((D + F) * 2, D * 4), D * 6),             // oa (yf, the unfused arm's qkv)
        Sx * std::max(D, F), Sx * 4,                                   // aq as
    };
    size_t off[sizeof sizes / sizeof sizes[0]];
    size_t total = 0;
    for (size_t i = 0; i < sizeof sizes / sizeof sizes[0]; ++i) {
        off[i] = total;
        total += (sizes[i] + 255) / 256 * 256;
    }
    if (hipMalloc(&c->pool, total) != hipSuccess) {
        delete c;
        return fail(nullptr, DIT_ENOMEM, "workspace allocation of %zu bytes failed", total);
    }
    c->pool_bytes = total;
    char *p = static_cast<char *>(c->pool);
    c->mod = reinterpret_cast<float *>(p + off[0]);
    c->vec = reinterpret_cast<float *>(p + off[1]);
    c->temb = reinterpret_cast<float *>(p + off[2]);
    c->t1 = reinterpret_cast<float *>(p + off[3]);
    c->fmod = reinterpret_cast<float *>(p + off[4]);
    c->h = reinterpret_cast<uint16_t *>(p + off[5]);
    c->h2 = reinterpret_cast<uint16_t *>(p + off[6]);
    c->q = reinterpret_cast<uint16_t *>(p + off[7]);
    c->k = reinterpret_cast<uint16_t *>(p + off[8]);
    c->vt = reinterpret_cast<uint16_t *>(p + off[9]);
    c->o = reinterpret_cast<uint16_t *>(p + off[10]);
    c->a = reinterpret_cast<uint16_t *>(p + off[11]);
    c->latb = reinterpret_cast<uint16_t *>(p + off[12]);
    c->ctxb = reinterpret_cast<uint16_t *>(p + off[13]);
    c->seq = reinterpret_cast<float *>(p + off[14]);
    c->vel = reinterpret_cast<float *>(p + off[15]);
    c->oa = reinterpret_cast<uint16_t *>(p + off[16]);
    c->yf = reinterpret_cast<float *>(p + off[16]);
    c->aq = reinterpret_cast<int8_t *>(p + off[17]);
    c->as = reinterpret_cast<float *>(p + off[18]);
    const size_t dbg[9] = {sizes[0], sizes[5], sizes[7], sizes[8], sizes[9], sizes[10], sizes[6], sizes[11], sizes[16]};
    for (int i = 0; i < 9; ++i) c->bytes[i] = dbg[i];
    *out = c;
    return DIT_OK;
}

void dit_ctx_destroy(dit_ctx *ctx) {
    if (!ctx) return;
    if (ctx->pool) {
        hipSetDevice(ctx->device);
        drop_records(ctx);
        for (hipEvent_t e : ctx->spare) hipEventDestroy(e);
        hipFree(ctx->pool);
        if (ctx->wdq) hipFree(ctx->wdq);
        if (ctx->plan_mem) hipFree(ctx->plan_mem);
        if (ctx->ev_fork) hipEventDestroy(ctx->ev_fork);
        for (hipEvent_t e : ctx->ev_ready)
            if (e) hipEventDestroy(e);
        if (ctx->side) hipStreamDestroy(ctx->side);
    }
    delete ctx;
}

dit_status dit_timing_enable(dit_ctx *ctx, int on) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    DIT_TRY(check_ctx(ctx));
    drop_records(ctx);
    ctx->timing = on != 0;
    return DIT_OK;
}

dit_status dit_timing_read(dit_ctx *ctx, double *ms, int64_t *count) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!ms || !count) return fail(ctx, DIT_EINVAL, "ms or count is NULL");
    DIT_TRY(check_ctx(ctx));
    for (int i = 0; i < DIT_NSTAGES; ++i) {
        ms[i] = 0.0;
        count[i] = 0;
    }
    dit_status st = DIT_OK;
    for (auto &r : ctx->recs) {
        float e = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&e, r.a, r.b) != hipSuccess) {
            st = fail(ctx, DIT_EDEVICE, "reading a timing event failed");
            break;
        }
        ms[r.stage] += e;
        count[r.stage] += 1;
    }
    drop_records(ctx);
    return st;
}

dit_status dit_ctx_set_stream(dit_ctx *ctx, void *stream) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    ctx->stream = static_cast<hipStream_t>(stream);
    return DIT_OK;
}

dit_status dit_positions(dit_ctx *ctx, int L, int h, int w, int32_t *pos) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!pos) return fail(ctx, DIT_EINVAL, "pos is NULL");
    if (L < 0 || h < 1 || w < 1) return fail(ctx, DIT_ERANGE, "L %d, h %d, w %d: need L >= 0, h, w >= 1", L, h, w);
    if (static_cast<int64_t>(h) * w + L > ctx->max_rows)
        return fail(ctx, DIT_ERANGE, "L + h*w exceeds max_rows %d", ctx->max_rows);
    DIT_TRY(check_ctx(ctx));
    DIT_LAUNCH(ctx, launch_positions(L, h, w, pos, ctx->stream), "positions");
    return DIT_OK;
}

dit_status dit_rope_tables(dit_ctx *ctx, const int32_t *pos, int S, float *cos_t, float *sin_t) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!pos || !cos_t || !sin_t) return fail(ctx, DIT_EINVAL, "pos, cos or sin is NULL");
    if (S < 1 || S > ctx->max_rows) return fail(ctx, DIT_ERANGE, "S = %d outside 1..%d", S, ctx->max_rows);
    DIT_TRY(check_ctx(ctx));
    const dit_arch &A = ctx->arch;
    DIT_LAUNCH(ctx, launch_rope_tables(pos, S, A.axes[0], A.axes[1], A.axes[2], A.rope_theta, cos_t, sin_t, ctx->stream),
               "rope tables");
    return DIT_OK;
}

dit_status dit_time_vector(dit_ctx *ctx, const uint16_t *w_t1, const uint16_t *w_t2, float t, float *vec) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!w_t1 || !w_t2 || !vec) return fail(ctx, DIT_EINVAL, "w_t1, w_t2 or vec is NULL");
    DIT_TRY(check_ctx(ctx));
    return time_vector(ctx, w_t1, w_t2, t, vec);
}

dit_status dit_modulation(dit_ctx *ctx, const uint16_t *w_mod, int chunks, const float *vec, float *mod) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!w_mod || !vec || !mod) return fail(ctx, DIT_EINVAL, "w_mod, vec or mod is NULL");
    if (chunks < 1 || chunks > 6) return fail(ctx, DIT_ERANGE, "chunks %d outside 1..6", chunks);
    DIT_TRY(check_ctx(ctx));
    const int D = ctx->arch.hidden;
    DIT_LAUNCH(ctx, launch_gemv(w_mod, vec, chunks * D, D, true, mod, ctx->stream), "modulation");
    return DIT_OK;
}

dit_status dit_modulated_norm(dit_ctx *ctx, const float *x, int rows, const float *shift, const float *scale,
                              const float *norm_w, float eps, uint16_t *out) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x || !shift || !scale || !out) return fail(ctx, DIT_EINVAL, "x, shift, scale or out is NULL");
    const bool rms = ctx->arch.norm == DIT_NORM_RMS;
    if (rms && !norm_w) return fail(ctx, DIT_EINVAL, "RMSNorm needs norm_w");
    if (rows < 1 || rows > ctx->max_rows) return fail(ctx, DIT_ERANGE, "rows %d outside 1..%d", rows, ctx->max_rows);
    if (!(eps > 0)) return fail(ctx, DIT_EINVAL, "eps must be positive");
    DIT_TRY(check_ctx(ctx));
    DIT_LAUNCH(ctx, launch_modnorm(x, rows, ctx->arch.hidden, shift, scale, norm_w, rms, eps, out, ctx->stream),
               "modulated norm");
    return DIT_OK;
}

dit_status dit_linear(dit_ctx *ctx, const uint16_t *a, const void *w, const uint16_t *scale, int wtype, int M, int N,
                      int K, float *out) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!a || !w || !out) return fail(ctx, DIT_EINVAL, "a, w or out is NULL");
    if (wtype != DIT_W_BF16 && wtype != DIT_W_INT8_B32) return fail(ctx, DIT_EINVAL, "unknown wtype %d", wtype);
    if (wtype == DIT_W_INT8_B32 && !scale) return fail(ctx, DIT_EINVAL, "int8 weight has no scales");
    if (wtype == DIT_W_BF16 && scale) return fail(ctx, DIT_EINVAL, "bf16 weight given scales");
    if (M < 1 || M > ctx->max_rows) return fail(ctx, DIT_ERANGE, "M %d outside 1..%d", M, ctx->max_rows);
    if (N < 64 || N % 64 || N > 65536) return fail(ctx, DIT_EINVAL, "N %d: must be a multiple of 64 in 64..65536", N);
    if (K < 64 || K % 64 || K > 65536) return fail(ctx, DIT_EINVAL, "K %d: must be a multiple of 64 in 64..65536", K);
    if (!aligned_to(a, 16) || !aligned_to(w, 16) || !aligned_to(scale, 4) || !aligned_to(out, 16))
        return fail(ctx, DIT_EINVAL, "a, w and out must be 16-byte and scale 4-byte aligned");
    DIT_TRY(check_ctx(ctx));
    GemmEpi e{};
    e.kind = EPI_F32;
    e.out = out;
    e.ldo = N;
    WeightArg wa{};
    const bool int8 = wtype == DIT_W_INT8_B32;
    if (int8 && !ctx->int8_in_product) DIT_TRY(ensure_wdq(ctx));
    // the largest slot of the first set
    int big = 0;
    for (int i = 1; i < 4; ++i)
        if (wdq_elems(ctx, i) > wdq_elems(ctx, big)) big = i;
    DIT_TRY(weight_arg_of(ctx, w, scale, int8, N, K, ctx->wdq ? wdq_slot(ctx, 0, big) : nullptr,
                          ctx->wdq ? wdq_elems(ctx, big) : 0, ctx->stream, &wa));
    DIT_LAUNCH(ctx, launch_gemm(a, wa.w, wa.scale, wa.w8, M, N, K, e, ctx->stream, false), "linear");
    return DIT_OK;
}

dit_status dit_sigma_schedule(const float *sample_sigmas, int n, float shift, float *sigmas, float *t) {
#pragma clang fp contract(off)
    if (!sample_sigmas || !sigmas || !t) return fail(nullptr, DIT_EINVAL, "sample_sigmas, sigmas or t is NULL");
    if (n < 1 || n > 10000) return fail(nullptr, DIT_ERANGE, "n = %d outside 1..10000", n);
    if (!(shift > 0.f) || !std::isfinite(shift)) return fail(nullptr, DIT_EINVAL, "shift must be positive and finite");
    for (int i = 0; i < n; ++i) {
        const float s0 = sample_sigmas[i];
        if (!(s0 >= 0.f && s0 <= 1.f)) return fail(nullptr, DIT_EINVAL, "sigma %d = %g outside [0, 1]", i, s0);
        // one float operation at a time, each rounded (no contraction)
        const float num = shift * s0;
        const float den = 1.f + (shift - 1.f) * s0;
        const float s = num / den;
        sigmas[i] = s;
        const float ts = s * 1000.f;
        t[i] = ts / 1000.f;
    }
    sigmas[n] = 0.f;
    return DIT_OK;
}

dit_status dit_set_qk_prep(dit_ctx *ctx, int fused) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (fused != 0 && fused != 1) return fail(ctx, DIT_EINVAL, "fused = %d is not 0 or 1", fused);
    ctx->qk_fused = fused != 0;
    return DIT_OK;
}

dit_status dit_set_int8_products(dit_ctx *ctx, int in_product) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (in_product != 0 && in_product != 1) return fail(ctx, DIT_EINVAL, "in_product = %d is not 0 or 1", in_product);
    ctx->int8_in_product = in_product != 0;
    return DIT_OK;
}

dit_status dit_qk_prep(dit_ctx *ctx, const uint16_t *qkv, int S, const float *q_norm, const float *k_norm,
                       const float *cos_t, const float *sin_t, uint16_t *q, uint16_t *k, uint16_t *vt) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!qkv || !q_norm || !k_norm || !cos_t || !sin_t || !q || !k || !vt)
        return fail(ctx, DIT_EINVAL, "qkv, q_norm, k_norm, cos, sin, q, k or vt is NULL");
    if (S < 1 || S > ctx->max_rows) return fail(ctx, DIT_ERANGE, "S %d outside 1..%d", S, ctx->max_rows);
    auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (!al16(qkv) || !al16(q_norm) || !al16(k_norm) || !al16(cos_t) || !al16(sin_t) || !al16(q) || !al16(k) || !al16(vt))
        return fail(ctx, DIT_EINVAL, "qkv, q_norm, k_norm, cos, sin, q, k and vt must be 16-byte aligned");
    DIT_TRY(check_ctx(ctx));
    const dit_arch &A = ctx->arch;
    Stage t(ctx, DIT_ST_QK_PREP);
    DIT_LAUNCH(ctx, launch_qk_prep(qkv, S, A.heads, S, q_norm, k_norm, cos_t, sin_t, A.qk_eps, q, k, vt, round_up(S, 64),
                                   ctx->stream),
               "qk prep");
    return DIT_OK;
}

dit_status dit_quantize_rows(dit_ctx *ctx, const uint16_t *x, int rows, int K, int8_t *q, float *s) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x || !q || !s) return fail(ctx, DIT_EINVAL, "x, q or s is NULL");
    if (rows < 1) return fail(ctx, DIT_ERANGE, "rows %d < 1", rows);
    if (K < 8 || K % 8 || K > 16384) return fail(ctx, DIT_EINVAL, "K %d: must be a multiple of 8 in 8..16384", K);
    DIT_TRY(check_ctx(ctx));
    DIT_LAUNCH(ctx, launch_quant_rows(x, rows, K, q, s, ctx->stream), "quantize rows");
    return DIT_OK;
}

dit_status dit_convrot_quantize_rows(dit_ctx *ctx, const uint16_t *x, int rows, int K, int8_t *q, float *s) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x || !q || !s) return fail(ctx, DIT_EINVAL, "x, q or s is NULL");
    if (rows < 1) return fail(ctx, DIT_ERANGE, "rows %d < 1", rows);
    if (K < 256 || K % 256 || K > 16384) return fail(ctx, DIT_EINVAL, "K %d: must be a multiple of 256 in 256..16384", K);
    DIT_TRY(check_ctx(ctx));
    DIT_LAUNCH(ctx, launch_quant_rows(x, rows, K, q, s, ctx->stream, true), "convrot quantize rows");
    return DIT_OK;
}

dit_status dit_modulated_norm_int8(dit_ctx *ctx, const float *x, int rows, const float *shift, const float *scale,
                                   const float *norm_w, float eps, int8_t *q, float *s) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x || !shift || !scale || !q || !s) return fail(ctx, DIT_EINVAL, "x, shift, scale, q or s is NULL");
    const bool rms = ctx->arch.norm == DIT_NORM_RMS;
    if (rms && !norm_w) return fail(ctx, DIT_EINVAL, "RMSNorm needs norm_w");
    if (rows < 1 || rows > ctx->max_rows) return fail(ctx, DIT_ERANGE, "rows %d outside 1..%d", rows, ctx->max_rows);
    if (!(eps > 0)) return fail(ctx, DIT_EINVAL, "eps must be positive");
    DIT_TRY(check_ctx(ctx));
    DIT_LAUNCH(ctx, launch_modnorm_i8(x, rows, ctx->arch.hidden, shift, scale, norm_w, rms, eps, q, s, ctx->stream),
               "modulated norm int8");
    return DIT_OK;
}

dit_status dit_linear_w8a8(dit_ctx *ctx, const int8_t *a, const float *a_scale, const int8_t *w, const float *w_scale,
                           int M, int N, int K, float *out) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!a || !a_scale || !w || !w_scale || !out) return fail(ctx, DIT_EINVAL, "a, a_scale, w, w_scale or out is NULL");
    if (M < 1 || M > ctx->max_rows) return fail(ctx, DIT_ERANGE, "M %d outside 1..%d", M, ctx->max_rows);
    if (N < 256 || N % 256 || N > 65536) return fail(ctx, DIT_EINVAL, "N %d: must be a multiple of 256 in 256..65536", N);
    const int Kmax = std::max(ctx->arch.hidden, ctx->arch.ffn);
    if (K < 128 || K % 128 || K > Kmax) return fail(ctx, DIT_EINVAL, "K %d: must be a multiple of 128 in 128..%d", K, Kmax);
    DIT_TRY(check_ctx(ctx));
    // the kernel reads A in whole 256-row tiles: the rows go to the
    // context's INT8 workspace, which has them
    if (hipMemcpyAsync(ctx->aq, a, static_cast<size_t>(M) * K, hipMemcpyDeviceToDevice, ctx->stream) != hipSuccess)
        return fail(ctx, DIT_EDEVICE, "copy of the INT8 rows failed");
    GemmEpi e{};
    e.kind = EPI_F32;
    e.out = out;
    e.ldo = N;
    DIT_LAUNCH(ctx, launch_gemm_w8a8(ctx->aq, a_scale, w, w_scale, M, N, K, e, ctx->stream), "linear w8a8");
    return DIT_OK;
}

dit_status dit_attention(dit_ctx *ctx, const uint16_t *q, const uint16_t *k, const uint16_t *vt, int heads, int S,
                         uint16_t *o) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!q || !k || !vt || !o) return fail(ctx, DIT_EINVAL, "q, k, vt or o is NULL");
    if (heads < 1 || heads > ctx->arch.heads) return fail(ctx, DIT_ERANGE, "heads %d outside 1..%d", heads, ctx->arch.heads);
    if (S < 1 || S > ctx->max_rows) return fail(ctx, DIT_ERANGE, "S %d outside 1..%d", S, ctx->max_rows);
    DIT_TRY(check_ctx(ctx));
    DIT_LAUNCH(ctx, launch_attention(q, k, vt, heads, S, round_up(S, 64), o, heads * 128, ctx->stream), "attention");
    return DIT_OK;
}

dit_status dit_block_forward(dit_ctx *ctx, const dit_block *b, float *x, const float *vec, const float *cos_t,
                             const float *sin_t, int L, int N) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x || !vec || !cos_t || !sin_t) return fail(ctx, DIT_EINVAL, "x, vec, cos or sin is NULL");
    if (!aligned_to(x, 16)) return fail(ctx, DIT_EINVAL, "x must be 16-byte aligned");
    DIT_TRY(check_block(ctx, b, false, true));
    DIT_TRY(check_rows(ctx, L, N));
    DIT_TRY(check_ctx(ctx));
    return block_forward(ctx, b, x, vec, cos_t, sin_t, L + N);
}

dit_status dit_parallel_block_forward(dit_ctx *ctx, const dit_block *b, float *x, const float *vec,
                                      const float *cos_t, const float *sin_t, int L, int N) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x || !vec || !cos_t || !sin_t) return fail(ctx, DIT_EINVAL, "x, vec, cos or sin is NULL");
    if (!aligned_to(x, 16)) return fail(ctx, DIT_EINVAL, "x must be 16-byte aligned");
    DIT_TRY(check_block(ctx, b, true));
    DIT_TRY(check_rows(ctx, L, N));
    DIT_TRY(check_ctx(ctx));
    return parallel_block_forward(ctx, b, x, vec, cos_t, sin_t, L + N);
}

dit_status dit_block_forward_runs(dit_ctx *ctx, const dit_block *b, float *x, const float *vecs, int R,
                                  const int32_t *runs, int n_runs, const float *cos_t, const float *sin_t, int L,
                                  int N) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x || !vecs || !runs || !cos_t || !sin_t) return fail(ctx, DIT_EINVAL, "x, vecs, runs, cos or sin is NULL");
    if (!aligned_to(x, 16)) return fail(ctx, DIT_EINVAL, "x must be 16-byte aligned");
    DIT_TRY(check_block(ctx, b, false, true));
    DIT_TRY(check_rows(ctx, L, N));
    if (R < 1 || R > kMaxModRows) return fail(ctx, DIT_ERANGE, "R = %d outside 1..%d", R, kMaxModRows);
    if (n_runs < 1 || n_runs > L + N) return fail(ctx, DIT_ERANGE, "n_runs = %d outside 1..%d", n_runs, L + N);
    int end = 0;
    for (int i = 0; i < n_runs; ++i) {
        const int f = runs[3 * i], e = runs[3 * i + 1], m = runs[3 * i + 2];
        if (f != end || e <= f) return fail(ctx, DIT_EINVAL, "run %d = (%d, %d) does not continue the runs at %d", i, f, e, end);
        if (m < 0 || m >= R) return fail(ctx, DIT_ERANGE, "run %d uses modulation row %d outside 0..%d", i, m, R - 1);
        end = e;
    }
    if (end != L + N) return fail(ctx, DIT_EINVAL, "runs end at %d, not at L + N = %d", end, L + N);
    DIT_TRY(check_ctx(ctx));
    return block_forward_runs(ctx, b, x, vecs, R, runs, n_runs, cos_t, sin_t, L + N);
}

dit_status dit_block_forward_cached(dit_ctx *ctx, const dit_block *b, float *x, const float *vec, const float *cos_t,
                                   const float *sin_t, int L, int N, int first, uint16_t *slot, int record) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x || !vec || !cos_t || !sin_t) return fail(ctx, DIT_EINVAL, "x, vec, cos or sin is NULL");
    if (!aligned_to(x, 16)) return fail(ctx, DIT_EINVAL, "x must be 16-byte aligned");
    DIT_TRY(check_block(ctx, b, false, true));
    DIT_TRY(check_rows(ctx, L, N));
    const int S = L + N;
    if (first < 1 || first > S) return fail(ctx, DIT_ERANGE, "first = %d outside 1..%d", first, S);
    if (first < S && !slot) return fail(ctx, DIT_EINVAL, "slot is NULL with %d reference rows", S - first);
    if (record != 0 && record != 1) return fail(ctx, DIT_EINVAL, "record = %d is not 0 or 1", record);
    DIT_TRY(check_ctx(ctx));
    if (record) {
        DIT_TRY(block_forward(ctx, b, x, vec, cos_t, sin_t, S));
        return ref_copy(ctx, slot, nullptr, first, S, true);
    }
    const int32_t one[3] = {0, first, 0};
    return block_forward_runs(ctx, b, x, vec, 1, one, 1, cos_t, sin_t, first, S, slot);
}

dit_status dit_double_block_forward(dit_ctx *ctx, const dit_block *txt, const dit_block *img, float *x,
                                    const float *vec, const float *cos_t, const float *sin_t, int L, int N) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x || !vec || !cos_t || !sin_t) return fail(ctx, DIT_EINVAL, "x, vec, cos or sin is NULL");
    if (!aligned_to(x, 16)) return fail(ctx, DIT_EINVAL, "x must be 16-byte aligned");
    DIT_TRY(check_block(ctx, txt));
    DIT_TRY(check_block(ctx, img));
    DIT_TRY(check_rows(ctx, L, N));
    DIT_TRY(check_ctx(ctx));
    return double_block_forward(ctx, txt, img, x, vec, cos_t, sin_t, L, N);
}

dit_status dit_prologue(dit_ctx *ctx, const dit_model *m, const float *ctx_feats, int L, float *txt) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!ctx_feats || !txt) return fail(ctx, DIT_EINVAL, "ctx_feats or txt is NULL");
    DIT_TRY(check_model(ctx, m));
    if (L < 1 || L > 512 || L > ctx->max_rows) return fail(ctx, DIT_ERANGE, "L = %d outside 1..512", L);
    DIT_TRY(check_ctx(ctx));
    const dit_arch &A = ctx->arch;
    Stage tm(ctx, DIT_ST_TXT_IN);
    DIT_LAUNCH(ctx, launch_to_bf16(ctx_feats, static_cast<int64_t>(L) * A.text_dim, ctx->ctxb, ctx->stream), "to bf16");
    GemmEpi e{};
    e.kind = EPI_F32;
    e.out = txt;
    e.ldo = A.hidden;
    DIT_LAUNCH(ctx, launch_gemm(ctx->ctxb, m->w_txt, nullptr, false, L, A.hidden, A.text_dim, e, ctx->stream, true), "txt_in");
    return DIT_OK;
}

dit_status dit_denoise_step(dit_ctx *ctx, const dit_model *m, float *x_lat, const float *txt, const float *cos_t,
                            const float *sin_t, int L, int N, float sigma, float sigma_next, float *vel_out) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!x_lat || !cos_t || !sin_t || (L > 0 && !txt)) return fail(ctx, DIT_EINVAL, "x_lat, txt, cos or sin is NULL");
    DIT_TRY(check_model(ctx, m));
    DIT_TRY(check_rows(ctx, L, N));
    DIT_TRY(check_ctx(ctx));
    const dit_arch &A = ctx->arch;
    const int D = A.hidden, S = L + N, lat = A.latent;
    hipStream_t st = ctx->stream;

    // a planned step takes its modulation rows from the plan
    const int pi = plan_step(ctx, m, sigma);
    if (pi < 0) DIT_TRY(time_vector(ctx, m->w_t1, m->w_t2, dit_time_input(sigma), ctx->vec));
    {
        Stage tm(ctx, DIT_ST_IMG_IN);
        if (L > 0 &&
            hipMemcpyAsync(ctx->seq, txt, static_cast<size_t>(L) * D * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
            return fail(ctx, DIT_EDEVICE, "copy of text rows failed");
        DIT_LAUNCH(ctx, launch_to_bf16(x_lat, static_cast<int64_t>(N) * lat, ctx->latb, st), "latent to bf16");
        GemmEpi e{};
        e.kind = EPI_F32;
        e.out = ctx->seq + static_cast<size_t>(L) * D;
        e.ldo = D;
        DIT_LAUNCH(ctx, launch_gemm(ctx->latb, m->w_in, nullptr, false, N, D, lat, e, st, true), "img_in");
    }
    for (int i = 0; i < m->n_blocks; ++i)
        DIT_TRY(block_forward(ctx, &m->blocks[i], ctx->seq, ctx->vec, cos_t, sin_t, S,
                              pi < 0 ? nullptr : ctx->plan_mod + (int64_t(pi) * m->n_blocks + i) * 6 * D));
    {
        Stage tm(ctx, DIT_ST_FINAL);
        const float *fm = pi < 0 ? ctx->fmod : ctx->plan_fmod + int64_t(pi) * 2 * D;
        if (pi < 0) DIT_LAUNCH(ctx, launch_gemv(m->w_fmod, ctx->vec, 2 * D, D, true, ctx->fmod, st), "final modulation");
        DIT_LAUNCH(ctx, launch_modnorm(ctx->seq + static_cast<size_t>(L) * D, N, D, fm, fm + D, nullptr,
                                       false, A.final_eps, ctx->h, st),
                   "final norm");
        GemmEpi f{};
        f.kind = EPI_F32;
        f.out = ctx->vel;
        f.ldo = lat;
        DIT_LAUNCH(ctx, launch_gemm(ctx->h, m->w_final, nullptr, false, N, lat, D, f, st, true), "final linear");
    }
    {
        Stage tm(ctx, DIT_ST_EULER);
        const float dt = sigma_next - sigma;
        DIT_LAUNCH(ctx, launch_euler(x_lat, ctx->vel, static_cast<int64_t>(N) * lat, dt, st), "euler");
        if (vel_out && hipMemcpyAsync(vel_out, ctx->vel, static_cast<size_t>(N) * lat * 4, hipMemcpyDeviceToDevice,
                                      st) != hipSuccess)
            return fail(ctx, DIT_EDEVICE, "copy of the velocity failed");
    }
    return DIT_OK;
}

dit_status dit_plan_schedule(dit_ctx *ctx, const dit_model *m, const float *sigmas, int n) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (n < 0 || n > kMaxPlanSteps) return fail(ctx, DIT_ERANGE, "n = %d outside 0..%d", n, kMaxPlanSteps);
    if (n > 0 && !sigmas) return fail(ctx, DIT_EINVAL, "sigmas is NULL");
    DIT_TRY(check_ctx(ctx));
    // whatever happens below, the old plan is gone
    ctx->plan_n = 0;
    ctx->plan_sig.clear();
    ctx->plan_keys.clear();
    if (n == 0) return DIT_OK;
    DIT_TRY(check_model(ctx, m));
    for (int i = 0; i < n; ++i)
        if (!std::isfinite(sigmas[i])) return fail(ctx, DIT_ERANGE, "sigmas[%d] is not finite", i);
    const int D = ctx->arch.hidden, nb = m->n_blocks;
    hipStream_t st = ctx->stream;
    const size_t need = (size_t(n) * D + size_t(n) * nb * 6 * D + size_t(n) * 2 * D) * sizeof(float);
    if (need > ctx->plan_bytes) {
        // earlier steps may still read the old rows
        if (hipStreamSynchronize(st) != hipSuccess) return fail(ctx, DIT_EDEVICE, "stream synchronize failed");
        if (ctx->plan_mem) hipFree(ctx->plan_mem);
        ctx->plan_mem = nullptr;
        ctx->plan_bytes = 0;
        void *p = nullptr;
        if (hipMalloc(&p, need) != hipSuccess) return fail(ctx, DIT_ENOMEM, "plan of %zu bytes failed", need);
        ctx->plan_mem = static_cast<float *>(p);
        ctx->plan_bytes = need;
    }
    ctx->plan_vec = ctx->plan_mem;
    ctx->plan_mod = ctx->plan_vec + size_t(n) * D;
    ctx->plan_fmod = ctx->plan_mod + size_t(n) * nb * 6 * D;
    for (int i = 0; i < n; ++i)
        DIT_TRY(time_vector(ctx, m->w_t1, m->w_t2, dit_time_input(sigmas[i]), ctx->plan_vec + int64_t(i) * D));
    // each weight read once for up to four steps
    for (int i0 = 0; i0 < n; i0 += 4) {
        const int nv = std::min(4, n - i0);
        const float *vec = ctx->plan_vec + int64_t(i0) * D;
        {
            Stage tm(ctx, DIT_ST_MOD);
            for (int b = 0; b < nb; ++b)
                DIT_LAUNCH(ctx, launch_gemv_multi(m->blocks[b].w_mod, vec, D, nv, 6 * D, D, true,
                                                  ctx->plan_mod + (int64_t(i0) * nb + b) * 6 * D, int64_t(nb) * 6 * D, st),
                           "planned modulation");
        }
        Stage tm(ctx, DIT_ST_FINAL);
        DIT_LAUNCH(ctx, launch_gemv_multi(m->w_fmod, vec, D, nv, 2 * D, D, true, ctx->plan_fmod + int64_t(i0) * 2 * D,
                                          2 * D, st),
                   "planned final modulation");
    }
    ctx->plan_sig.assign(sigmas, sigmas + n);
    ctx->plan_keys = plan_keys_of(m);
    ctx->plan_n = n;
    return DIT_OK;
}

dit_status dit_euler_step(dit_ctx *ctx, float *x, const float *v, int64_t n, float sigma, float sigma_next) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (n < 0) return fail(ctx, DIT_ERANGE, "n = %lld is negative", static_cast<long long>(n));
    if (n > 0 && (!x || !v)) return fail(ctx, DIT_EINVAL, "x or v is NULL");
    DIT_TRY(check_ctx(ctx));
    const float dt = sigma_next - sigma;
    DIT_LAUNCH(ctx, launch_euler(x, v, n, dt, ctx->stream), "euler");
    return DIT_OK;
}

dit_status dit_dequant_int8_b32(dit_ctx *ctx, const int8_t *q, const uint16_t *s, int out, int in, float *w_out) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (!q || !s || !w_out) return fail(ctx, DIT_EINVAL, "q, s or w_out is NULL");
    if (out < 1 || in < 32) return fail(ctx, DIT_ERANGE, "out %d, in %d: need out >= 1, in >= 32", out, in);
    if (in % 32) return fail(ctx, DIT_EINVAL, "in = %d is not a multiple of 32", in);
    DIT_TRY(check_ctx(ctx));
    DIT_LAUNCH(ctx, launch_dequant(q, s, out, in, w_out, ctx->stream), "dequant");
    return DIT_OK;
}

dit_status dit_debug_copy(dit_ctx *ctx, int which, void *dst, int64_t bytes) {
    if (!ctx) return fail(nullptr, DIT_EINVAL, "context is NULL");
    if (which < 0 || which > 8) return fail(ctx, DIT_ERANGE, "buffer %d outside 0..8", which);
    if (bytes <= 0) return DIT_OK;
    if (!dst) return fail(ctx, DIT_EINVAL, "dst is NULL");
    if (static_cast<size_t>(bytes) > ctx->bytes[which])
        return fail(ctx, DIT_ERANGE, "%lld bytes exceed buffer %d (%zu bytes)", static_cast<long long>(bytes), which,
                    ctx->bytes[which]);
    DIT_TRY(check_ctx(ctx));
    const void *p[9] = {ctx->mod, ctx->h, ctx->q, ctx->k, ctx->vt, ctx->o, ctx->h2, ctx->a, ctx->oa};
    if (hipMemcpyAsync(dst, p[which], static_cast<size_t>(bytes), hipMemcpyDeviceToDevice, ctx->stream) != hipSuccess)
        return fail(ctx, DIT_EDEVICE, "debug copy failed");
    return DIT_OK;
}

}  // extern "C"
