/*
 * dit.h -- C ABI of libdit, the gfx950 (MI355X) hot path of an AdaLN
 * diffusion-transformer (DiT) block and its few-step Euler denoise loop.
 *
 * Sources (web pages, cited by title and section):
 *   [HC] "Host contract -- RGBA-Image-2.1-Turbo (Core AI port of
 *        Qwen-Image-2.1-Turbo)": s.1 The graphs, s.4 Sequence layout and
 *        RoPE, s.6 Sampler.
 *   [K4] "944 -> 346 ms: optimizing FLUX.2 klein-4B on one TPU v6e chip":
 *        s.2 cast points, s.4.1 device-resident weights, s.4.3 flash
 *        attention, s.4.4 fused qk-prep.
 *   [GZ] "gizai:dit" module reference: Arch, Block, Modulation, Sequence,
 *        Work, gluRows, gatedInto, normedInto, prepOf, sinusoids,
 *        Block.forward, Block.parallel, runsOf, gatedInto, RefSlot,
 *        Sequence.active, HEAD, CHUNK.
 *
 * Conventions (all entry points):
 *  - Every tensor argument is a DEVICE pointer to caller-owned memory on the
 *    context's device, row-major and densely packed, unless stated otherwise.
 *    The library never frees caller memory and keeps no pointer after a call
 *    returns ([K4] s.4.1: weights stay resident; nothing is copied from the
 *    host inside a call).
 *  - bf16 tensors are passed as `const uint16_t *` holding bf16 bit patterns.
 *  - Every call only enqueues work on the context's HIP stream and returns;
 *    there is no host synchronisation inside a call.  Results are visible
 *    after the caller synchronises that stream.  Device faults surface at the
 *    caller's next synchronisation.
 *  - Arguments are validated on the host BEFORE any device work; a non-OK
 *    status means nothing was enqueued, and dit_last_error() describes it.
 *  - One context per stream; a context is not safe to use from two threads
 *    at once.  Calls on one context share its workspace, so they must be
 *    ordered on its stream (they are, when issued from one thread).
 */
#ifndef DIT_H
#define DIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dit_ctx dit_ctx;

typedef enum {
    DIT_OK = 0,
    DIT_EINVAL = -1,        /* null pointer, inconsistent shape, bad enum */
    DIT_ERANGE = -2,        /* a size outside its supported range */
    DIT_ENOMEM = -3,        /* workspace allocation failed */
    DIT_EDEVICE = -4,       /* no usable gfx950 device, or a launch failed */
    DIT_EUNSUPPORTED = -5   /* valid but not implemented (e.g. head_dim != 128) */
} dit_status;

/* Weight storage of the four block linears ([HC] s.1: bf16, or int8 with
 * one bf16 scale per block of 32 along the input axis). */
typedef enum { DIT_W_BF16 = 0, DIT_W_INT8_B32 = 1, DIT_W_INT8_ROW = 2, DIT_W_INT8_ROT = 3 } dit_wtype;

/* Norm before attention and MLP: LayerNorm without affine, or RMSNorm times
 * a per-feature weight ([GZ] normedInto; Block.parallel's modulated LayerNorm). */
typedef enum { DIT_NORM_LAYER = 0, DIT_NORM_RMS = 1 } dit_norm;

/* Architecture ([GZ] Arch).  Supported: head_dim == 128 ([GZ] HEAD),
 * hidden == heads * head_dim, hidden and ffn multiples of 256,
 * axes[0] + axes[1] + axes[2] == head_dim with every axis even
 * ([HC] s.4: 16, 56, 56), time_dim even, latent and text_dim multiples of 64. */
typedef struct {
    int32_t hidden;         /* D, e.g. 3072 */
    int32_t heads;          /* H, e.g. 24 */
    int32_t head_dim;       /* 128 */
    int32_t ffn;            /* F, SwiGLU width, e.g. 12288 */
    int32_t axes[3];        /* rotary axis widths (frame, height, width) */
    float eps;              /* modulated-norm epsilon */
    float qk_eps;           /* head RMSNorm epsilon */
    float final_eps;        /* final-layer norm epsilon */
    float rope_theta;       /* 10000 */
    int32_t norm;           /* dit_norm */
    int32_t time_dim;       /* sinusoid width, 256 */
    int32_t latent;         /* latent channels per image token, 64 */
    int32_t text_dim;       /* text feature width, 4096 */
} dit_arch;

/* One block's weights ([GZ] Block; linears stored [out, in]).
 *   w[0] QKV  [3*H*hd, D]  rows: all queries, all keys, all values; head j
 *                          of each is rows j*hd .. (j+1)*hd-1
 *   w[1] OUT  [D, H*hd]
 *   w[2] UP   [2F, D]      gate j at row 2j, up j at row 2j+1 ([GZ] gluRows)
 *   w[3] DOWN [D, F]
 * wtype DIT_W_BF16: w[i] are bf16; scale[i] must be NULL.
 * wtype DIT_W_INT8_B32: w[i] are int8 [out, in]; scale[i] are bf16
 *   [out, in/32]; weight = code * scale[o][k/32], which the products take
 *   rounded to bf16 (nearest even): by default dequantised by a pass of
 *   its own into a context scratch buffer just before each product (see
 *   dit_set_int8_products).
 * wtype DIT_W_INT8_ROW (W8A8 with per-token activations and per-output
 *   weights, [K4] Appendix B D4): w[i] are int8 [out, in], scale[i] fp32
 *   [out]; weight = code * scale[o].  Each product's input rows are taken
 *   to INT8 with one scale a row (s = max|row| / 127, codes rint(v * 127 /
 *   max|row|)), fused into the modulated norm for QKV and UP; the int32
 *   sums times both scales.  Only the sequential forms take it (ffn up to
 *   16384); cos and sin must then be 16-byte aligned (the INT8 products
 *   have no unaligned fallback: DIT_EDEVICE).
 * wtype DIT_W_INT8_ROT ([GZ] linearInto, quantizedOf, Block.quantized:
 *   ConvRot): as DIT_W_INT8_ROW with the INT8 rows stored in the rotated
 *   basis -- every 256 consecutive inputs of a product's input row are
 *   rotated by the regular (Sylvester-order) Hadamard of 256, scaled by
 *   1/16, before the row is quantized; the weights of the unrotated input
 *   are code * scale times that rotation ([GZ] Block.dequantized).
 * norm_w: fp32.  [0] NORM1, [1] NORM2 ([D], required for DIT_NORM_RMS,
 *   ignored for DIT_NORM_LAYER), [2] Q_NORM, [3] K_NORM ([hd], required).
 * w_mod: bf16 [6D, D]; its output rows are shift, scale, gate of the
 *   attention, then of the MLP ([GZ] Modulation).
 * post_w: fp32 [D] or NULL.  A sandwich block ([GZ] POST_ATTN, POST_MLP)
 *   sets both: [0] after the attention, [1] after the MLP; each half's
 *   product output row is normed (the arch's norm kind and eps, times the
 *   weight) before its gate.  Both NULL: the gated outputs are added as
 *   they are.  Only the sequential forms (dit_block_forward,
 *   dit_block_forward_runs, the blocks of dit_denoise_step) take them.
 * Alignment: w[i], w_mod, norm_w[i] and post_w[i] 16-byte aligned,
 *   scale[i] 4-byte aligned, and the block forms' x 16-byte aligned
 *   (DIT_EINVAL otherwise; the kernels read them in 16- and 4-byte
 *   pieces). */
typedef struct {
    int32_t wtype;
    const void *w[4];
    const void *scale[4];
    const float *norm_w[4];
    const uint16_t *w_mod;
    const float *post_w[2];
} dit_block;

/* The whole DiT ([HC] s.1 DiT graph).  All bf16 [out, in]:
 *   w_t1 [D, time_dim], w_t2 [D, D]   time MLP (silu between)
 *   w_in [D, latent]                  image tokens in
 *   w_txt [D, text_dim]               text features in
 *   w_fmod [2D, D]                    final (shift, scale)
 *   w_final [latent, D]               final linear
 * blocks: HOST array of n_blocks descriptors (device weight pointers). */
typedef struct {
    int32_t n_blocks;
    const dit_block *blocks;
    const uint16_t *w_t1, *w_t2, *w_in, *w_txt, *w_fmod, *w_final;
} dit_model;

/* Create a context on `device` whose calls enqueue on `stream` (a
 * hipStream_t; NULL = the device's null stream).  The workspace ([GZ] Work)
 * is allocated here once, sized for sequences of up to `max_rows` rows
 * (L + N), and reused by every call.  Errors: DIT_EINVAL (null out, bad
 * arch), DIT_EUNSUPPORTED (head_dim != 128 and the like), DIT_ERANGE
 * (max_rows outside 1..65536), DIT_EDEVICE (no such device, or it is not
 * gfx950), DIT_ENOMEM.  On error *out is NULL and the message is available
 * from dit_last_error(NULL). */
dit_status dit_ctx_create(dit_ctx **out, int device, void *stream, const dit_arch *arch,
                          int max_rows);

/* Free the workspace and the context.  NULL is a no-op.  The caller must
 * synchronise the stream first if calls are still in flight. */
void dit_ctx_destroy(dit_ctx *ctx);

/* Change the stream later calls enqueue on.  Work already enqueued on the
 * previous stream (which uses the context's workspace, and a planned
 * schedule's rows) is not waited for: the caller orders the two streams,
 * e.g. by synchronising the old one, before calls on the new one. */
dit_status dit_ctx_set_stream(dit_ctx *ctx, void *stream);

/* Text of the last non-OK status on this context (or of the last failed
 * dit_ctx_create / null-context call when ctx is NULL).  Never NULL. */
const char *dit_last_error(const dit_ctx *ctx);

/* Library version string. */
const char *dit_version(void);

/* [HC] s.4 positions: pos [L + h*w, 3] int32 device.  Text token i ->
 * (i, i, i); image token y*w + x -> (L, y - (h - h/2), x - (w - w/2)).
 * Requires 0 <= L, 1 <= h, 1 <= w, L + h*w <= max_rows. */
dit_status dit_positions(dit_ctx *ctx, int L, int h, int w, int32_t *pos);

/* [HC] s.4 rotary tables from positions pos [S, 3] int32: for each axis a
 * of width d_a, angles pos[:, a] * theta^(-2j/d_a), j < d_a/2; a token's
 * row is the three axes' rows concatenated (head_dim/2 values).
 * cos, sin: fp32 [S, head_dim/2] outputs (angle and cos/sin taken in fp64,
 * rounded once to fp32).  Requires 1 <= S <= max_rows. */
dit_status dit_rope_tables(dit_ctx *ctx, const int32_t *pos, int S, float *cos, float *sin);

/* Conditioning vector ([GZ] sinusoids + the time MLP): vec = w_t2 *
 * silu(w_t1 * [cos | sin](1000 t * 10000^(-i/(time_dim/2)))).
 * w_t1 bf16 [D, time_dim], w_t2 bf16 [D, D]; vec fp32 [D] output. */
dit_status dit_time_vector(dit_ctx *ctx, const uint16_t *w_t1, const uint16_t *w_t2, float t,
                           float *vec);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * conditioning vector of dit_time_vector with no context.  Same kernels
 * and result as dit_time_vector (bit for bit) for an arch with these hidden
 * and time_dim, on the calling thread's current device, enqueued on
 * `stream` (a hipStream_t of that device; NULL = its null stream).
 * w_t1 bf16 [hidden, time_dim], w_t2 bf16 [hidden, hidden], vec fp32
 * [hidden] output, all caller-owned device memory.  The two intermediate
 * rows live in a fixed device array of the library, 2 * 4096 floats per
 * device (held until the process ends): hidden and time_dim must each be a
 * multiple of 8 in 8..4096, else DIT_ERANGE.  Nothing in it must start at
 * zero.  Calls that overlap on one device (other streams, other threads)
 * race on that array; order them.  The first call on a device looks the
 * array's address up (hipGetSymbolAddress) and keeps it: make that call
 * before capturing.  Allocates nothing.  Errors: DIT_EINVAL (NULL pointer),
 * DIT_ERANGE, DIT_EDEVICE (no current device, lookup or launch failed);
 * message in dit_last_error(NULL). */
dit_status dit_time_vector_noalloc(void *stream, int hidden, int time_dim, const uint16_t *w_t1,
                                   const uint16_t *w_t2, float t, float *vec);

/* Modulation GEMV ([GZ] Modulation): mod = w_mod * silu(vec), w_mod bf16
 * [chunks*D, D], vec fp32 [D], mod fp32 [chunks*D].  chunks in 1..6. */
dit_status dit_modulation(dit_ctx *ctx, const uint16_t *w_mod, int chunks, const float *vec,
                          float *mod);

/* Modulated norm ([GZ] normedInto): out[r] = bf16(norm(x[r]) * (1 + scale)
 * + shift) for r < rows; norm is the arch's (norm_w fp32 [D] for RMS, may
 * be NULL for LayerNorm); x fp32 [rows, D]; shift, scale fp32 [D];
 * out bf16 [rows, D]; eps as given. */
dit_status dit_modulated_norm(dit_ctx *ctx, const float *x, int rows, const float *shift,
                              const float *scale, const float *norm_w, float eps,
                              uint16_t *out);

/* Plain product out = a * W^T ([GZ] linearInto): a bf16 [M, K]; W bf16
 * [N, K] (wtype DIT_W_BF16, scale NULL) or int8 [N, K] with bf16 scales
 * [N, K/32] (DIT_W_INT8_B32); out fp32 [M, N].  K a multiple of 64,
 * N a multiple of 64, 1 <= M <= max_rows; a, W and out 16-byte aligned,
 * the scales 4-byte aligned (DIT_EINVAL otherwise). */
dit_status dit_linear(dit_ctx *ctx, const uint16_t *a, const void *w, const uint16_t *scale,
                      int wtype, int M, int N, int K, float *out);

/* The sampler's grid ([HC] s.6, FlowMatch Euler with a fixed grid), host
 * memory, no context: for the n given sigmas s in [0, 1], sigmas[i] =
 * shift*s / (1 + (shift - 1)*s) and the DiT time input t[i] = (sigmas[i] *
 * 1000) / 1000, every step one rounded fp32 operation; sigmas[n] = 0 (the
 * grid holds n + 1 values, t n).  Step i runs dit_denoise_step with
 * sigma = sigmas[i] and sigma_next = sigmas[i+1]; that step's time input is
 * t[i], computed from sigma the same way.  DIT_EINVAL for NULL pointers, a shift
 * that is not positive and finite or a sigma outside [0, 1]; DIT_ERANGE
 * for n outside 1..10000.  dit_last_error(NULL) holds the message. */
dit_status dit_sigma_schedule(const float *sample_sigmas, int n, float shift, float *sigmas, float *t);

/* INT8 rows ([GZ] quantizedOf; [K4] Appendix B D4 per-token quantization):
 * x bf16 [rows, K] -> q int8 [rows, K] and s fp32 [rows] with, per row,
 * amax = max|x|, s = amax / 127 and q = clamp(rint(x * (127 / amax)),
 * -127, 127), each step one correctly rounded fp32 operation (an all-zero
 * row: s = 0, q = 0).  K a multiple of 8, at most 16384. */
dit_status dit_quantize_rows(dit_ctx *ctx, const uint16_t *x, int rows, int K, int8_t *q, float *s);

/* ConvRot then INT8 rows ([GZ] linearInto, quantizedOf): x bf16 [rows, K]
 * -> each 256 consecutive values y = R x with R the regular Hadamard of 256
 * (Sylvester order, entries +-1/16), in fp32 -> q int8 [rows, K] and s fp32
 * [rows] quantized as dit_quantize_rows quantizes.  K a multiple of 256, at
 * most 16384. */
dit_status dit_convrot_quantize_rows(dit_ctx *ctx, const uint16_t *x, int rows, int K, int8_t *q, float *s);

/* dit_modulated_norm with its output rows as INT8 codes q [rows, D] and a
 * scale a row s [rows], quantized as dit_quantize_rows quantizes (from the
 * fp32 norm output, in the same pass: [GZ] normedInto, INT8 rows). */
dit_status dit_modulated_norm_int8(dit_ctx *ctx, const float *x, int rows, const float *shift,
                                   const float *scale, const float *norm_w, float eps, int8_t *q, float *s);

/* W8A8 product ([GZ] linear): out[m][n] = (sum_k a[m][k] w[n][k]) *
 * a_scale[m] * w_scale[n] in fp32, int32 sums on the INT8 matrix cores.
 * a int8 [M, K], a_scale fp32 [M], w int8 [N, K], w_scale fp32 [N], out
 * fp32 [M, N]; 1 <= M <= max_rows, N a multiple of 256, K a multiple of
 * 128 up to max(hidden, ffn). */
dit_status dit_linear_w8a8(dit_ctx *ctx, const int8_t *a, const float *a_scale, const int8_t *w,
                           const float *w_scale, int M, int N, int K, float *out);

/* The q/k/v preparation as a pass of its own ([K4] s.4.4 runs it as a
 * separate kernel over the stored projection; [GZ] prepOf): qkv bf16
 * [S, 3*H*128] (the QKV product's output: all queries, all keys, all
 * values, head j of each at columns j*128..) -> q, k bf16 [H, S, 128], each
 * 128-wide head RMS-normed (fp32 statistics, the arch's qk_eps) times
 * q_norm / k_norm [128] fp32 and turned by the adjacent-pair rotation with
 * cos/sin [S, 64] fp32; vt bf16 [H, 128, Sp] the value heads transposed
 * (Sp = S rounded up to 64; columns S..Sp-1 are not written).  H = the
 * arch's heads; all pointers 16-byte aligned; 1 <= S <= max_rows. */
dit_status dit_qk_prep(dit_ctx *ctx, const uint16_t *qkv, int S, const float *q_norm, const float *k_norm,
                       const float *cos, const float *sin, uint16_t *q, uint16_t *k, uint16_t *vt);

/* Which arm of the q/k preparation the sequential block forms run
 * (dit_block_forward, dit_block_forward_runs, dit_block_forward_cached,
 * the blocks of dit_denoise_step): fused = 1 (the default) folds the head
 * norm and rotation into the QKV product's epilogue; fused = 0 stores the
 * product's projection in bf16 and runs dit_qk_prep's pass (an extra bf16
 * rounding of the projection, and 6 * S * hidden bytes more traffic).  The
 * parallel and double-stream blocks always run the fused epilogue. */
dit_status dit_set_qk_prep(dit_ctx *ctx, int fused);

/* Where int8 block-32 products (DIT_W_INT8_B32, in every block form and
 * dit_linear) turn codes into bf16 weights ([HC] s.1: dequantised inside
 * the graph, products in bf16): in_product = 0 (the default) runs a
 * dequantisation pass per weight into a scratch buffer the context
 * allocates on first use (two sets of one slot per block weight,
 * 2 * (4*hidden + 3*ffn) * hidden bf16 values, kept until dit_ctx_destroy;
 * DIT_ENOMEM if that fails), then the bf16 product (the sequential forms
 * convert their OUT, UP and DOWN weights on a second stream of the context,
 * ordered by events against the context's stream; dit_linear weights that
 * fit no slot are converted inside the product); in_product = 1 converts
 * each k-tile's codes inside the product
 * (no scratch; the conversion's vector instructions then share the SIMDs
 * with the matrix instructions).  Both give the same bf16 weights, bit for
 * bit.  DIT_EINVAL for other values. */
dit_status dit_set_int8_products(dit_ctx *ctx, int in_product);

/* Joint attention ([K4] s.4.3): for each head h, o[:, h*128:(h+1)*128] =
 * bf16(softmax(q_h k_h^T / sqrt(128)) v_h), no mask.  q, k bf16
 * [heads, S, 128]; vt bf16 [heads, 128, Sp] with Sp = S rounded up to a
 * multiple of 64 (values transposed, feature-major; columns S..Sp-1 are
 * never used and may hold anything); o bf16 [S, heads*128].
 * 1 <= S <= max_rows, 1 <= heads <= arch heads. */
dit_status dit_attention(dit_ctx *ctx, const uint16_t *q, const uint16_t *k, const uint16_t *vt,
                         int heads, int S, uint16_t *o);

/* One AdaLN block, in place ([GZ] Block.forward): with (shift_a, scale_a,
 * gate_a, shift_m, scale_m, gate_m) = w_mod * silu(vec),
 *   x += gate_a * OUT(attention(prep(QKV(norm1(x)*(1+scale_a)+shift_a))))
 *   x += gate_m * DOWN(swiglu(UP(norm2(x)*(1+scale_m)+shift_m)))
 * where prep is the per-head RMSNorm times Q_NORM/K_NORM followed by the
 * adjacent-pair rotation with cos/sin ([GZ] prepOf).  x fp32 [L+N, D]
 * (text rows first), vec fp32 [D], cos/sin fp32 [L+N, 64] (from
 * dit_rope_tables).  Requires 0 <= L <= 512, 1 <= N <= 4096 (the DiT graph
 * axes of [HC] s.1, extended down to 0 and 1 for small tests),
 * L + N <= max_rows.  Operands of the products are bf16, accumulation and
 * the residual stream fp32 ([K4] s.2 cast points). */
dit_status dit_block_forward(dit_ctx *ctx, const dit_block *b, float *x, const float *vec,
                             const float *cos, const float *sin, int L, int N);

/* The parallel block ([GZ] Block.parallel): one modulated norm feeds both
 * the attention and the SwiGLU MLP, and one gate scales their sum:
 *   (shift, scale, gate) = w_mod * silu(vec)          w_mod bf16 [3D, D]
 *   h = norm1(x) * (1 + scale) + shift
 *   x += gate * ( OUT(attention(prep(Q(h)), prep(K(h)), V(h)))
 *                 + DOWN(swiglu(UP(h))) )
 * with the same weights, prep, rotary tables and row ranges as
 * dit_block_forward; NORM2 is not used (RMSNorm needs only NORM1).  For bf16
 * weights the four products run as two ([QKV | UP] on h, [OUT | DOWN] on the
 * concatenated [attention output | SwiGLU output] rows). */
dit_status dit_parallel_block_forward(dit_ctx *ctx, const dit_block *b, float *x, const float *vec,
                                      const float *cos, const float *sin, int L, int N);

/* The block with several modulation rows ([GZ] Sequence: map gives each
 * row its modulation row, runs are (first, end, row) triples of rows that
 * share one; Modulation: [modulation rows, hidden] shift/scale/gate;
 * gatedInto: one gated product per run).  vecs fp32 [R, D] on the device
 * are the R conditioning vectors (1 <= R <= 8); runs int32 [n_runs][3] in
 * HOST memory tile rows [0, L+N) in order (first of run i = end of run
 * i-1, first of run 0 = 0, end of the last = L+N, first < end) and name a
 * modulation row 0..R-1 each.  Every row gets dit_block_forward's
 * arithmetic with its run's shifts, scales and gates; the products and the
 * joint attention are shared.  A single run over all rows is
 * dit_block_forward.  Errors as dit_block_forward, and DIT_ERANGE for R or
 * a row outside range, DIT_EINVAL for runs that do not tile the rows.
 * Debug buffer 0 holds the modulation rows [R, 6, D]. */
dit_status dit_block_forward_runs(dit_ctx *ctx, const dit_block *b, float *x, const float *vecs, int R,
                                  const int32_t *runs, int n_runs, const float *cos, const float *sin, int L,
                                  int N);

/* The block with cached reference rows ([GZ] RefSlot, Sequence.active):
 * rows [first, L+N) are a reference whose keys and values are kept across
 * steps in `slot` (device bf16: K [H, count, 128] then V^T [H, 128, count],
 * count = L + N - first; the caller owns it, 2 * H * count * 128 values).
 * record = 1: the whole block over all rows (dit_block_forward), then the
 * reference rows' keys and values (after the head norm and rotary) are
 * copied into the slot.  record = 0: only rows [0, first) are updated -- their
 * norm, QKV, attention against the first rows' keys and the slot's, the
 * output product and the MLP -- and rows [first, L+N) of x stay as they
 * are.  first in 1..L+N (first = L+N: no reference rows, slot may be NULL).
 * Takes the weights the sequential block takes.  Errors as
 * dit_block_forward, DIT_ERANGE for first, DIT_EINVAL for a NULL slot with
 * reference rows or a record flag other than 0 or 1. */
dit_status dit_block_forward_cached(dit_ctx *ctx, const dit_block *b, float *x, const float *vec,
                                    const float *cos, const float *sin, int L, int N, int first,
                                    uint16_t *slot, int record);

/* The double-stream block ([K4] Appendix B: the FLUX.2 double blocks, one
 * set of attention and MLP weights per stream, the q/k preparation run per
 * stream with its rows of the joint rotary table, the attention joint):
 * rows [0, L) of x are the text stream and use `txt` (its w_mod [6D, D],
 * norms, head norms and the four linears), rows [L, L+N) the image stream
 * and use `img`; each stream's rows get exactly dit_block_forward's
 * arithmetic with its own weights, except that the attention runs once
 * over all L + N rows (text first).  Both blocks must have the same wtype
 * rules as dit_block_forward; arguments and errors as dit_block_forward. */
dit_status dit_double_block_forward(dit_ctx *ctx, const dit_block *txt, const dit_block *img, float *x,
                                    const float *vec, const float *cos, const float *sin, int L, int N);

/* Text rows of the sequence, step-invariant ([K4] Appendix B, D2 hoists
 * them out of the Euler loop): txt fp32 [L, D] = ctx_feats * w_txt^T with
 * ctx_feats fp32 [L, text_dim] (taken to bf16 for the product). */
dit_status dit_prologue(dit_ctx *ctx, const dit_model *m, const float *ctx_feats, int L,
                        float *txt);

/* One denoise step ([HC] s.6): the DiT's time input t = (sigma * 1000) /
 * 1000 (two fp32 operations, as dit_sigma_schedule's t); vel = DiT(x_lat, txt, t) (image
 * rows x_lat*w_in^T after the text rows txt, every block, the final
 * modulated LayerNorm of the image rows with (shift, scale) = w_fmod *
 * silu(vec), then w_final); x_lat += (sigma_next - sigma) * vel in fp32.
 * x_lat fp32 [N, latent] in place; txt fp32 [L, D] from dit_prologue;
 * cos/sin fp32 [L+N, 64]; vel_out fp32 [N, latent] or NULL. */
dit_status dit_denoise_step(dit_ctx *ctx, const dit_model *m, float *x_lat, const float *txt,
                            const float *cos, const float *sin, int L, int N, float sigma,
                            float sigma_next, float *vel_out);

/* Plans a schedule's modulation on the context.  The modulation of every
 * block and of the final layer depends on the step only through sigma
 * ([HC] s.6: the time input of each step), so, like the text rows and the
 * rotary tables that [K4] Appendix B D2 hoists out of the Euler loop, it
 * can be computed before the loop: for each of the n host values sigmas[i]
 * the time vector, every block's six modulation rows (w_mod * silu(vec))
 * and the final layer's two, reading each modulation weight once for up to
 * four steps.  A later dit_denoise_step on this context whose sigma has the
 * same bits as a planned sigma, with a model naming the same time-MLP,
 * final-modulation and block modulation weights (pointers), takes the
 * planned rows instead of computing them: the same values, bit for bit.
 * Any other step computes its own, as without a plan.  The plan holds the
 * rows as computed here: plan again after changing those weights in place.
 * n = 0 drops the plan.  The context allocates the plan's memory
 * (n * (3 + 6 * blocks) * D floats) on first use and keeps the largest
 * until dit_ctx_destroy; a call replaces the previous plan, on failure
 * leaving none.  Errors: DIT_ERANGE (n outside 0..64, a sigma not finite),
 * DIT_EINVAL (NULL sigmas with n > 0, a bad model), DIT_ENOMEM. */
dit_status dit_plan_schedule(dit_ctx *ctx, const dit_model *m, const float *sigmas, int n);

/* [HC] s.6 Euler update, fp32, unfused: x[i] = x[i] + (float)(sigma_next -
 * sigma) * v[i] (difference, product and sum each rounded to fp32).
 * x, v fp32 [n]; n >= 0 (0 is a no-op). */
dit_status dit_euler_step(dit_ctx *ctx, float *x, const float *v, int64_t n, float sigma,
                          float sigma_next);

/* [HC] s.1 int8lin dequantisation, exposed for tests: w_out fp32 [out, in]
 * = q[o][k] * s[o][k/32] (exact in fp32).  q int8 [out, in], s bf16
 * [out, in/32]; in a multiple of 32. */
dit_status dit_dequant_int8_b32(dit_ctx *ctx, const int8_t *q, const uint16_t *s, int out,
                                int in, float *w_out);

/* Launch stages of the block forward, denoise step and prologue, for
 * per-kernel timing (dit_timing_read). */
typedef enum {
    DIT_ST_MOD = 0,     /* modulation GEMV */
    DIT_ST_NORM1 = 1,   /* modulated norm before attention */
    DIT_ST_QKV = 2,     /* QKV product + head norm + rotary epilogue */
    DIT_ST_ATTN = 3,    /* joint attention */
    DIT_ST_OUT = 4,     /* output product + gated residual */
    DIT_ST_NORM2 = 5,   /* modulated norm before the MLP */
    DIT_ST_UP = 6,      /* UP product + SwiGLU epilogue */
    DIT_ST_DOWN = 7,    /* DOWN product + gated residual */
    DIT_ST_TIME = 8,    /* sinusoid + time MLP */
    DIT_ST_IMG_IN = 9,  /* latent -> bf16, image-in product, text-row copy */
    DIT_ST_FINAL = 10,  /* final modulation, norm and product */
    DIT_ST_EULER = 11,  /* Euler update (+ velocity copy) */
    DIT_ST_TXT_IN = 12, /* prologue: text features -> bf16, text-in product */
    DIT_ST_PAR_IN = 13, /* parallel block: [QKV | UP] product, both epilogues */
    DIT_ST_PAR_OUT = 14,/* parallel block: [OUT | DOWN] product + gated residual */
    DIT_ST_POST = 15,   /* sandwich block: norm of a product's output, gate, residual */
    DIT_ST_QUANT = 16,  /* W8A8 block: attention / SwiGLU rows to INT8 */
    DIT_ST_QK_PREP = 17,/* unfused arm: q/k head norm + rotary, v transposed */
    DIT_ST_DEQUANT = 18,/* int8 block-32 weights to bf16 before a product */
    DIT_NSTAGES = 19
} dit_stage;

/* Per-stage timing, a measurement aid ([K4] s.3: every op of the busy time
 * is accounted to a bucket).  While enabled (on != 0), each stage above that
 * a call enqueues is bracketed by a pair of HIP events on the context's
 * stream.  Enabling or disabling discards pending records. */
dit_status dit_timing_enable(dit_ctx *ctx, int on);

/* Wait for the recorded events and return, per stage, the summed elapsed
 * milliseconds ms[DIT_NSTAGES] and the number of timed launches
 * count[DIT_NSTAGES] since the last read; then reset.  Synchronises with the
 * recorded events (host blocks until they complete). */
dit_status dit_timing_read(dit_ctx *ctx, double *ms, int64_t *count);

/* Copy an intermediate buffer of the last dit_block_forward on this
 * context into dst (device memory, at least `bytes` long), enqueued on the
 * context's stream; for per-step checks.  Valid until the next call that
 * uses the workspace.  Buffers, packed for that call's S = L + N with
 * Sp = S rounded up to 64:
 *   0 mod  fp32 [6, D]        1 h   bf16 [S, D] (norm1 output)
 *          (double-stream block: [12, D], the text stream's six rows
 *          then the image stream's)
 *   2 q    bf16 [H, S, 128]   3 k   bf16 [H, S, 128] (after head norm + rotary)
 *   4 vt   bf16 [H, 128, Sp]  5 o   bf16 [S, D] (attention output)
 *   6 h2   bf16 [S, D]        7 a   bf16 [S, F] (SwiGLU output)
 *   8 oa   bf16 [S, D + F]   (parallel block with bf16 weights: attention
 *                             output | SwiGLU output; with int8 weights
 *                             those are in 5 and 7)
 * Errors: DIT_ERANGE if `which` is outside 0..8 or `bytes` exceeds the
 * workspace buffer (bytes <= 0 is a no-op). */
dit_status dit_debug_copy(dit_ctx *ctx, int which, void *dst, int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* DIT_H */
