// Internal launch interface between the C ABI layer (dit_api.cpp) and the
// HIP kernels.  Every launcher only enqueues on `st` and returns the launch
// status; shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

// ---- small kernels (k_misc.hip) ------------------------------------------
hipError_t launch_positions(int L, int h, int w, int32_t *pos, hipStream_t st);
hipError_t launch_rope_tables(const int32_t *pos, int S, int a0, int a1, int a2, float theta,
                              float *cos, float *sin, hipStream_t st);
hipError_t launch_time_embedding(float t, int dim, float *temb, hipStream_t st);
hipError_t launch_euler(float *x, const float *v, int64_t n, float dt, hipStream_t st);
// w bf16 [out, in] = bf16(q * s) of int8 block-32 weights (in % 32 == 0,
// q 8-byte and w 16-byte aligned).
hipError_t launch_dequant_bf16(const int8_t *q, const uint16_t *s, int out, int in, uint16_t *w, hipStream_t st);
hipError_t launch_dequant(const int8_t *q, const uint16_t *s, int out, int in, float *w,
                          hipStream_t st);
hipError_t launch_to_bf16(const float *x, int64_t n, uint16_t *y, hipStream_t st);

// y[o] = sum_i W[o, i] * f(x[i]); f = silu when silu_in, else identity.
// W bf16 [O, I]; x, y fp32.  I a multiple of 8, at most 4096.
hipError_t launch_gemv(const uint16_t *W, const float *x, int O, int I, bool silu_in, float *y,
                       hipStream_t st);
// The same for nv <= 4 vectors at once, W read once: vector v is x + v*ldx,
// its result y + v*ldy; each result equals launch_gemv's bit for bit.
hipError_t launch_gemv_multi(const uint16_t *W, const float *x, int64_t ldx, int nv, int O, int I, bool silu_in,
                             float *y, int64_t ldy, hipStream_t st);

// out[r] = bf16(norm(x[r]) * (1 + scale) + shift), r < rows; D <= 4096,
// D a multiple of 4.  rms: RMSNorm times norm_w; else LayerNorm.
// The modulated norm's rows as INT8 codes out [rows, D] and a scale a row
// s [rows] (symmetric: s = amax / 127, q = rint(v * 127 / amax)).
// rot: each 256 values of the row rotated by the regular Hadamard of 256
// (ConvRot) before the quantization; D % 256 == 0.
hipError_t launch_modnorm_i8(const float *x, int rows, int D, const float *shift, const float *scale,
                             const float *norm_w, bool rms, float eps, int8_t *out, float *s, hipStream_t st,
                             bool rot = false);

// bf16 rows x [rows, K] as INT8 codes and a scale a row (as above);
// K % 8 == 0, K <= 16384; rot as above (K % 256 == 0).
hipError_t launch_quant_rows(const uint16_t *x, int rows, int K, int8_t *out, float *s, hipStream_t st,
                             bool rot = false);

// x[r] += gate * (norm(y[r]) * w) for r < rows: a sandwich block's norm of
// a product's output rows before the gate ([GZ] POST_ATTN / POST_MLP); the
// norm is LayerNorm (rms false) or RMSNorm, eps as given; y, x fp32 [rows, D]
hipError_t launch_post_norm_gate(const float *y, int rows, int D, const float *w, bool rms, float eps,
                                 const float *gate, float *x, hipStream_t st);

hipError_t launch_modnorm(const float *x, int rows, int D, const float *shift, const float *scale,
                          const float *norm_w, bool rms, float eps, uint16_t *out, hipStream_t st);

// The unfused q/k/v prep: qkv bf16 [S, 3H*128] -> q, k bf16 [H, Sh, 128]
// (head norm x weight, rotation with cos/sin [S, 64]), vt bf16 [H, 128, ldv]
// (rows [0, S) of each; ldv % 8 == 0, 16-byte aligned buffers).
hipError_t launch_qk_prep(const uint16_t *qkv, int S, int H, int Sh, const float *qn, const float *kn, const float *cs,
                          const float *sn, float eps, uint16_t *q, uint16_t *k, uint16_t *vt, int ldv, hipStream_t st);

// ---- products (k_gemm.hip) -------------------------------------------------
enum EpiKind { EPI_F32 = 0, EPI_GATE_RES = 1, EPI_SWIGLU = 2, EPI_QKV = 3, EPI_QKV_SWIGLU = 4, EPI_BF16 = 5 };

struct GemmEpi {
    int kind;
    float *out;            // EPI_F32: out [M, ldo] fp32; EPI_GATE_RES: x [M, ldo] += gate * acc
    int ldo;
    const float *gate;     // EPI_GATE_RES: [N]
    uint16_t *act;         // EPI_SWIGLU: bf16 [M, N/2]; EPI_BF16: bf16 [M, ld_act] = C
    // EPI_QKV
    uint16_t *q, *k, *vt;  // q, k [H, M, 128]; vt [H, 128, ldv]
    int heads, ldv;
    const float *qn, *kn;  // [128] head-norm weights
    const float *cos, *sin;// [M, 64]
    float qk_eps;
    int ld_act;            // EPI_SWIGLU: row stride of act (0: N/2); EPI_BF16: row stride (0: N)
    // Two-weight products of the parallel block (bf16 weights only):
    //  EPI_QKV_SWIGLU: columns < n_split take W [n_split, K] and the QKV
    //    epilogue; columns >= n_split take w2 [N - n_split, K] and the SwiGLU
    //    epilogue into act (column n_split + c -> act column c/2)
    //  k_split > 0: k < k_split multiplies W [N, k_split], k >= k_split
    //    multiplies w2 [N, K - k_split]; A is one [M, K] operand
    const uint16_t *w2;
    int n_split;
    int k_split;
    // EPI_QKV over a row range of a longer sequence (the double-stream
    // block's streams): local row r is row row_base + r of q, k ([H,
    // rows_total, 128]; rows_total 0 means M) and column row_base + r of vt;
    // cos and sin are passed already offset to row_base.
    int row_base;
    int rows_total;
    // W8A8 products (launch_gemm_w8a8 sets them): fp32 scale per A row and
    // per output column
    const float *a_scale;
    const float *w_scale;
    // int8 block-32 weights on the ping-pong kernel (launch_gemm sets it):
    // the weight's bf16 scales [N, K/32]
    const uint16_t *w_bscale;
};

// C = A[M,K] * W[N,K]^T, A bf16; W bf16 (w8 = false) or int8 with bf16
// scales [N, K/32] (w8 = true); then the epilogue.  K % 64 == 0, N % 64 == 0.
// a_rows_padded: A's allocation holds at least M rounded up to 256 rows
// (rows past M are read and their results discarded).
hipError_t launch_gemm(const uint16_t *A, const void *W, const uint16_t *Wscale, bool w8, int M,
                       int N, int K, const GemmEpi &epi, hipStream_t st, bool a_rows_padded);
// Two products with the same N, K, epilogue kind and weight type (the
// double-stream block's streams), each A with whole 256-row tiles
// allocated: one ping-pong launch over both tile sets when both qualify,
// else launch_gemm for each.  M or M2 may be 0.
hipError_t launch_gemm2(const uint16_t *A, const void *W, const uint16_t *Ws, int M, const GemmEpi &ep,
                        const uint16_t *A2, const void *W2, const uint16_t *Ws2, int M2, const GemmEpi &ep2,
                        bool w8, int N, int K, hipStream_t st);
// W8A8: C = (A_q W_q^T) * a_scale[row] * w_scale[col], A_q int8 [M, K] (rows
// allocated to a whole 256-row tile), W_q int8 [N, K]; N % 256 == 0,
// K % 128 == 0; epilogues EPI_F32, EPI_GATE_RES, EPI_SWIGLU, EPI_QKV.
hipError_t launch_gemm_w8a8(const int8_t *A, const float *a_scale, const int8_t *W, const float *w_scale, int M,
                            int N, int K, const GemmEpi &ep, hipStream_t st);

// Whether launch_gemm runs this product as the 256x256 ping-pong kernel (the
// only one that takes EPI_QKV_SWIGLU and k_split > 0; asked before using them).
bool gemm_pingpong_ok(int M, int N, int K, bool w8, const GemmEpi &epi, bool a_rows_padded);

// ---- attention (k_attn.hip) ------------------------------------------------
// o = softmax(q k^T / sqrt(128)) v per head over S keys; the queries are
// rows [0, Sq) (Sq < 0: all S), q keeping the head stride S.
hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *vt, int heads,
                            int S, int ldv, uint16_t *o, int ldo, hipStream_t st, int Sq = -1);

}  // namespace dit

// Sets the text dit_last_error(NULL) returns (dit_api.cpp).
void dit_set_global_error(const char *msg);
