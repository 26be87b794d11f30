// Small HBM- or launch-bound kernels of the DiT path: positions and rotary
// tables, the timestep sinusoid, the modulation / time-MLP GEMV, the
// modulated norm, the Euler update, int8 dequantisation and fp32->bf16.
//
// Sources: "Host contract -- RGBA-Image-2.1-Turbo" s.4 (positions, rotary
// tables), s.6 (Euler update, fp32); "gizai:dit" reference: sinusoids,
// Modulation, normedInto; s.1 of the host contract for the int8 format.
#include <type_traits>

#include <algorithm>
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace dit {

// ------------------------------------------------------------------ positions
// Text token i -> (i, i, i); image token y*w + x -> (L, y - (h - h/2),
// x - (w - w/2)) (host contract s.4; the grid is centred on zero).
__global__ void k_positions(int L, int h, int w, int32_t *pos) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    int S = L + h * w;
    if (i >= S) return;
    int a, b, c;
    if (i < L) {
        a = b = c = i;
    } else {
        int t = i - L, y = t / w, x = t - y * w;
        a = L;
        b = y - (h - h / 2);
        c = x - (w - w / 2);
    }
    pos[3 * i + 0] = a;
    pos[3 * i + 1] = b;
    pos[3 * i + 2] = c;
}

hipError_t launch_positions(int L, int h, int w, int32_t *pos, hipStream_t st) {
    int S = L + h * w;
    k_positions<<<(S + 255) / 256, 256, 0, st>>>(L, h, w, pos);
    return hipGetLastError();
}

// ------------------------------------------------------------- rotary tables
// One thread per (token, pair).  Pair p belongs to axis 0 for p < a0/2, to
// axis 1 for the next a1/2, then axis 2.  The angle pos * theta^(-2j/d) and
// its cos/sin are computed in fp64 and rounded once to fp32.
__global__ void k_rope_tables(const int32_t *pos, int S, int a0, int a1, int a2, double theta,
                              float *cs, float *sn) {
    int P = (a0 + a1 + a2) / 2;
    int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= S * P) return;
    int r = idx / P, p = idx - r * P;
    int axis, j, d;
    if (p < a0 / 2) {
        axis = 0; j = p; d = a0;
    } else if (p < (a0 + a1) / 2) {
        axis = 1; j = p - a0 / 2; d = a1;
    } else {
        axis = 2; j = p - (a0 + a1) / 2; d = a2;
    }
    double inv = 1.0 / pow(theta, static_cast<double>(2 * j) / static_cast<double>(d));
    double ang = static_cast<double>(pos[3 * r + axis]) * inv;
    cs[idx] = static_cast<float>(cos(ang));
    sn[idx] = static_cast<float>(sin(ang));
}

hipError_t launch_rope_tables(const int32_t *pos, int S, int a0, int a1, int a2, float theta,
                              float *cos_t, float *sin_t, hipStream_t st) {
    int P = (a0 + a1 + a2) / 2;
    int64_t n = static_cast<int64_t>(S) * P;
    k_rope_tables<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(pos, S, a0, a1, a2,
                                                                          theta, cos_t, sin_t);
    return hipGetLastError();
}

// ------------------------------------------------------------ time embedding
// [cos | sin] of (1000 t) * 10000^(-i/(dim/2)) ("gizai:dit" sinusoids), taken
// in fp64 and stored fp32.
__global__ void k_time_embedding(float t, int dim, float *temb) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    int half = dim / 2;
    if (i >= dim) return;
    int f = i < half ? i : i - half;
    double freq = pow(10000.0, -static_cast<double>(f) / static_cast<double>(half));
    double ang = 1000.0 * static_cast<double>(t) * freq;
    temb[i] = static_cast<float>(i < half ? cos(ang) : sin(ang));
}

hipError_t launch_time_embedding(float t, int dim, float *temb, hipStream_t st) {
    k_time_embedding<<<(dim + 255) / 256, 256, 0, st>>>(t, dim, temb);
    return hipGetLastError();
}

// ---------------------------------------------------------------------- Euler
// x + dt * v in fp32 with the product and the sum each rounded (no fused
// multiply-add): the host contract writes the update as plain fp32 ops.
__global__ void k_euler(float *__restrict__ x, const float *__restrict__ v, int64_t n, float dt) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) x[i] = __fadd_rn(x[i], __fmul_rn(dt, v[i]));
}

hipError_t launch_euler(float *x, const float *v, int64_t n, float dt, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    k_euler<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(x, v, n, dt);
    return hipGetLastError();
}

// ------------------------------------------------------------------- dequant
// w[o][k] = q[o][k] * s[o][k/32]; exact in fp32 (|q| <= 127, bf16 scale).
__global__ void k_dequant(const int8_t *q, const uint16_t *s, int out, int in, float *w) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    int64_t n = static_cast<int64_t>(out) * in;
    if (i >= n) return;
    int64_t o = i / in, k = i - o * in;
    w[i] = static_cast<float>(q[i]) * bf16_to_f32(s[o * (in / 32) + k / 32]);
}

hipError_t launch_dequant(const int8_t *q, const uint16_t *s, int out, int in, float *w,
                          hipStream_t st) {
    int64_t n = static_cast<int64_t>(out) * in;
    if (n == 0) return hipSuccess;
    k_dequant<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(q, s, out, in, w);
    return hipGetLastError();
}

// bf16 weights from int8 block-32 codes for the bf16 products: w[o][k] =
// bf16(q[o][k] * s[o][k/32]), the exact product rounded to nearest even.
// Thread i converts codes 8i .. 8i+7 of the flat array (one 8-byte load;
// with in % 32 == 0 the 8 share one block), so a wave's load reads 512
// contiguous bytes and its store writes 1 KB.  The product is exact in
// fp32: with the code's sign bit flipped, u = q + 128 in 0..255 converts
// exactly and u * s - 128 * s is q * s (at most 16 significant bits).
__global__ void __launch_bounds__(256) k_dequant_bf16(const u32x2 *__restrict__ q, const uint16_t *__restrict__ s,
                                                      int64_t n8, u32x4 *__restrict__ w) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n8;
         i += static_cast<int64_t>(gridDim.x) * 256) {
        const u32x2 c = __builtin_nontemporal_load(q + i);
        const float sc = bf16_to_f32(s[i >> 2]), msc = -128.0f * sc;
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t u = c[j] ^ 0x80808080u;
            auto dq = [&](int b) { return __builtin_fmaf(static_cast<float>((u >> (8 * b)) & 0xffu), sc, msc); };
            o[2 * j] = pack_bf16x2(dq(0), dq(1));
            o[2 * j + 1] = pack_bf16x2(dq(2), dq(3));
        }
        w[i] = u32x4{o[0], o[1], o[2], o[3]};
    }
}

hipError_t launch_dequant_bf16(const int8_t *q, const uint16_t *s, int out, int in, uint16_t *w, hipStream_t st) {
    const int64_t n = static_cast<int64_t>(out) * in;
    if (n == 0) return hipSuccess;
    if (in % 32 || (reinterpret_cast<uintptr_t>(q) & 7) || (reinterpret_cast<uintptr_t>(w) & 15))
        return hipErrorInvalidValue;
    const int64_t n8 = n / 8;
    const int64_t want = (n8 + 255) / 256;
    const unsigned grid = static_cast<unsigned>(want < 8192 ? want : 8192);
    k_dequant_bf16<<<grid, 256, 0, st>>>(reinterpret_cast<const u32x2 *>(q), s, n8, reinterpret_cast<u32x4 *>(w));
    return hipGetLastError();
}

// ------------------------------------------------------------------- to bf16
__global__ void k_to_bf16(const float *x, int64_t n, uint16_t *y) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) y[i] = f32_to_bf16(x[i]);
}

hipError_t launch_to_bf16(const float *x, int64_t n, uint16_t *y, hipStream_t st) {
    if (n == 0) return hipSuccess;
    k_to_bf16<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(x, n, y);
    return hipGetLastError();
}

// ---------------------------------------------------------------------- GEMV
// One wave per output row, 16-byte loads of W (8 bf16 per lane per step).
// A lane always takes the same columns (chunks lane + 64j of 8), so it holds
// its columns of the input vectors in registers, loaded once (with silu
// applied) before its first row.  The weight is read exactly once: the
// kernel is HBM-bound, so a lane issues all its loads of a row before the
// first multiply, keeping several in flight per wave; the sum runs in the
// same order as a one-load loop.  NV vectors share each row's loads (the
// planned schedule's steps); every vector's sum is formed by the same
// expressions in the same order whatever NV is, so a row's result does not
// depend on how many vectors share the launch.  JM chunks per lane at most
// (I <= 512 * JM).
constexpr int kGemvThreads = 256;
constexpr int kGemvMaxI = 4096;
constexpr int kGemvMaxV = 4;

template <int NV, int JM>
__global__ void __launch_bounds__(kGemvThreads)
k_gemv(const uint16_t *__restrict__ W, const float *__restrict__ x, int64_t ldx, int O, int I, int silu_in,
       float *__restrict__ y, int64_t ldy) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nchunk = I / 8;
    float4 xr[NV][JM][2];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const int c = lane + 64 * j;
            float4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
            if (c < nchunk) {
                a = *reinterpret_cast<const float4 *>(x + v * ldx + c * 8);
                b = *reinterpret_cast<const float4 *>(x + v * ldx + c * 8 + 4);
                if (silu_in) {
                    a = float4{silu_f(a.x), silu_f(a.y), silu_f(a.z), silu_f(a.w)};
                    b = float4{silu_f(b.x), silu_f(b.y), silu_f(b.z), silu_f(b.w)};
                }
            }
            xr[v][j][0] = a;
            xr[v][j][1] = b;
        }
    for (int o = blockIdx.x * 4 + wv; o < O; o += gridDim.x * 4) {
        const u32x4 *row = reinterpret_cast<const u32x4 *>(W + static_cast<int64_t>(o) * I);
        u32x4 wr[JM];
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const int c = lane + 64 * j;
            wr[j] = c < nchunk ? __builtin_nontemporal_load(row + c) : u32x4{0u, 0u, 0u, 0u};
        }
        float acc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = 0.f;
#pragma unroll
        for (int j = 0; j < JM; ++j) {
            const int c = lane + 64 * j;
            if (c >= nchunk) break;
            const u32x4 w = wr[j];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const float4 a = xr[v][j][0], b = xr[v][j][1];
                acc[v] += bf16lo_to_f32(w.x) * a.x + bf16hi_to_f32(w.x) * a.y;
                acc[v] += bf16lo_to_f32(w.y) * a.z + bf16hi_to_f32(w.y) * a.w;
                acc[v] += bf16lo_to_f32(w.z) * b.x + bf16hi_to_f32(w.z) * b.y;
                acc[v] += bf16lo_to_f32(w.w) * b.z + bf16hi_to_f32(w.w) * b.w;
            }
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const float t = wave_sum(acc[v]);
            if (lane == 0) y[v * ldy + o] = t;
        }
    }
}

// One launch of k_gemv<NV, JM>: as many blocks as the device holds at once
// (each wave loads its vector columns once, then walks its rows), at most
// one row per wave.
template <int NV, int JM>
hipError_t launch_gemv_nv(const uint16_t *W, const float *x, int64_t ldx, int O, int I, int si, float *y,
                          int64_t ldy, hipStream_t st) {
    // blocks the device holds at once, per device id (computed once; calls
    // from several threads may both compute it, with the same result)
    static std::atomic<int> resident[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int res = resident[dev].load(std::memory_order_relaxed);
    if (res == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gemv<NV, JM>, kGemvThreads, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidValue;
        res = std::max(1, per_cu) * std::max(1, cus);
        resident[dev].store(res, std::memory_order_relaxed);
    }
    const int blocks = std::min((O + 3) / 4, res);
    k_gemv<NV, JM><<<blocks, kGemvThreads, 0, st>>>(W, x, ldx, O, I, si, y, ldy);
    return hipGetLastError();
}

hipError_t launch_gemv_multi(const uint16_t *W, const float *x, int64_t ldx, int nv, int O, int I, bool silu_in,
                             float *y, int64_t ldy, hipStream_t st) {
    if (O <= 0 || nv == 0) return hipSuccess;
    if (I <= 0 || I > kGemvMaxI || I % 8 || nv < 0 || nv > kGemvMaxV) return hipErrorInvalidValue;
    const int si = silu_in ? 1 : 0;
    // the vectors' columns a lane holds: 8 * JM of each (JM 6 covers I <= 3072)
    if (I <= 3072) {
        switch (nv) {
            case 1: return launch_gemv_nv<1, 6>(W, x, ldx, O, I, si, y, ldy, st);
            case 2: return launch_gemv_nv<2, 6>(W, x, ldx, O, I, si, y, ldy, st);
            case 3: return launch_gemv_nv<3, 6>(W, x, ldx, O, I, si, y, ldy, st);
            default: return launch_gemv_nv<4, 6>(W, x, ldx, O, I, si, y, ldy, st);
        }
    }
    switch (nv) {
        case 1: return launch_gemv_nv<1, 8>(W, x, ldx, O, I, si, y, ldy, st);
        case 2: return launch_gemv_nv<2, 8>(W, x, ldx, O, I, si, y, ldy, st);
        case 3: return launch_gemv_nv<3, 8>(W, x, ldx, O, I, si, y, ldy, st);
        default: return launch_gemv_nv<4, 8>(W, x, ldx, O, I, si, y, ldy, st);
    }
}

hipError_t launch_gemv(const uint16_t *W, const float *x, int O, int I, bool silu_in, float *y,
                       hipStream_t st) {
    return launch_gemv_multi(W, x, I, 1, O, I, silu_in, y, O, st);
}

// ------------------------------------------------------------ modulated norm
// One row per block of 256 threads; each thread keeps up to 4 float4 of the
// row in registers (D <= 4096).  Statistics in fp32 with a two-pass
// variance over the register-resident row; output bf16.
constexpr int kNormThreads = 256;

__device__ __forceinline__ float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wv] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kNormThreads / 64; ++i) t += red[i];
    return t;
}

__global__ void __launch_bounds__(kNormThreads)
k_modnorm(const float *__restrict__ x, int D, const float *__restrict__ shift,
          const float *__restrict__ scale, const float *__restrict__ nw, int rms, float eps,
          uint16_t *__restrict__ out) {
    __shared__ float red[kNormThreads / 64];
    const int64_t r = blockIdx.x;
    const float4 *xr = reinterpret_cast<const float4 *>(x + r * D);
    const int n4 = D / 4;
    float4 v[4];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kNormThreads;
        v[i] = c < n4 ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    const float invD = 1.0f / static_cast<float>(D);
    float mu = 0.f, rstd;
    if (!rms) {
        mu = block_sum(s, red) * invD;
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int c = threadIdx.x + i * kNormThreads;
            if (c < n4) {
                float a = v[i].x - mu, b = v[i].y - mu, cc = v[i].z - mu, d = v[i].w - mu;
                q += (a * a + b * b) + (cc * cc + d * d);
            }
        }
        rstd = rsqrtf(block_sum(q, red) * invD + eps);
    } else {
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
        rstd = rsqrtf(block_sum(q, red) * invD + eps);
    }
    u32x2 *orow = reinterpret_cast<u32x2 *>(out + r * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kNormThreads;
        if (c >= n4) continue;
        float4 sh = reinterpret_cast<const float4 *>(shift)[c];
        float4 sc = reinterpret_cast<const float4 *>(scale)[c];
        float4 w = rms ? reinterpret_cast<const float4 *>(nw)[c] : make_float4(1.f, 1.f, 1.f, 1.f);
        float a = (v[i].x - mu) * rstd * w.x * (1.f + sc.x) + sh.x;
        float b = (v[i].y - mu) * rstd * w.y * (1.f + sc.y) + sh.y;
        float cc = (v[i].z - mu) * rstd * w.z * (1.f + sc.z) + sh.z;
        float d = (v[i].w - mu) * rstd * w.w * (1.f + sc.w) + sh.w;
        u32x2 o2 = {pack_bf16x2(a, b), pack_bf16x2(cc, d)};
        orow[c] = o2;
    }
}

// One row per workgroup, as k_modnorm: the row of y stays in registers
// between the statistics and the update.
__global__ void __launch_bounds__(kNormThreads)
k_post_norm_gate(const float *__restrict__ y, int D, const float *__restrict__ nw, int rms, float eps,
                 const float *__restrict__ gate, float *__restrict__ x) {
    __shared__ float red[kNormThreads / 64];
    const int64_t r = blockIdx.x;
    const float4 *yr = reinterpret_cast<const float4 *>(y + r * D);
    const int n4 = D / 4;
    float4 v[4];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kNormThreads;
        v[i] = c < n4 ? yr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    const float invD = 1.0f / static_cast<float>(D);
    float mu = 0.f;
    if (!rms) mu = block_sum(s, red) * invD;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kNormThreads;
        if (c < n4) {
            float a = v[i].x - mu, b = v[i].y - mu, cc = v[i].z - mu, d = v[i].w - mu;
            q += (a * a + b * b) + (cc * cc + d * d);
        }
    }
    const float rstd = rsqrtf(block_sum(q, red) * invD + eps);
    float4 *xr = reinterpret_cast<float4 *>(x + r * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kNormThreads;
        if (c >= n4) continue;
        const float4 w = reinterpret_cast<const float4 *>(nw)[c];
        const float4 g = reinterpret_cast<const float4 *>(gate)[c];
        float4 o = xr[c];
        o.x += g.x * ((v[i].x - mu) * rstd * w.x);
        o.y += g.y * ((v[i].y - mu) * rstd * w.y);
        o.z += g.z * ((v[i].z - mu) * rstd * w.z);
        o.w += g.w * ((v[i].w - mu) * rstd * w.w);
        xr[c] = o;
    }
}

hipError_t launch_post_norm_gate(const float *y, int rows, int D, const float *w, bool rms, float eps,
                                 const float *gate, float *x, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    if (D % 4 != 0 || D > 16 * kNormThreads) return hipErrorInvalidValue;
    k_post_norm_gate<<<rows, kNormThreads, 0, st>>>(y, D, w, rms ? 1 : 0, eps, gate, x);
    return hipGetLastError();
}

// ------------------------------------------------------------ q/k/v prep
// The QKV projection's heads made ready for the attention in a pass of their
// own, the unfused arm of the QKV product's epilogue ("944 -> 346 ms:
// optimizing FLUX.2 klein-4B on one TPU v6e chip" s.4.4 runs this prep as a
// separate kernel over the stored projection; "gizai:dit" prepOf): per
// 128-wide head of q and k, RMSNorm (fp32 statistics) times the head-norm
// weight, then the adjacent-pair rotation with the row's cos/sin, to bf16
// q, k [H, Sh, 128]; v heads transposed to vt [H, 128, ldv].  qkv bf16
// [S, 3 * H * 128] (all queries, all keys, all values).  One workgroup per
// (64-row tile, head of q, k or v): 16 KB in, 16 KB out, HBM-bound.
constexpr int kPrepRows = 64;

__global__ void __launch_bounds__(256)
k_qk_prep(const uint16_t *__restrict__ qkv, int S, int H, int Sh, const float *__restrict__ qn,
          const float *__restrict__ kn, const float *__restrict__ cs, const float *__restrict__ sn, float eps,
          uint16_t *__restrict__ q, uint16_t *__restrict__ k, uint16_t *__restrict__ vt, int ldv) {
    __shared__ uint16_t tile[kPrepRows][128 + 8];
    const int r0 = blockIdx.x * kPrepRows;
    const int hh = blockIdx.y, region = hh / H, head = hh % H;
    const int64_t ld = static_cast<int64_t>(3) * H * 128;
    const int t = threadIdx.x;
    if (region < 2) {
        // 16 lanes to a (row, head): lane l16 holds features 8 l16 .. 8 l16 + 7,
        // i.e. rotation pairs 4 l16 .. 4 l16 + 3
        const float *nw = region == 0 ? qn : kn;
        uint16_t *dst = region == 0 ? q : k;
        const int l16 = t & 15;
        const f32x4 w0 = *reinterpret_cast<const f32x4 *>(nw + 8 * l16);
        const f32x4 w1 = *reinterpret_cast<const f32x4 *>(nw + 8 * l16 + 4);
        const float w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
        for (int it = 0; it < kPrepRows / 16; ++it) {
            const int r = r0 + it * 16 + (t >> 4);
            const int rr = min(r, S - 1);
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(qkv + rr * ld + hh * 128 + 8 * l16);
            float v[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[2 * j] = bf16lo_to_f32(raw[j]);
                v[2 * j + 1] = bf16hi_to_f32(raw[j]);
            }
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
            ss = row16_sum(ss);
            const float rstd = rsqrtf(ss * (1.0f / 128.0f) + eps);
            const f32x4 c = *reinterpret_cast<const f32x4 *>(cs + static_cast<int64_t>(rr) * 64 + 4 * l16);
            const f32x4 sv = *reinterpret_cast<const f32x4 *>(sn + static_cast<int64_t>(rr) * 64 + 4 * l16);
            uint32_t o[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float a = v[2 * p] * rstd * w[2 * p], b = v[2 * p + 1] * rstd * w[2 * p + 1];
                o[p] = rotate_pack(a, b, c[p], sv[p]);
            }
            if (r < S)
                *reinterpret_cast<u32x4 *>(dst + (static_cast<int64_t>(head) * Sh + r) * 128 + 8 * l16) =
                    u32x4{o[0], o[1], o[2], o[3]};
        }
    } else {
        // v: 64 rows x 128 features through LDS, out as 128 feature rows of 64 keys
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = t + 256 * i, row = c >> 4, col = (c & 15) * 8;
            const int r = min(r0 + row, S - 1);
            *reinterpret_cast<u32x4 *>(&tile[row][col]) =
                *reinterpret_cast<const u32x4 *>(qkv + r * ld + hh * 128 + col);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = t + 256 * i, d = e >> 3, kb = (e & 7) * 8;
            uint16_t *out = vt + (static_cast<int64_t>(head) * 128 + d) * ldv + r0 + kb;
            const int valid = S - (r0 + kb);
            if (valid >= 8) {
                u32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    o[j] = static_cast<uint32_t>(tile[kb + 2 * j][d]) | (static_cast<uint32_t>(tile[kb + 2 * j + 1][d]) << 16);
                *reinterpret_cast<u32x4 *>(out) = o;
            } else {
                for (int j = 0; j < valid; ++j) out[j] = tile[kb + j][d];
            }
        }
    }
}

hipError_t launch_qk_prep(const uint16_t *qkv, int S, int H, int Sh, const float *qn, const float *kn, const float *cs,
                          const float *sn, float eps, uint16_t *q, uint16_t *k, uint16_t *vt, int ldv, hipStream_t st) {
    if (S <= 0) return hipSuccess;
    if (Sh < S || ldv < S || ldv % 8) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>((S + kPrepRows - 1) / kPrepRows), static_cast<unsigned>(3 * H));
    k_qk_prep<<<grid, 256, 0, st>>>(qkv, S, H, Sh, qn, kn, cs, sn, eps, q, k, vt, ldv);
    return hipGetLastError();
}

// ------------------------------------------------------------ INT8 rows
// Symmetric INT8 codes of a row over one scale (W8A8 products' inputs):
// inv = 127 / amax and q = rint(v * inv) clamped to +-127, s = amax / 127,
// each a correctly rounded fp32 operation (the division is IEEE-exact by
// default in HIP); an all-zero row gets s = 0 and q = 0.
__device__ __forceinline__ float block_max(float v, float *red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wv] = v;
    __syncthreads();
    float t = red[0];
#pragma unroll
    for (int i = 1; i < kNormThreads / 64; ++i) t = fmaxf(t, red[i]);
    return t;
}

// The value lane ^ m holds (m = 1 .. 32), without the LDS: DPP row
// permutations for m < 16 (quad_perm for 1, 2 and 3, half-row mirror = 7,
// row mirror = 15; 4 = 7 then 3, 8 = 15 then 7), the gfx950 row swaps for
// 16 and 32 (swapping a value with itself leaves each lane its own value in
// one result and its partner's in the other).
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    const int u = __float_as_int(v);
    auto dpp = [](int x, auto ctrl) { return __builtin_amdgcn_mov_dpp(x, decltype(ctrl)::value, 0xf, 0xf, false); };
    using Q1 = std::integral_constant<int, 0xb1>;    // quad_perm(1, 0, 3, 2)
    using Q2 = std::integral_constant<int, 0x4e>;    // quad_perm(2, 3, 0, 1)
    using Q3 = std::integral_constant<int, 0x1b>;    // quad_perm(3, 2, 1, 0)
    using HM = std::integral_constant<int, 0x141>;   // row_half_mirror: lane ^ 7 within 8
    using RM = std::integral_constant<int, 0x140>;   // row_mirror: lane ^ 15 within 16
    if constexpr (M == 1) return __int_as_float(dpp(u, Q1{}));
    if constexpr (M == 2) return __int_as_float(dpp(u, Q2{}));
    if constexpr (M == 4) return __int_as_float(dpp(dpp(u, HM{}), Q3{}));
    if constexpr (M == 8) return __int_as_float(dpp(dpp(u, RM{}), HM{}));
    const int lane = threadIdx.x & 63;
    if constexpr (M == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(u), static_cast<unsigned>(u), false, false);
        return __uint_as_float((lane & 16) ? p[0] : p[1]);
    }
    if constexpr (M == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(u), static_cast<unsigned>(u), false, false);
        return __uint_as_float((lane & 32) ? p[0] : p[1]);
    }
    return v;
}

// One cross-lane butterfly stage: lanes with bit m clear keep a + b, the
// others b - a (a their own value, b their partner's).
template <int M, int NPL>
__device__ __forceinline__ void butterfly_lanes(float (&v)[NPL]) {
    const float sgn = (threadIdx.x & M) ? -1.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < NPL; ++k) v[k] = __builtin_fmaf(sgn, v[k], xor_lane<M>(v[k]));
}

// ConvRot's rotation ("gizai:dit" reference: linearInto and
// Block.dequantized: each 256 inputs x go to y = R x, R the regular
// Hadamard of 256): the fast transform over the 8 index bits, butterflies
// (a, b) -> (a + b, a - b) in the Hadamard's own (Sylvester) order, then the
// exact 1/16.  A group of 256 values is spread over 256/NPL lanes, NPL
// values a lane: value index NPL * (lane % (256/NPL)) + k is v[k], so the
// low bits are a lane's own and the others pair lanes lane ^ m.
template <int NPL>
__device__ __forceinline__ void convrot256(float (&v)[NPL]) {
#pragma unroll
    for (int h = 1; h < NPL; h <<= 1)
#pragma unroll
        for (int k = 0; k < NPL; ++k)
            if (!(k & h)) {
                const float a = v[k], b = v[k + h];
                v[k] = a + b;
                v[k + h] = a - b;
            }
    butterfly_lanes<1>(v);
    butterfly_lanes<2>(v);
    butterfly_lanes<4>(v);
    butterfly_lanes<8>(v);
    butterfly_lanes<16>(v);
    if constexpr (256 / NPL > 32) butterfly_lanes<32>(v);
#pragma unroll
    for (int k = 0; k < NPL; ++k) v[k] *= 0.0625f;
}

__device__ __forceinline__ uint32_t q8x4(float a, float b, float c, float d, float inv) {
    auto q = [inv](float v) -> uint32_t {
        const float r = fminf(fmaxf(rintf(v * inv), -127.f), 127.f);
        return static_cast<uint32_t>(static_cast<int>(r)) & 0xffu;
    };
    return q(a) | (q(b) << 8) | (q(c) << 16) | (q(d) << 24);
}

// The modulated norm of k_modnorm with its row taken to INT8 codes (out)
// and one fp32 scale (s[r]) in the same pass; ROT: rotated by ConvRot
// first (D a multiple of 256: slot i of wave w holds group 4i + w).
template <bool ROT>
__global__ void __launch_bounds__(kNormThreads)
k_modnorm_i8(const float *__restrict__ x, int D, const float *__restrict__ shift,
             const float *__restrict__ scale, const float *__restrict__ nw, int rms, float eps,
             int8_t *__restrict__ out, float *__restrict__ s_out) {
    __shared__ float red[kNormThreads / 64];
    const int64_t r = blockIdx.x;
    const float4 *xr = reinterpret_cast<const float4 *>(x + r * D);
    const int n4 = D / 4;
    float4 v[4];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kNormThreads;
        v[i] = c < n4 ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
    const float invD = 1.0f / static_cast<float>(D);
    float mu = 0.f;
    if (!rms) mu = block_sum(s, red) * invD;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kNormThreads;
        if (c < n4) {
            float a = v[i].x - mu, b = v[i].y - mu, cc = v[i].z - mu, d = v[i].w - mu;
            q += (a * a + b * b) + (cc * cc + d * d);
        }
    }
    const float rstd = rsqrtf(block_sum(q, red) * invD + eps);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kNormThreads;
        if (c >= n4) continue;
        float4 sh = reinterpret_cast<const float4 *>(shift)[c];
        float4 sc = reinterpret_cast<const float4 *>(scale)[c];
        float4 w = rms ? reinterpret_cast<const float4 *>(nw)[c] : make_float4(1.f, 1.f, 1.f, 1.f);
        v[i].x = (v[i].x - mu) * rstd * w.x * (1.f + sc.x) + sh.x;
        v[i].y = (v[i].y - mu) * rstd * w.y * (1.f + sc.y) + sh.y;
        v[i].z = (v[i].z - mu) * rstd * w.z * (1.f + sc.z) + sh.z;
        v[i].w = (v[i].w - mu) * rstd * w.w * (1.f + sc.w) + sh.w;
        if constexpr (ROT) {
            float g[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            convrot256<4>(g);     // the whole wave takes this branch (D % 256 == 0)
            v[i] = make_float4(g[0], g[1], g[2], g[3]);
        }
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    amax = block_max(amax, red);
    const float inv = amax > 0.f ? 127.f / amax : 0.f;
    uint32_t *orow = reinterpret_cast<uint32_t *>(out + r * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = threadIdx.x + i * kNormThreads;
        if (c < n4) orow[c] = q8x4(v[i].x, v[i].y, v[i].z, v[i].w, inv);
    }
    if (threadIdx.x == 0) s_out[r] = amax / 127.f;
}

// bf16 rows [rows, K] to INT8 codes and a scale a row; K % 8 == 0, K <= 16384.
// ROT: rotated by ConvRot first (K a multiple of 256: chunk slot i of lane
// group t / 32 holds group 8i + t / 32, 8 values a lane); the rotation runs
// on every slot, zeros past the row included, so that all lanes take part.
template <bool ROT>
__global__ void __launch_bounds__(kNormThreads)
k_quant_rows(const uint16_t *__restrict__ x, int K, int8_t *__restrict__ out, float *__restrict__ s_out) {
    __shared__ float red[kNormThreads / 64];
    const int64_t r = blockIdx.x;
    const u32x4 *xr = reinterpret_cast<const u32x4 *>(x + r * K);
    const int n8 = K / 8;
    if constexpr (ROT) {
        float f[8][8];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = threadIdx.x + i * kNormThreads;
            const u32x4 w = c < n8 ? xr[c] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f[i][2 * j] = bf16lo_to_f32(w[j]);
                f[i][2 * j + 1] = bf16hi_to_f32(w[j]);
            }
            if (i * kNormThreads < n8) convrot256<8>(f[i]);   // uniform over the block
#pragma unroll
            for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(f[i][k]));
        }
        amax = block_max(amax, red);
        const float inv = amax > 0.f ? 127.f / amax : 0.f;
        u32x2 *orow = reinterpret_cast<u32x2 *>(out + r * K);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = threadIdx.x + i * kNormThreads;
            if (c < n8)
                orow[c] = u32x2{q8x4(f[i][0], f[i][1], f[i][2], f[i][3], inv), q8x4(f[i][4], f[i][5], f[i][6], f[i][7], inv)};
        }
        if (threadIdx.x == 0) s_out[r] = amax / 127.f;
        return;
    }
    u32x4 v[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = threadIdx.x + i * kNormThreads;
        v[i] = c < n8 ? xr[c] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            amax = fmaxf(amax, fmaxf(fabsf(bf16lo_to_f32(v[i][j])), fabsf(bf16hi_to_f32(v[i][j]))));
    }
    amax = block_max(amax, red);
    const float inv = amax > 0.f ? 127.f / amax : 0.f;
    u32x2 *orow = reinterpret_cast<u32x2 *>(out + r * K);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = threadIdx.x + i * kNormThreads;
        if (c >= n8) continue;
        const u32x4 w = v[i];
        orow[c] = u32x2{q8x4(bf16lo_to_f32(w[0]), bf16hi_to_f32(w[0]), bf16lo_to_f32(w[1]), bf16hi_to_f32(w[1]), inv),
                        q8x4(bf16lo_to_f32(w[2]), bf16hi_to_f32(w[2]), bf16lo_to_f32(w[3]), bf16hi_to_f32(w[3]), inv)};
    }
    if (threadIdx.x == 0) s_out[r] = amax / 127.f;
}

hipError_t launch_modnorm_i8(const float *x, int rows, int D, const float *shift, const float *scale,
                             const float *norm_w, bool rms, float eps, int8_t *out, float *s, hipStream_t st,
                             bool rot) {
    if (rows <= 0) return hipSuccess;
    if (D % 4 != 0 || D > 16 * kNormThreads || (rot && D % 256 != 0)) return hipErrorInvalidValue;
    if (rot)
        k_modnorm_i8<true><<<rows, kNormThreads, 0, st>>>(x, D, shift, scale, norm_w, rms ? 1 : 0, eps, out, s);
    else
        k_modnorm_i8<false><<<rows, kNormThreads, 0, st>>>(x, D, shift, scale, norm_w, rms ? 1 : 0, eps, out, s);
    return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t *x, int rows, int K, int8_t *out, float *s, hipStream_t st, bool rot) {
    if (rows <= 0) return hipSuccess;
    if (K % 8 != 0 || K > 64 * kNormThreads || (rot && K % 256 != 0)) return hipErrorInvalidValue;
    if (rot)
        k_quant_rows<true><<<rows, kNormThreads, 0, st>>>(x, K, out, s);
    else
        k_quant_rows<false><<<rows, kNormThreads, 0, st>>>(x, K, out, s);
    return hipGetLastError();
}

hipError_t launch_modnorm(const float *x, int rows, int D, const float *shift, const float *scale,
                          const float *norm_w, bool rms, float eps, uint16_t *out, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    k_modnorm<<<rows, kNormThreads, 0, st>>>(x, D, shift, scale, norm_w, rms ? 1 : 0, eps, out);
    return hipGetLastError();
}

}  // namespace dit
