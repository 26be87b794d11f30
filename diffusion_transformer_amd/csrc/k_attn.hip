// Joint full attention, flash-style, for gfx950.
//
// For each head: o = softmax(q k^T / sqrt(128)) v over all S rows, no mask
// ("944 -> 346 ms: optimizing FLUX.2 klein-4B on one TPU v6e chip" s.4.3:
// tile the queries, stream the keys and values through on-chip memory with a
// running row maximum and sum, rescaling the partial output when the
// maximum grows; the score scale is applied in fp32).
//
// Design (CDNA4, 64-wide waves, MFMA 16x16x32 bf16):
//  - block = 4 waves = 128 queries of one head; each wave owns 32 queries.
//    Two blocks share a CU (<= 256 registers per lane, 64 KB LDS each), so
//    each SIMD interleaves one wave's exponentials with the other's MFMAs.
//  - the wave computes the TRANSPOSED scores S^T = K Q^T for a 64-key tile:
//    K (from LDS) is the A operand, the wave's queries (registers, loaded
//    once) the B operand.  A lane then holds one query column and 16 of its
//    keys, so P^T is already in the B-operand layout of O^T += V^T P^T.
//  - values arrive feature-major (vt [H, 128, Sp], as the QKV product's
//    epilogue writes them).  The K tile's rows are placed in LDS in the key
//    order kappa(r) = 8*((r%16)/4) + 4*(r/16) + r%4 within each 32 keys, so
//    the 8 scores a lane holds for one 32-key step are keys 8g .. 8g+7 and
//    each V^T fragment is a single 16-byte LDS read.
//  - K and V^T tiles go global -> LDS directly (global_load_lds_dwordx4,
//    no register staging), double-buffered; each lane fetches the global
//    chunk that belongs at its LDS position under the XOR swizzle.
//  - the row sum is one more MFMA per 32 keys with an all-ones A operand
//    (it sums the same bf16-rounded P the values are weighted with);
//    the running maximum is rescaled lazily: only when a tile's maximum
//    exceeds it by more than 2^8 (exponents stay <= 2^8, exact either way).
//  - the exponentials are the vector-unit bottleneck, so the softmax is
//    trimmed to them: queries are pre-multiplied by log2(e)/sqrt(128) and the
//    score MFMAs start from minus the running maximum, so p = 2^score needs
//    no separate scale-and-subtract; the maxima use three-input max and
//    lane-row swaps.
//  - blocks are remapped so that each XCD (own L2) serves whole heads.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {
constexpr int QB = 128;   // queries per block
constexpr int QW = 32;    // queries per wave
constexpr int KT = 64;    // keys per tile
constexpr int HD = 128;   // head dim
constexpr int NT = 256;
constexpr int K_U4 = KT * 16;     // K tile: 64 rows x 16 chunks of 16 B
constexpr int V_U4 = HD * 8;      // V^T tile: 128 rows x 8 chunks
constexpr int STAGE = K_U4 + V_U4;
constexpr float kLazy = 8.0f;     // rescale when the maximum grows by > 2^8

__device__ __forceinline__ int kidx(int row, int c) { return row * 16 + (c ^ (row & 15)); }
__device__ __forceinline__ int vidx(int d, int c) { return K_U4 + d * 8 + (c ^ ((d >> 1) & 7)); }

typedef __attribute__((address_space(3))) void lds_void;

// max with the lane 16 (32) positions away, through the gfx950 row-swap
// permutes (no LDS round trip): swapping a value with itself leaves each
// lane holding its own value in one result and its partner's in the other
__device__ __forceinline__ float fmax_xor16(float v) {
    const unsigned u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float fmax_xor32(float v) {
    const unsigned u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ void g2l16(const void *g, u32x4 *l) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)(l), 16, 0, 0);
}
}  // namespace

__global__ void __launch_bounds__(NT, 2)
k_attention(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kg,
            const uint16_t *__restrict__ Vt, int S, int ldv, int heads, uint16_t *__restrict__ O,
            int ldo) {
    __shared__ u32x4 lds[2 * STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;

    // XCD-compact order: consecutive work ids on one XCD share a head
    const int nqb = (S + QB - 1) / QB;
    const int total = nqb * heads;
    int bid = blockIdx.x;
    {
        const int per = total / 8, rem = total % 8, xcd = bid % 8, loc = bid / 8;
        bid = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    }
    const int h = bid / nqb;
    const int q0 = (bid % nqb) * QB + wave * QW;

    const uint16_t *Qh = Q + static_cast<int64_t>(h) * S * HD;
    const uint16_t *Kh = Kg + static_cast<int64_t>(h) * S * HD;
    const uint16_t *Vh = Vt + static_cast<int64_t>(h) * HD * ldv;

    // queries of this lane as B operands: [tq][kstep over d], multiplied by
    // log2(e)/sqrt(128) (and rounded to bf16 again) so that the scores come
    // out of the MFMAs in base-2 exponent units
    const float sc = 0.08838834764831845f * 1.4426950408889634f;
    bf16x8 qf[2][4];
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
        const int qr = min(q0 + tq * 16 + l16, S - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(Qh + static_cast<int64_t>(qr) * HD + ks * 32 + g * 8);
            const u32x4 u = {pack_bf16x2(bf16lo_to_f32(w[0]) * sc, bf16hi_to_f32(w[0]) * sc),
                             pack_bf16x2(bf16lo_to_f32(w[1]) * sc, bf16hi_to_f32(w[1]) * sc),
                             pack_bf16x2(bf16lo_to_f32(w[2]) * sc, bf16hi_to_f32(w[2]) * sc),
                             pack_bf16x2(bf16lo_to_f32(w[3]) * sc, bf16hi_to_f32(w[3]) * sc)};
            qf[tq][ks] = __builtin_bit_cast(bf16x8, u);
        }
    }

    const int ntiles = (S + KT - 1) / KT;
    // direct global -> LDS: wave instruction i writes 1 KB = 4 K rows or 8 V^T rows
    // load i (0..7) of tile t: i < 4 the K rows, else the V^T rows
    auto issue_one = [&](int t, int buf, int i) {
        const int kv0 = t * KT;
        u32x4 *L = lds + buf * STAGE;
        const int blk = wave * 4 + (i & 3);               // 0..15
        if (i < 4) {
            const int r = blk * 4 + (lane >> 4);          // LDS K row 0..63
            const int c = (lane & 15) ^ (r & 15);         // global chunk for LDS position lane&15
            const int rr = r & 31;
            const int kk = (r & 32) + 8 * ((rr & 15) >> 2) + 4 * (rr >> 4) + (rr & 3);   // kappa
            const int key = min(kv0 + kk, S - 1);
            g2l16(Kh + static_cast<int64_t>(key) * HD + c * 8, L + blk * 64);
        } else {
            const int d = blk * 8 + (lane >> 3);          // V^T row 0..127
            const int c = (lane & 7) ^ ((d >> 1) & 7);
            g2l16(Vh + static_cast<int64_t>(d) * ldv + kv0 + c * 8, L + K_U4 + blk * 64);
        }
    };
    auto issue_tile = [&](int t, int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) issue_one(t, buf, i);
    };

    f32x4 oacc[8][2], rsum[2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    rsum[0] = rsum[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // running maximum (base-2 units) per query; the score MFMAs start from
    // -mb, so the scores arrive with it already subtracted.  mb = 0 and
    // started = false until the first tile has set it.
    float mb[2] = {0.f, 0.f};
    bool started = false;
    const u32x4 ones_u = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_u);

    issue_tile(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        const int kv0 = t * KT;
        const bool tail = kv0 + KT > S;
        if (tail) {
            // keys >= S: zero their values so that 0-weight * garbage stays 0
            u32x4 *L = lds + cur * STAGE;
            uint16_t *V16 = reinterpret_cast<uint16_t *>(L + K_U4);
            const int valid = S - kv0;
            for (int e = tid; e < HD * KT; e += NT) {
                const int d = e / KT, key = e % KT;
                if (key >= valid) {
                    const int c = key >> 3;
                    V16[(d * 8 + (c ^ ((d >> 1) & 7))) * 8 + (key & 7)] = 0;
                }
            }
            __syncthreads();
        }
        const u32x4 *L = lds + cur * STAGE;

        // ---- S^T = K Q^T for 64 keys x 32 queries (raw scores), with the
        // next tile's 8 loads into LDS spread between the MFMAs: issued in a
        // row they stall the wave on the vector-memory queue.  The last tile
        // loads itself again (into the idle buffer) to keep one code path.
        const int tn = min(t + 1, ntiles - 1);
        f32x4 s[4][2];
        const f32x4 init[2] = {f32x4{-mb[0], -mb[0], -mb[0], -mb[0]}, f32x4{-mb[1], -mb[1], -mb[1], -mb[1]}};
        bf16x8 kf[4][4];                                   // all K fragments first (LDS reads
#pragma unroll                                            // may not pass the loads into LDS)
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int tk = 0; tk < 4; ++tk) kf[ks][tk] = __builtin_bit_cast(bf16x8, L[kidx(tk * 16 + l16, ks * 4 + g)]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int tk = 0; tk < 4; ++tk) {
                if ((tk & 1) == 0) issue_one(tn, cur ^ 1, ks * 2 + (tk >> 1));
#pragma unroll
                for (int tq = 0; tq < 2; ++tq)
                    s[tk][tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks][tk], qf[tq][ks], ks == 0 ? init[tq] : s[tk][tq], 0, 0, 0);
            }
        }

        // ---- online softmax per query column (lane): s[tk][tq][r] holds
        // x = score * log2(e)/sqrt(128) - mb for key kv0 + 32*(tk/2) + 8g +
        // 4*(tk%2) + r.  Common case: the tile's maximum of x is <= 2^8 above
        // the running maximum and p = 2^x needs no subtraction.  Otherwise
        // (and for the first tile) the maximum moves up by the tile's max m:
        // the partial output and sums are scaled by 2^-m and p = 2^(x - m).
        if (tail) {
#pragma unroll
            for (int tk = 0; tk < 4; ++tk)
#pragma unroll
                for (int tq = 0; tq < 2; ++tq)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (kv0 + 32 * (tk >> 1) + 8 * g + 4 * (tk & 1) + r >= S) s[tk][tq][r] = -INFINITY;
        }
        float mt[2];
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) {
            float m0 = fmaxf(s[0][tq][0], s[0][tq][1]), m1 = fmaxf(s[0][tq][2], s[0][tq][3]);
#pragma unroll
            for (int tk = 1; tk < 4; ++tk) {
                m0 = fmaxf(fmaxf(m0, s[tk][tq][0]), s[tk][tq][1]);   // v_max3
                m1 = fmaxf(fmaxf(m1, s[tk][tq][2]), s[tk][tq][3]);
            }
            mt[tq] = fmax_xor32(fmax_xor16(fmaxf(m0, m1)));
        }
        const bool grow = !started || mt[0] > kLazy || mt[1] > kLazy;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) {
                const float m = mt[tq];
                const float alpha = __builtin_amdgcn_exp2f(-m);
#pragma unroll
                for (int dd = 0; dd < 8; ++dd) oacc[dd][tq] *= alpha;
                rsum[tq] *= alpha;
                mb[tq] += m;
#pragma unroll
                for (int tk = 0; tk < 4; ++tk) s[tk][tq] -= m;
            }
            started = true;
        }
        bf16x8 pf[2][2];
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const f32x4 a = s[2 * j][tq], b = s[2 * j + 1][tq];
                u32x4 u = {pack_bf16x2(__builtin_amdgcn_exp2f(a[0]), __builtin_amdgcn_exp2f(a[1])),
                           pack_bf16x2(__builtin_amdgcn_exp2f(a[2]), __builtin_amdgcn_exp2f(a[3])),
                           pack_bf16x2(__builtin_amdgcn_exp2f(b[0]), __builtin_amdgcn_exp2f(b[1])),
                           pack_bf16x2(__builtin_amdgcn_exp2f(b[2]), __builtin_amdgcn_exp2f(b[3]))};
                pf[j][tq] = __builtin_bit_cast(bf16x8, u);
            }
        }

        // ---- O^T += V^T P^T and the row sums, two 32-key steps
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int tq = 0; tq < 2; ++tq)
                rsum[tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[j][tq], rsum[tq], 0, 0, 0);
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                // keys 32j + 8g .. +7 of value row d: one 16-byte chunk
                const bf16x8 vf = __builtin_bit_cast(bf16x8, L[vidx(dd * 16 + l16, 4 * j + g)]);
#pragma unroll
                for (int tq = 0; tq < 2; ++tq)
                    oacc[dd][tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[j][tq], oacc[dd][tq], 0, 0, 0);
            }
        }

        __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile t+1 have landed
        __syncthreads();                 // everyone's have, and nobody still reads tile t
    }

    // ---- normalise and store o[q][h*128 + d], d = dd*16 + 4g + r
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
        const float inv = 1.0f / rsum[tq][0];
        const int q = q0 + tq * 16 + l16;
        if (q >= S) continue;
        uint16_t *orow = O + static_cast<int64_t>(q) * ldo + h * HD;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            const f32x4 a = oacc[dd][tq];
            *reinterpret_cast<u32x2 *>(orow + dd * 16 + 4 * g) =
                u32x2{pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv)};
        }
    }
}

hipError_t launch_attention(const uint16_t *q, const uint16_t *k, const uint16_t *vt, int heads,
                            int S, int ldv, uint16_t *o, int ldo, hipStream_t st) {
    if (S <= 0 || heads <= 0) return hipSuccess;
    const int grid = ((S + QB - 1) / QB) * heads;
    k_attention<<<grid, NT, 0, st>>>(q, k, vt, S, ldv, heads, o, ldo);
    return hipGetLastError();
}

}  // namespace dit
