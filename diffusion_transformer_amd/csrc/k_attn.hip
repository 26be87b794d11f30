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
//  - the wave computes the TRANSPOSED scores S^T = K Q^T for a 64-key tile:
//    K (from LDS) is the A operand, the wave's queries (registers, loaded
//    once) the B operand.  A lane then holds one query column and 16 of its
//    keys, so the softmax statistics are per lane (plus two cross-lane
//    steps) and P^T is already in the B-operand layout of O^T += V^T P^T.
//  - values arrive feature-major (vt [H, 128, Sp], written that way by the
//    QKV product's epilogue), so V^T fragments are two 8-byte LDS reads.
//  - K and V^T tiles are double-buffered in LDS (64 KB per block, two blocks
//    per CU); XOR-swizzled chunk placement avoids bank conflicts.
//  - exp2 with log2(e) folded into the fp32 score scale; the row sum is kept
//    per lane and reduced once at the end.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {
constexpr int QB = 128;   // queries per block
constexpr int QW = 32;    // queries per wave
constexpr int KT = 64;    // keys per tile
constexpr int HD = 128;   // head dim
constexpr int NT = 256;
constexpr int K_U4 = KT * 16;     // K tile: 64 rows x 16 chunks
constexpr int V_U4 = HD * 8;      // V^T tile: 128 rows x 8 chunks
constexpr int STAGE = K_U4 + V_U4;

__device__ __forceinline__ int kidx(int row, int c) { return row * 16 + (c ^ (row & 15)); }
__device__ __forceinline__ int vidx(int d, int c) { return K_U4 + d * 8 + (c ^ ((d >> 1) & 7)); }
}  // namespace

__global__ void __launch_bounds__(NT)
k_attention(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kg,
            const uint16_t *__restrict__ Vt, int S, int ldv, uint16_t *__restrict__ O, int ldo) {
    __shared__ u32x4 lds[2 * STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y;
    const int q0 = blockIdx.x * QB + wave * QW;
    const int g = lane >> 4, l16 = lane & 15;

    const uint16_t *Qh = Q + static_cast<int64_t>(h) * S * HD;
    const uint16_t *Kh = Kg + static_cast<int64_t>(h) * S * HD;
    const uint16_t *Vh = Vt + static_cast<int64_t>(h) * HD * ldv;

    // queries of this lane as B operands: [tq][kstep over d]
    bf16x8 qf[2][4];
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
        const int qr = min(q0 + tq * 16 + l16, S - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qf[tq][ks] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(Qh + static_cast<int64_t>(qr) * HD + ks * 32 + g * 8));
    }

    // global -> LDS assignment
    const int kc = tid & 15, kr0 = tid >> 4;   // K: 4 rows (kr0 + 16 i), chunk kc
    const int vc = tid & 7, vr0 = tid >> 3;    // V^T: 4 rows (vr0 + 32 i), chunk vc
    u32x4 rk[4], rv[4];
    const int ntiles = (S + KT - 1) / KT;

    auto load_tile = [&](int t) {
        const int kv0 = t * KT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = min(kv0 + kr0 + 16 * i, S - 1);
            rk[i] = *reinterpret_cast<const u32x4 *>(Kh + static_cast<int64_t>(key) * HD + kc * 8);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = vr0 + 32 * i;
            u32x4 v = *reinterpret_cast<const u32x4 *>(Vh + static_cast<int64_t>(d) * ldv + kv0 + vc * 8);
            const int k8 = kv0 + vc * 8;
            if (k8 + 8 > S) {   // zero the values of keys >= S (their weights are 0)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    uint32_t w = v[j];
                    if (k8 + 2 * j >= S) w &= 0xffff0000u;
                    if (k8 + 2 * j + 1 >= S) w &= 0x0000ffffu;
                    v[j] = w;
                }
            }
            rv[i] = v;
        }
    };
    auto store_tile = [&](int buf) {
        u32x4 *L = lds + buf * STAGE;
#pragma unroll
        for (int i = 0; i < 4; ++i) L[kidx(kr0 + 16 * i, kc)] = rk[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) L[vidx(vr0 + 32 * i, vc)] = rv[i];
    };

    f32x4 oacc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrun[2] = {-INFINITY, -INFINITY};
    float lsum[2] = {0.f, 0.f};
    const float sc = 0.08838834764831845f * 1.4426950408889634f;   // log2(e) / sqrt(128)

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < ntiles) load_tile(t + 1);
        const u32x4 *L = lds + cur * STAGE;
        const int kv0 = t * KT;

        // ---- S^T = K Q^T for 64 keys x 32 queries
        f32x4 s[4][2];
#pragma unroll
        for (int tk = 0; tk < 4; ++tk)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) s[tk][tq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int tk = 0; tk < 4; ++tk) {
                const bf16x8 kf = __builtin_bit_cast(bf16x8, L[kidx(tk * 16 + l16, ks * 4 + g)]);
#pragma unroll
                for (int tq = 0; tq < 2; ++tq)
                    s[tk][tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[tq][ks], s[tk][tq], 0, 0, 0);
            }
        }

        // ---- online softmax per query column (lane); keys of this lane:
        // kv0 + tk*16 + 4g + r
        const bool tail = kv0 + KT > S;
        float alpha[2];
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) {
            float mx = -INFINITY;
#pragma unroll
            for (int tk = 0; tk < 4; ++tk)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = s[tk][tq][r] * sc;
                    if (tail && kv0 + tk * 16 + 4 * g + r >= S) v = -INFINITY;
                    s[tk][tq][r] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mnew = fmaxf(mrun[tq], mx);
            alpha[tq] = exp2f(mrun[tq] - mnew);
            mrun[tq] = mnew;
            float ps = 0.f;
#pragma unroll
            for (int tk = 0; tk < 4; ++tk)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float p = exp2f(s[tk][tq][r] - mnew);
                    s[tk][tq][r] = p;
                    ps += p;
                }
            lsum[tq] = lsum[tq] * alpha[tq] + ps;
        }
#pragma unroll
        for (int dd = 0; dd < 8; ++dd)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) oacc[dd][tq] *= alpha[tq];

        // ---- O^T += V^T P^T, two 32-key steps
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            bf16x8 pf[2];
#pragma unroll
            for (int tq = 0; tq < 2; ++tq) {
                const f32x4 a = s[2 * j][tq], b = s[2 * j + 1][tq];
                u32x4 u = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                           pack_bf16x2(b[2], b[3])};
                pf[tq] = __builtin_bit_cast(bf16x8, u);
            }
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                const int d = dd * 16 + l16;
                const u32x2 *L2 = reinterpret_cast<const u32x2 *>(L);
                const u32x2 lo = L2[2 * vidx(d, 4 * j + (g >> 1)) + (g & 1)];
                const u32x2 hi = L2[2 * vidx(d, 4 * j + 2 + (g >> 1)) + (g & 1)];
                const u32x4 u = {lo[0], lo[1], hi[0], hi[1]};
                const bf16x8 vf = __builtin_bit_cast(bf16x8, u);
#pragma unroll
                for (int tq = 0; tq < 2; ++tq)
                    oacc[dd][tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[tq], oacc[dd][tq], 0, 0, 0);
            }
        }

        if (t + 1 < ntiles) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- normalise and store o[q][h*128 + d], d = dd*16 + 4g + r
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
        float l = lsum[tq];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const float inv = 1.0f / l;
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
    dim3 grid(static_cast<unsigned>((S + QB - 1) / QB), static_cast<unsigned>(heads));
    k_attention<<<grid, NT, 0, st>>>(q, k, vt, S, ldv, o, ldo);
    return hipGetLastError();
}

}  // namespace dit
