// Joint full attention, flash-style, for gfx950.
//
// For each head: o = softmax(q k^T / sqrt(128)) v over all S rows, no mask
// ("944 -> 346 ms: optimizing FLUX.2 klein-4B on one TPU v6e chip" s.4.3:
// tile the queries, stream the keys and values through on-chip memory with a
// running row maximum and sum, rescaling the partial output when the
// maximum grows; the score scale is applied in fp32).
//
// Design (CDNA4, 64-wide waves, MFMA 16x16x32 bf16):
//  - block = 8 waves = 256 queries of one head, one block per CU; each wave
//    owns 32 queries.  The waves form two groups of four (one wave of each
//    per SIMD) that run half a key tile apart, so that on every SIMD one
//    wave feeds the matrix core while the other computes exponentials:
//
//      phase 2j   : group 0  PV(j-1), QK(j)   | group 1  softmax(j-1), loads K(j+1)
//      phase 2j+1 : group 0  softmax(j), loads V(j+1) | group 1  PV(j-1), QK(j)
//
//    (QK(j): scores of key tile j; softmax(j): their exponentials and the
//    running maximum; PV(j): the output and row-sum products of tile j).
//    A workgroup barrier ends every phase.
//  - the wave computes the TRANSPOSED scores S^T = K Q^T for a 64-key tile:
//    K (from LDS) is the A operand, the wave's queries (registers, loaded
//    once) the B operand.  A lane then holds one query column and 16 of its
//    keys, so P^T is already in the B-operand layout of O^T += V^T P^T.
//  - values arrive feature-major (vt [H, 128, Sp], as the QKV product's
//    epilogue writes them).  The K tile's rows are placed in LDS in the key
//    order kappa(r) = 8*((r%16)/4) + 4*(r/16) + r%4 within each 32 keys, so
//    the 8 scores a lane holds for one 32-key step are keys 8g .. 8g+7 and
//    each V^T fragment is a single 16-byte LDS read.
//  - K and V^T tiles go global -> LDS directly (buffer loads into LDS, no
//    register staging), issued during the softmax phases two tiles ahead:
//    K(j) is read in phases 2j and 2j+1 (three K buffers), V(j) in phases
//    2j+1 to 2j+3 (four V buffers); each load has two or more phases to
//    land.  In the
//    matrix phases the LDS fragment reads run two batches ahead of the MFMAs,
//    the first batch already issued at the end of the wave's softmax phase.
//  - the row sum is one more MFMA per 32 keys with an all-ones A operand
//    (it sums the same bf16-rounded P the values are weighted with); the
//    running maximum is rescaled lazily: only when a tile's maximum exceeds
//    it by more than 2^8 (exponents stay <= 2^8, exact either way), and
//    only upward, so no factor above 1 ever multiplies the partial sums.
//  - the score scale is applied in fp32: q enters the MFMAs exactly as
//    stored (bf16), the fp32 scores s = q.k are turned into base-2 exponent
//    units relative to the running maximum by one fused multiply-add each,
//    x = s * log2(e)/sqrt(128) - m, and p = 2^x; the maxima use three-input
//    max and lane-row swaps.
//  - blocks are remapped so that each XCD (own L2) serves whole heads.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {
constexpr int QB = 256;   // queries per block
constexpr int QW = 32;    // queries per wave
constexpr int KT = 64;    // keys per tile
constexpr int HD = 128;   // head dim
constexpr int NT = 512;
constexpr int K_U4 = KT * 16;     // K tile: 64 rows x 16 chunks of 16 B
constexpr int V_U4 = HD * 8;      // V^T tile: 128 rows x 8 chunks
constexpr int NKB = 3, NVB = 4;   // K and V^T buffers
constexpr float kLazy = 8.0f;     // rescale when the maximum grows by > 2^8

__device__ __forceinline__ int kidx(int row, int c) { return row * 16 + (c ^ (row & 15)); }
__device__ __forceinline__ int vidx(int d, int c) { return d * 8 + (c ^ ((d >> 1) & 7)); }

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

__device__ __forceinline__ void att_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void att_wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void att_wait_vm4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }
// lgkmcnt(0) as the builtin (vmcnt and expcnt fields at their maxima), so
// that the compiler's own wait insertion knows the LDS accesses completed
__device__ __forceinline__ void att_lgkm_done() { __builtin_amdgcn_s_waitcnt(0xc07f); }
}  // namespace

__global__ void __launch_bounds__(NT, 1)
k_attention(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kg,
            const uint16_t *__restrict__ Vt, int S, int ldv, int heads, uint16_t *__restrict__ O,
            int ldo, int Sq) {
    __shared__ u32x4 lds[NKB * K_U4 + NVB * V_U4];   // 112 KB
    u32x4 *const Kb = lds;
    u32x4 *const Vb = lds + NKB * K_U4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = wave >> 2, wg = wave & 3;
    const int g = lane >> 4, l16 = lane & 15;

    // XCD-compact order: consecutive work ids on one XCD share a head.
    // Queries are rows [0, Sq) (Sq <= S; q keeps the head stride S), keys
    // and values all S rows.
    const int nqb = (Sq + QB - 1) / QB;
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

    // queries of this lane as B operands: [tq][kstep over d], as stored
    bf16x8 qf[2][4];
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
        const int qr = min(q0 + tq * 16 + l16, Sq - 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qf[tq][ks] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(Qh + static_cast<int64_t>(qr) * HD + ks * 32 + g * 8));
    }
    // fp32 score scale in base-2 units: 1/sqrt(128) * log2(e)
    const float sc = 0.08838834764831845f * 1.4426950408889634f;

    const int ntiles = (S + KT - 1) / KT;
    // Direct global -> LDS through buffer loads, one wave instruction = 1 KB:
    // load i (0..3) of this wave moves LDS K rows r = 16wg + 4i + (lane>>4)
    // or V^T rows d = 32wg + 8i + (lane>>3) of a tile; each lane fetches the
    // global chunk that belongs at its LDS position under the XOR swizzle.
    // Both offsets are one per-lane base XOR (i's chunk bits) plus a uniform
    // step:
    //   K row r holds key kappa(r) = 32(wg>>1) + 4(wg&1) + (lane>>4) + 8i and
    //     chunk (lane&15) ^ (4i + (lane>>4));
    //   V^T row d takes chunk (lane&7) ^ (lane>>4) ^ 4(i&1).
    // The K descriptor ends at row S, so keys past S read as zeros (their
    // scores are masked); the V^T descriptor covers all Sp columns.
    const __amdgpu_buffer_rsrc_t rK =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(Kh), static_cast<short>(0), S * HD * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rV =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(Vh), static_cast<short>(0), HD * ldv * 2, 0x00020000);
    const int lg = lane >> 4;
    const uint32_t k_lane = static_cast<uint32_t>((32 * (wg >> 1) + 4 * (wg & 1) + lg) * HD * 2 + (((lane & 15) ^ lg) << 4));
    const uint32_t v_lane = static_cast<uint32_t>((32 * wg + (lane >> 3)) * ldv * 2 + ((((lane & 7) ^ lg)) << 4));
    auto issue_k = [&](int t, int i) {
        const uint32_t off = (k_lane ^ static_cast<uint32_t>(i << 6)) + static_cast<uint32_t>((t * KT + 8 * i) * HD * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_void *)(Kb + (t % NKB) * K_U4 + (wg * 4 + i) * 64), 16, off, 0, 0, 0);
    };
    auto issue_v = [&](int t, int i) {
        const uint32_t off = (v_lane ^ static_cast<uint32_t>((i & 1) << 6)) + static_cast<uint32_t>(8 * i * ldv * 2 + t * KT * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_void *)(Vb + (t % NVB) * V_U4 + (wg * 4 + i) * 64), 16, off, 0, 0, 0);
    };
    // keys >= S of the last tile: zero their values in LDS, so that a 0
    // weight never meets padding (which may hold anything); by group 0
    const int last = ntiles - 1, valid_last = S - last * KT;
    auto zero_tail = [&]() {
        if (valid_last == KT) return;
        uint16_t *V16 = reinterpret_cast<uint16_t *>(Vb + (last % NVB) * V_U4);
        for (int e = tid; e < HD * KT; e += NT / 2) {
            const int d = e / KT, key = e % KT;
            if (key >= valid_last) V16[vidx(d, key >> 3) * 8 + (key & 7)] = 0;
        }
    };

    f32x4 oacc[8][2], rsum[2], s[4][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    rsum[0] = rsum[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // running maximum (base-2 units) per query, subtracted from the scaled
    // scores in the softmax.  mb = 0 and started = false until the first
    // tile has set it.
    float mb[2] = {0.f, 0.f};
    bool started = false;
    const u32x4 ones_u = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_u);
    bf16x8 pf[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) pf[j][tq] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

    // ---- the matrix phase: O^T += V^T P^T and the row sums of tile tv (two
    // 32-key steps; its first V^T fragments are already in fa), then
    // S^T = K Q^T of tile tk (64 keys x 32 queries; s[tk][tq][r] holds the
    // fp32 score q.k of key 32*(tk/2) + 8g + 4*(tk%2) + r).
    // The LDS reads go in quarters of 4 fragments, written two quarters
    // before the MFMAs that use them; the compiler interleaves the reads and
    // the MFMAs within the phase (no scheduling fences: measured 4 % faster
    // than keeping each quarter's reads ahead of the MFMAs by a fence).
    bf16x8 fa[8], fb[8];
    auto prefetch_v = [&](int t) {   // V^T fragments of keys 8g .. 8g+7 of tile t >= -1
        const u32x4 *L = Vb + ((t + NVB) % NVB) * V_U4;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) fa[dd] = __builtin_bit_cast(bf16x8, L[vidx(dd * 16 + l16, g)]);
    };
    // quarter h (0, 1) of the V^T fragments of 32-key step j; of the K
    // fragments of k-step ks
    auto read_v4 = [&](bf16x8 *f, const u32x4 *L, int j, int h) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            f[u] = __builtin_bit_cast(bf16x8, L[vidx((4 * h + u) * 16 + l16, 4 * j + g)]);
    };
    auto read_k4 = [&](bf16x8 *f, const u32x4 *L, int ks) {
#pragma unroll
        for (int tk = 0; tk < 4; ++tk) f[tk] = __builtin_bit_cast(bf16x8, L[kidx(tk * 16 + l16, ks * 4 + g)]);
    };
    auto pv4 = [&](const bf16x8 *f, int j, int h) {   // value rows 64h .. 64h+63 of step j
        if (h == 0) {
#pragma unroll
            for (int tq = 0; tq < 2; ++tq)
                rsum[tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[j][tq], rsum[tq], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq)
                oacc[4 * h + u][tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[u], pf[j][tq], oacc[4 * h + u][tq], 0, 0, 0);
    };
    auto qk4 = [&](const bf16x8 *f, int ks) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tk = 0; tk < 4; ++tk)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq)
                s[tk][tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[tk], qf[tq][ks], ks == 0 ? zero : s[tk][tq], 0, 0, 0);
    };
    // tv = -1 (the first matrix phase) reads V^T buffer NVB-1, which is
    // zeroed before the loop, with P = 0; tk = ntiles (the last) computes
    // scores that are never used: the phase has no branches
    auto mma = [&](int tv, int tk) {
        const u32x4 *LK = Kb + (tk % NKB) * K_U4;
        const u32x4 *LV = Vb + ((tv + NVB) % NVB) * V_U4;
#define DIT_STEP(read, use) do { read; use; } while (0)
        DIT_STEP(read_v4(fb, LV, 1, 0), pv4(fa, 0, 0));
        DIT_STEP(read_v4(fb + 4, LV, 1, 1), pv4(fa + 4, 0, 1));
        DIT_STEP(read_k4(fa, LK, 0), pv4(fb, 1, 0));
        DIT_STEP(read_k4(fa + 4, LK, 1), pv4(fb + 4, 1, 1));
        DIT_STEP(read_k4(fb, LK, 2), qk4(fa, 0));
        DIT_STEP(read_k4(fb + 4, LK, 3), qk4(fa + 4, 1));
        qk4(fb, 2);
        qk4(fb + 4, 3);
#undef DIT_STEP
    };

    // ---- online softmax of tile t: x = s * sc - mb (one fma each).  Common
    // case: the tile's maximum of x is <= 2^8 above the running maximum and
    // p = 2^x needs no further subtraction.  Otherwise the maximum moves up
    // by the tile's max m (never down: m >= 0 once started) and the partial
    // output and sums are scaled by 2^-m <= 1, p = 2^(x - m).  The first
    // tile sets the maximum to its own (any value); the partial results are
    // still zero then and are not scaled.
    auto softmax = [&](int t) {
        const int kv0 = t * KT;
#pragma unroll
        for (int tk = 0; tk < 4; ++tk)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq)
#pragma unroll
                for (int r = 0; r < 4; ++r) s[tk][tq][r] = __builtin_fmaf(s[tk][tq][r], sc, -mb[tq]);
        if (kv0 + KT > S) {
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
                const float m = started ? fmaxf(mt[tq], 0.f) : mt[tq];
                if (started) {
                    const float alpha = __builtin_amdgcn_exp2f(-m);
#pragma unroll
                    for (int dd = 0; dd < 8; ++dd) oacc[dd][tq] *= alpha;
                    rsum[tq] *= alpha;
                }
                mb[tq] += m;
#pragma unroll
                for (int tk = 0; tk < 4; ++tk) s[tk][tq] -= m;
            }
            started = true;
        }
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
    };

    // prologue: group 0 loads K(0) and K(1), group 1 V(0) and V(1); V^T
    // buffer NVB-1 (first used by V(NVB-1)) is zeroed for the branch-free
    // first matrix phase
    for (int t = 0; t < min(2, ntiles); ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (grp == 0) issue_k(t, i);
            else issue_v(t, i);
        }
    for (int e = tid; e < V_U4; e += NT) Vb[(NVB - 1) * V_U4 + e] = u32x4{0u, 0u, 0u, 0u};
    att_wait_vm0();
    att_lgkm_done();
    att_barrier();
    if (grp == 0 && last == 0) zero_tail();
    att_lgkm_done();
    att_barrier();
    if (grp == 0) {
        prefetch_v(-1);
        att_lgkm_done();
    }

    // Main loop over the phases.  Loads and waits: group 1 issues K(j+2) in
    // phase 2j (K(j+2) reuses the buffer of K(j-1), last read in 2j-1) and
    // waits for K(j+1) at the end of 2j+1 (read from 2j+2 on); group 0
    // issues V(j+2) in phase 2j+1 (the buffer of V(j-2), last read in 2j-1)
    // and waits for V(j) at the end of 2j, where it also zeroes the padding
    // keys of the last tile's values (read from 2j+1 on: each group fetches
    // the first V^T fragments of tile j at the end of its softmax phase
    // before PV(j)).  A wait leaves in flight the 4 loads issued after the
    // ones it needs, if there were any.
    for (int j = 0; j <= ntiles; ++j) {
        // phase 2j
        if (grp == 0) {
            mma(j - 1, j);
            if (j + 1 < ntiles) att_wait_vm4();   // V(j) has landed, V(j+1) may not
            else att_wait_vm0();
            if (j == last && j > 0) zero_tail();
            att_lgkm_done();
        } else {
            if (j >= 1) softmax(j - 1);
            if (j + 2 < ntiles) {
#pragma unroll
                for (int i = 0; i < 4; ++i) issue_k(j + 2, i);
            }
            prefetch_v(j - 1);
            att_lgkm_done();
        }
        att_barrier();
        // phase 2j+1
        if (grp == 0) {
            if (j < ntiles) {
                softmax(j);
                if (j + 2 < ntiles) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) issue_v(j + 2, i);
                }
                prefetch_v(j);
                att_lgkm_done();
            }
        } else {
            mma(j - 1, j);
            if (j + 2 < ntiles) att_wait_vm4();   // K(j+1) has landed, K(j+2) may not
            else att_wait_vm0();
        }
        att_barrier();
    }

    // ---- normalise and store o[q][h*128 + d], d = dd*16 + 4g + r
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
        const float inv = 1.0f / rsum[tq][0];
        const int q = q0 + tq * 16 + l16;
        if (q >= Sq) continue;
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
                            int S, int ldv, uint16_t *o, int ldo, hipStream_t st, int Sq) {
    if (Sq < 0) Sq = S;
    if (S <= 0 || heads <= 0 || Sq == 0) return hipSuccess;
    if (Sq > S) return hipErrorInvalidValue;
    const int grid = ((Sq + QB - 1) / QB) * heads;
    k_attention<<<grid, NT, 0, st>>>(q, k, vt, S, ldv, heads, o, ldo, Sq);
    return hipGetLastError();
}

}  // namespace dit
