// Joint full attention, flash-style, for gfx950.
//
// For each head: o = softmax(q k^T / sqrt(128)) v over all S rows, no mask
// ("944 -> 346 ms: optimizing FLUX.2 klein-4B on one TPU v6e chip" s.4.3:
// tile the queries, stream the keys and values through on-chip memory with a
// running row maximum and sum, rescaling the partial output when the
// maximum grows; the score scale is applied in fp32).
//
// Design (CDNA4, 64-wide waves, MFMA 16x16x32 bf16):
//  - block = 8 waves = 256 queries of one head, one block per CU (two waves
//    per SIMD); each wave owns 32 queries and runs a software pipeline over
//    the 64-key tiles on its own:
//
//      tile j, half A: QK(j+1) MFMAs  interleaved with  exp2 + bf16 pack of tile j
//      tile j, half B: PV(j) MFMAs    interleaved with  scale + lane maxima of tile j+1
//
//    (QK(t): scores of key tile t; PV(t): the output and row-sum products of
//    tile t).  On gfx950 a wave's vector instructions overlap its own
//    independent MFMAs far better than another wave's on the same SIMD, so
//    each wave keeps the matrix core fed with its own softmax work in
//    between; sched_barrier fences hold the slots (and the slots hold no
//    branches, past which the compiler would sink the exponentials).  A
//    workgroup barrier ends every tile; wave priorities stepped down through
//    each tile keep the two waves of a SIMD level with each other.
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
//    register staging), three buffers each: in tile j the block reads K(j+1)
//    and V(j) and loads K(j+3) and V(j+2).  Fragments are read from LDS two
//    MFMA slots ahead of their use.
//  - the row sum is one more MFMA per 32 keys with an all-ones A operand
//    (it sums the same bf16-rounded P the values are weighted with); the
//    running maximum is rescaled lazily: only when a tile's scores exceed
//    it by more than 2^8 (exponents stay <= 2^8, exact either way), and
//    only upward, so no factor above 1 ever multiplies the partial sums.
//    Each lane checks its own 32 scores with three-input maxima; the row
//    maxima (lane-row swaps) are only taken when some lane finds one above.
//  - the score scale is applied in fp32: q enters the MFMAs exactly as
//    stored (bf16), the fp32 scores s = q.k are turned into base-2 exponent
//    units relative to the running maximum by one fused multiply-add each,
//    x = s * log2(e)/sqrt(128) - m, and p = 2^x.
//  - blocks are remapped so that each XCD (own L2) serves whole heads.
#include <type_traits>

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
constexpr int NKB = 3, NVB = 3;   // K and V^T buffers
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
    __shared__ u32x4 lds[NKB * K_U4 + NVB * V_U4];   // 96 KB
    u32x4 *const Kb = lds;
    u32x4 *const Vb = lds + NKB * K_U4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wg = wave & 3, i0 = 2 * (wave >> 2);
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
    // load i (0..3) of the wave pair (w, w+4) moves LDS K rows
    // r = 16wg + 4i + (lane>>4) or V^T rows d = 32wg + 8i + (lane>>3) of a
    // tile (wave w takes i = 0, 1, wave w+4 i = 2, 3); each lane fetches the
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
    // weight never meets padding (which may hold anything)
    const int last = ntiles - 1, valid_last = S - last * KT;
    auto zero_tail = [&]() {
        uint16_t *V16 = reinterpret_cast<uint16_t *>(Vb + (last % NVB) * V_U4);
        for (int e = tid; e < HD * KT; e += NT) {
            const int d = e / KT, key = e % KT;
            if (key >= valid_last) V16[vidx(d, key >> 3) * 8 + (key & 7)] = 0;
        }
    };

    f32x4 oacc[8][2], rsum[2], sa[4][2], sb[4][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) oacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    rsum[0] = rsum[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // running maximum (base-2 units) per query, subtracted from the scaled
    // scores.  mb = 0 and started = false until the first tile has set it.
    float mb[2] = {0.f, 0.f}, mt[2], m0[2], m1[2];
    bool started = false;
    const u32x4 ones_u = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_u);
    bf16x8 kb[3], vb[3];
    u32x4 pu[2][2];   // P of the tile, bf16 pairs: [32-key step][query block]

    // s[tk][tq][r]: fp32 score q.k of key 32*(tk/2) + 8g + 4*(tk%2) + r of
    // the tile (the K row order kappa) and query tq*16 + (lane & 15).
    // QK slot i (0..15): the 16-key rows tk = i/4, k-step ks = i%4 (32 of
    // d), both query blocks (row-major, so each score block completes, and
    // the previous tile's scores die, as the slots go); its K fragment goes
    // into ring entry i%3
    auto read_k = [&](const u32x4 *L, int i) {
        kb[i % 3] = __builtin_bit_cast(bf16x8, L[kidx((i / 4) * 16 + l16, (i % 4) * 4 + g)]);
    };
    auto qk_m = [&](f32x4 (&s)[4][2], int i, int tq) {
        const int ks = i % 4, tk = i / 4;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        s[tk][tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[i % 3], qf[tq][ks], ks == 0 ? zero : s[tk][tq], 0, 0, 0);
    };
    // the pair p (0..15) of exponentials p = 2^x of one lane's 32, packed
    // to bf16: query tq = p/8, 32-key step j = (p/4)%2, word w = p%4
    auto exp_pair = [&](f32x4 (&s)[4][2], int p) {
        const int tq = p / 8, j = (p / 4) % 2, w = p % 4;
        const f32x4 &v = s[2 * j + (w >> 1)][tq];
        const int r = 2 * (w & 1);
        pu[j][tq][w] = pack_bf16x2(__builtin_amdgcn_exp2f(v[r]), __builtin_amdgcn_exp2f(v[r + 1]));
    };
    // V^T fragment of PV slot i (0..17: 32-key step i/9, value rows
    // 16*(i%9); i%9 = 8 is the row-sum pair) into the ring
    auto read_v = [&](const u32x4 *L, int i) {
        const int j = i / 9, dd = i % 9;
        if (dd < 8) vb[i % 3] = __builtin_bit_cast(bf16x8, L[vidx(dd * 16 + l16, 4 * j + g)]);
    };
    auto pv_m = [&](int i, int tq) {
        const int j = i / 9, dd = i % 9;
        const bf16x8 p = __builtin_bit_cast(bf16x8, pu[j][tq]);
        if (dd == 8) rsum[tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, p, rsum[tq], 0, 0, 0);
        else oacc[dd][tq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[i % 3], p, oacc[dd][tq], 0, 0, 0);
    };
    // x = s * sc - mb for 4 of the 32 scores (piece k of 8), from the
    // products' s into x
    auto scale4 = [&](f32x4 (&x)[4][2], const f32x4 (&s)[4][2], int k) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int n = 4 * k + e, tk = n / 8, tq = (n / 4) % 2, r = n % 4;
            x[tk][tq][r] = __builtin_fmaf(s[tk][tq][r], sc, -mb[tq]);
        }
    };
    // the tile's maximum of x per query in 10 pieces (v_max3 chains, then
    // the row's lanes through the row-swap permutes)
    auto max_piece = [&](f32x4 (&s)[4][2], int k) {
        const int tq = k / 5, q = k % 5;
        auto v = [&](int e) { return s[e / 4][tq][e % 4]; };
        if (q == 0) { m0[tq] = fmaxf(fmaxf(v(0), v(1)), v(4)); m1[tq] = fmaxf(fmaxf(v(2), v(3)), v(6)); }
        if (q == 1) { m0[tq] = fmaxf(fmaxf(m0[tq], v(5)), v(8)); m1[tq] = fmaxf(fmaxf(m1[tq], v(7)), v(10)); }
        if (q == 2) { m0[tq] = fmaxf(fmaxf(m0[tq], v(9)), v(12)); m1[tq] = fmaxf(fmaxf(m1[tq], v(11)), v(14)); }
        if (q == 3) m0[tq] = fmaxf(fmaxf(m0[tq], v(13)), fmaxf(m1[tq], v(15)));
        if (q == 4) mt[tq] = fmax_xor32(fmax_xor16(m0[tq]));
    };
    // keys >= S of tile t get x = -inf (p = 0); selects, no branches
    auto mask = [&](f32x4 (&s)[4][2], int t) {
        const int lim = S - t * KT - 8 * g;
#pragma unroll
        for (int tk = 0; tk < 4; ++tk)
#pragma unroll
            for (int tq = 0; tq < 2; ++tq)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s[tk][tq][r] = 32 * (tk >> 1) + 4 * (tk & 1) + r >= lim ? -INFINITY : s[tk][tq][r];
    };
    // the lane's largest x of the tile (over both query blocks) in 8 pieces
    // of two three-input maxima: all the common case needs to know
    float lm = -INFINITY;
    auto lane_max_piece = [&](const f32x4 (&s)[4][2], int k) {
        const int tk = k / 2, tq = k % 2;
        lm = fmaxf(fmaxf(lm, s[tk][tq][0]), s[tk][tq][1]);
        lm = fmaxf(fmaxf(lm, s[tk][tq][2]), s[tk][tq][3]);
    };
    // ---- the running maximum after a tile's x and maxima mt.  Common case:
    // the tile's maximum is <= 2^8 above the running maximum and p = 2^x
    // needs no further subtraction.  Otherwise the maximum moves up by m
    // (never down: m >= 0 once started) and the partial output and sums
    // (which hold every earlier tile) are scaled by 2^-m <= 1, p = 2^(x - m).
    // The first tile sets the maximum to its own (any value); the partial
    // results are still zero then and are not scaled.
    auto rescale = [&](f32x4 (&s)[4][2]) {
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
    };
    auto settle = [&](f32x4 (&s)[4][2]) {
        const bool grow = !started || mt[0] > kLazy || mt[1] > kLazy;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) rescale(s);
    };
    // in the tiles after the first: rescale only when some x of the tile
    // exceeds kLazy (the lane maxima tell); the row maxima are then taken
    auto settle_lazy = [&](f32x4 (&s)[4][2]) {
        if (__builtin_amdgcn_ballot_w64(lm > kLazy) != 0) {
#pragma unroll
            for (int k = 0; k < 10; ++k) max_piece(s, k);
            rescale(s);
        }
    };

    // One key tile j < last, on the scaled scores x (sa) of tile j.  Half A:
    // the products' scores of tile j+1 (S^T = K Q^T into sb, 32 MFMAs, K
    // fragments two slots ahead) interleaved with the exponentials of tile
    // j; half B: the output and row-sum products of tile j (36 MFMAs, V^T
    // fragments two slots ahead) interleaved with the scale (sb into sa) and
    // maxima of tile j+1.  So every wave keeps its matrix core fed with its
    // own vector work in between (sched_barrier fences keep the slots; the
    // slots hold no branches, which would let the compiler sink work past
    // them).  K(t), V(t) live in LDS buffers t % 3: during tile j the block
    // reads K(j+1) and V(j) and loads K(j+3) and V(j+2) into the buffers of
    // K(j) and V(j-1), read in tile j-1.  The loads are issued in every
    // tile: past the last tile they fetch zeros (the descriptors' bounds)
    // into a buffer no later tile reads.  Each wave waits for its loads of
    // tile j-1 at the end of tile j, and one barrier ends every tile.  The
    // form for j = last-1 also masks the keys past S of tile j+1.
    auto step = [&](auto last_tag, int j) {
        const u32x4 *LK = Kb + ((j + 1) % NKB) * K_U4;
        const u32x4 *LV = Vb + (j % NVB) * V_U4;
        // wave priority steps down through the tile (3, 2 after a quarter of
        // the score products, 1 at the output products, 0 after two thirds
        // of them): the SIMD's issue arbitration otherwise favours the older
        // of its two waves, which then finishes each tile far ahead and
        // leaves the younger one to run alone; this way the wave behind in
        // the tile wins and both stay busy
        __builtin_amdgcn_s_setprio(3);
        read_k(LK, 0);
        read_k(LK, 1);
#pragma unroll
        for (int p = 0; p < 4; ++p) exp_pair(sa, p);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 2 < 16) read_k(LK, i + 2);
            if (i == 14) read_v(LV, 0);
            if (i == 15) read_v(LV, 1);
            if (i == 2) issue_k(j + 3, i0);
            if (i == 6) issue_k(j + 3, i0 + 1);
            if (i == 10) issue_v(j + 2, i0);
            if (i == 13) issue_v(j + 2, i0 + 1);
            if (i == 4) __builtin_amdgcn_s_setprio(2);
            qk_m(sb, i, 0);
            qk_m(sb, i, 1);
            if (i < 12) exp_pair(sa, i + 4);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i == 0) __builtin_amdgcn_s_setprio(1);
            read_v(LV, i + 2);
            pv_m(i, 0);
            pv_m(i, 1);
            scale4(sa, sb, i);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (decltype(last_tag)::value) mask(sa, j + 1);
        lm = -INFINITY;
#pragma unroll
        for (int i = 8; i < 18; ++i) {
            if (i + 2 < 18) read_v(LV, i + 2);
            if (i == 12) __builtin_amdgcn_s_setprio(0);
            pv_m(i, 0);
            pv_m(i, 1);
            if (i < 16) lane_max_piece(sa, i - 8);
            __builtin_amdgcn_sched_barrier(0);
        }
        settle_lazy(sa);
        // the loads of tile j-1 (K(j+2), V(j+1)) have landed; this tile's
        // may still be in flight
        att_wait_vm4();
        att_lgkm_done();
        att_barrier();
    };
    // the last tile: its exponentials and products (V(last) landed at the
    // barrier that ended the tile before; its padding keys are zeroed first)
    auto final_step = [&]() {
        const u32x4 *LV = Vb + (last % NVB) * V_U4;
        att_wait_vm0();   // no load into LDS may be in flight when the block ends
        if (last > 0 && valid_last < KT) {
            zero_tail();
            att_lgkm_done();
            att_barrier();
        }
        read_v(LV, 0);
        read_v(LV, 1);
#pragma unroll
        for (int p = 0; p < 16; ++p) exp_pair(sa, p);
#pragma unroll
        for (int i = 0; i < 18; ++i) {
            if (i + 2 < 18) read_v(LV, i + 2);
            pv_m(i, 0);
            pv_m(i, 1);
        }
    };

    // prologue: K(0..2) and V(0..1), then the scores of tile 0
    for (int t = 0; t < min(3, ntiles); ++t) {
        issue_k(t, i0);
        issue_k(t, i0 + 1);
    }
    for (int t = 0; t < min(2, ntiles); ++t) {
        issue_v(t, i0);
        issue_v(t, i0 + 1);
    }
    att_wait_vm0();
    att_barrier();
    if (last == 0 && valid_last < KT) {
        zero_tail();
        att_lgkm_done();
        att_barrier();
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        read_k(Kb, i);
        qk_m(sb, i, 0);
        qk_m(sb, i, 1);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) scale4(sa, sb, k);
    if (last == 0) mask(sa, 0);
#pragma unroll
    for (int k = 0; k < 10; ++k) max_piece(sa, k);
    settle(sa);
    // K(0) is read: its buffer takes K(3) in tile 0
    att_lgkm_done();
    att_barrier();

    for (int j = 0; j + 1 < last; ++j) step(std::false_type{}, j);
    if (last > 0) step(std::true_type{}, last - 1);
    final_step();

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
