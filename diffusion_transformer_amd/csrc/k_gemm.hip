// bf16 MFMA products of the DiT block with fused epilogues, for gfx950.
//
//   C[M, N] = A[M, K] * W[N, K]^T      A bf16 row-major; W bf16 or int8+scales
//
// Epilogues ("gizai:dit" reference: linearInto, gatedInto, prepOf, gluRows;
// "944 -> 346 ms: optimizing FLUX.2 klein-4B on one TPU v6e chip" s.4.4 for
// the fused head norm + rotary):
//   EPI_F32       out[r][c] = C                              (plain fp32 store)
//   EPI_BF16      act[r][c] = bf16(C)                        (plain bf16 store)
//   EPI_GATE_RES  x[r][c] += gate[c] * C                     (gated residual, in place)
//   EPI_SWIGLU    act[r][j] = bf16(silu(C[r][2j]) * C[r][2j+1])   (UP rows interleaved)
//   EPI_QKV       per 128-wide head of Q and K: RMSNorm times the head-norm
//                 weight, then the adjacent-pair rotation with cos/sin[r];
//                 bf16 to q, k [H, M, 128]; V heads to vt [H, 128, ldv]
//
// Design (CDNA4): wave tile 64 x 128 (4 x 8 MFMA 16x16x32 bf16 sub-tiles),
// fp32 accumulators in registers, k-tiles of 64.  LDS rows are 128 bytes
// (64 bf16 of K) in 16-byte chunks placed at chunk ^ ((slot >> 1) & 7), which
// keeps both the 16-byte writes and the MFMA operand reads free of bank
// conflicts on the 64-bank LDS.  W rows are de-interleaved into LDS (even
// rows first, then odd rows), so each lane ends up holding output columns
// 2p and 2p+1 in two accumulators: the rotary pairs and the SwiGLU
// (gate, up) pairs meet in one lane without shuffles.  Blocks are remapped
// so that each XCD works on a compact group of tiles (its own L2), in groups
// of 6 row-tiles.  Two kernels:
//  - k_gemm_p3, 256x256 tiles: a two-group ping-pong schedule with direct
//    global -> LDS loads (below), for bf16 weights (int8 block-32 weights
//    arrive here dequantised by a pass of their own by default), with forms
//    for INT8 rows on the INT8 matrix cores and for int8 block-32 codes
//    converted in LDS;
//  - k_gemm, small or ragged shapes: 256x256 or 128x128 tiles, LDS double
//    buffer with register staging of the next k-tile; int8 block-32 weights
//    are dequantised (code * scale, rounded to bf16) on the way into LDS,
//    once per block.
#include "common.h"
#include <type_traits>

#include "kernels.h"

namespace dit {

namespace {

constexpr int BK = 64;
constexpr int WM = 64, WN = 128;
constexpr int TM = WM / 16, TN = WN / 16;

template <int BM, int BN>
struct Cfg {
    static constexpr int WAVES_M = BM / WM;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int NT = NW * 64;
    static constexpr int A_PER_T = BM * 8 / NT;   // 16-byte chunks per thread per k-tile
    static constexpr int B_PER_T = BN * 8 / NT;
    static constexpr int B8_PER_T = BN * 4 / NT;  // int8: 16 codes per chunk
    static constexpr int STAGE = (BM + BN) * 8;   // u32x4 per LDS buffer
    static_assert(A_PER_T >= 1 && B_PER_T >= 1 && B8_PER_T >= 1, "tile too small");
};

__device__ __forceinline__ int swz(int slot) { return (slot >> 1) & 7; }
__device__ __forceinline__ int lidx(int slot, int chunk) { return slot * 8 + (chunk ^ swz(slot)); }

// W row n of the tile -> LDS slot: even rows in the first half, odd rows in
// the second half.
template <int BN>
__device__ __forceinline__ int bslot(int n) { return (n & 1) * (BN / 2) + (n >> 1); }

// 16 int8 codes times one scale -> 16 bf16 (two 16-byte chunks).
__device__ __forceinline__ void dequant16(u32x4 q, float s, u32x4 &lo, u32x4 &hi) {
    float f[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t w = q[j];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            f[4 * j + b] = static_cast<float>(static_cast<int8_t>((w >> (8 * b)) & 0xff)) * s;
    }
    lo = u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
               pack_bf16x2(f[6], f[7])};
    hi = u32x4{pack_bf16x2(f[8], f[9]), pack_bf16x2(f[10], f[11]), pack_bf16x2(f[12], f[13]),
               pack_bf16x2(f[14], f[15])};
}

}  // namespace

// Four consecutive rows of two value features into V^T (d0: feature 2p,
// d1: feature 2p+1): col is the first row's column in vt, valid the number
// of those rows that exist.  Whole aligned groups leave as 8-byte stores,
// others one bf16 at a time (a stream's first or last rows).
__device__ __forceinline__ void store_v4(uint16_t *d0, uint16_t *d1, f32x4 e, f32x4 o, int col, int valid) {
    if (valid >= 4 && (col & 3) == 0) {
        *reinterpret_cast<u32x2 *>(d0) = u32x2{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
        *reinterpret_cast<u32x2 *>(d1) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (r < valid) {
                d0[r] = f32_to_bf16(e[r]);
                d1[r] = f32_to_bf16(o[r]);
            }
    }
}

// Epilogue shared by the products (wave tile TMW*16 rows x 128 columns).
// Lane holds rows m0 + wm*TMW*16 + tm*16 + 4*(lane>>4) + r and output pairs
// P = (n0 + wn*128)/2 + tp*16 + (lane & 15): column 2P in acc[tm][tp][r],
// column 2P+1 in acc[tm][tp+4][r].
template <int EPI, int TMW>
__device__ __forceinline__ void gemm_epilogue(f32x4 (&acc)[TMW][TN], int m0, int n0, int wm, int wn, int lane,
                                              int M, int N, const GemmEpi &ep) {
    const int col0 = n0 + wn * WN;
    if (col0 >= N) return;
    const int rbase = m0 + wm * TMW * 16 + 4 * (lane >> 4);
    const int pl = lane & 15;

    if constexpr (EPI == EPI_BF16) {
        const int ld = ep.ld_act ? ep.ld_act : N;
#pragma unroll
        for (int tm = 0; tm < TMW; ++tm) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rbase + tm * 16 + r;
                if (row >= M) continue;
#pragma unroll
                for (int tp = 0; tp < TN / 2; ++tp) {
                    const int c = col0 + 2 * (tp * 16 + pl);
                    if (c >= N) continue;
                    *reinterpret_cast<uint32_t *>(ep.act + static_cast<int64_t>(row) * ld + c) =
                        pack_bf16x2(acc[tm][tp][r], acc[tm][tp + TN / 2][r]);
                }
            }
        }
    } else if constexpr (EPI == EPI_F32 || EPI == EPI_GATE_RES) {
#pragma unroll
        for (int tm = 0; tm < TMW; ++tm) {
            __builtin_amdgcn_sched_barrier(0);   // bound the loads kept in flight
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rbase + tm * 16 + r;
                if (row >= M) continue;
#pragma unroll
                for (int tp = 0; tp < TN / 2; ++tp) {
                    const int c = col0 + 2 * (tp * 16 + pl);
                    if (c >= N) continue;
                    float2 *dst = reinterpret_cast<float2 *>(ep.out + static_cast<int64_t>(row) * ep.ldo + c);
                    float e = acc[tm][tp][r], o = acc[tm][tp + TN / 2][r];
                    if constexpr (EPI == EPI_F32) {
                        *dst = make_float2(e, o);
                    } else {
                        float2 g = *reinterpret_cast<const float2 *>(ep.gate + c);
                        float2 x = *dst;
                        x.x += g.x * e;
                        x.y += g.y * o;
                        *dst = x;
                    }
                }
            }
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
        const int half = ep.ld_act ? ep.ld_act : N / 2;
#pragma unroll
        for (int tm = 0; tm < TMW; ++tm) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = rbase + tm * 16 + r;
                if (row >= M) continue;
#pragma unroll
                for (int tp = 0; tp < TN / 2; ++tp) {
                    const int p = col0 / 2 + tp * 16 + pl;
                    if (2 * p >= N) continue;
                    float g = acc[tm][tp][r], u = acc[tm][tp + TN / 2][r];
                    ep.act[static_cast<int64_t>(row) * half + p] = f32_to_bf16(silu_f(g) * u);
                }
            }
        }
    } else if constexpr (EPI == EPI_QKV) {
        const int H = ep.heads;
        const int hb = col0 / 128;
        const int region = hb / H, head = hb % H;
        if (region < 2) {
            const float *nw = region == 0 ? ep.qn : ep.kn;
            uint16_t *dst = region == 0 ? ep.q : ep.k;
            float we[TN / 2], wo[TN / 2];
#pragma unroll
            for (int tp = 0; tp < TN / 2; ++tp) {
                const int p = tp * 16 + pl;
                we[tp] = nw[2 * p];
                wo[tp] = nw[2 * p + 1];
            }
#pragma unroll
            for (int tm = 0; tm < TMW; ++tm)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float ss = 0.f;
#pragma unroll
                    for (int tp = 0; tp < TN / 2; ++tp) {
                        float e = acc[tm][tp][r], o = acc[tm][tp + TN / 2][r];
                        ss += e * e + o * o;
                    }
                    // sum over the 16 lanes that share this row (lane bits 0..3)
                    ss = row16_sum(ss);
                    const float rstd = rsqrtf(ss * (1.0f / 128.0f) + ep.qk_eps);
                    const int row = rbase + tm * 16 + r;
                    const int rr = min(row, M - 1);
#pragma unroll
                    for (int tp = 0; tp < TN / 2; ++tp) {
                        const int p = tp * 16 + pl;
                        const float c = ep.cos[static_cast<int64_t>(rr) * 64 + p];
                        const float s = ep.sin[static_cast<int64_t>(rr) * 64 + p];
                        const float a = acc[tm][tp][r] * rstd * we[tp];
                        const float b = acc[tm][tp + TN / 2][r] * rstd * wo[tp];
                        if (row < M)
                            *reinterpret_cast<uint32_t *>(
                                dst + (static_cast<int64_t>(head) * (ep.rows_total ? ep.rows_total : M) +
                                       ep.row_base + row) * 128 + 2 * p) =
                                rotate_pack(a, b, c, s);
                    }
                }
        } else {
            // V: rows rbase + tm*16 + 0..3 are consecutive -> 4 bf16 along vt's row
#pragma unroll
            for (int tm = 0; tm < TMW; ++tm) {
                const int row0 = rbase + tm * 16;
                if (row0 >= M) continue;
#pragma unroll
                for (int tp = 0; tp < TN / 2; ++tp) {
                    const int p = tp * 16 + pl;
                    uint16_t *d0 = ep.vt + (static_cast<int64_t>(head) * 128 + 2 * p) * ep.ldv + ep.row_base + row0;
                    const f32x4 e = acc[tm][tp], o = acc[tm][tp + TN / 2];
                    store_v4(d0, d0 + ep.ldv, e, o, ep.row_base + row0, M - row0);
                }
            }
        }
    }
}

template <int BM, int BN, bool W8, int EPI>
__global__ void __launch_bounds__((BM / 64) * (BN / 128) * 64)
k_gemm(const uint16_t *__restrict__ A, const void *__restrict__ Wv,
       const uint16_t *__restrict__ Ws, int M, int N, int K, GemmEpi ep) {
    using C = Cfg<BM, BN>;
    __shared__ u32x4 lds[2 * C::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    // ---- tile mapping: XCD-compact, then grouped row-major
    const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
    const int total = ntm * ntn;
    int bid = blockIdx.x;
    {
        const int per = total / 8, rem = total % 8, xcd = bid % 8, loc = bid / 8;
        bid = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    }
    constexpr int GM = 6;
    const int group = bid / (GM * ntn), first = group * GM;
    const int gsz = min(ntm - first, GM);
    const int tile_m = first + (bid % (GM * ntn)) % gsz;
    const int tile_n = (bid % (GM * ntn)) / gsz;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    // ---- global load assignment
    const int a_c = tid & 7;
    const uint16_t *a_src[C::A_PER_T];
    int a_dst[C::A_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
        int r = (tid >> 3) + i * (C::NT / 8);
        int gr = min(m0 + r, M - 1);
        a_src[i] = A + static_cast<int64_t>(gr) * K + a_c * 8;
        a_dst[i] = lidx(r, a_c);
    }
    const uint8_t *b_src[W8 ? C::B8_PER_T : C::B_PER_T];
    const uint16_t *s_src[W8 ? C::B8_PER_T : 1];
    int b_dst[W8 ? C::B8_PER_T : C::B_PER_T];
    int b_dst2[W8 ? C::B8_PER_T : 1];
    if constexpr (!W8) {
        const uint16_t *W = static_cast<const uint16_t *>(Wv);
#pragma unroll
        for (int i = 0; i < C::B_PER_T; ++i) {
            int q = (tid >> 3) + i * (C::NT / 8);
            // rows 4a+{0,2,1,3}: the two rows a 16-lane group writes land in
            // different halves of the 64 banks
            int r = (q & ~3) | ((q & 1) << 1) | ((q >> 1) & 1);
            int gr = min(n0 + r, N - 1);
            b_src[i] = reinterpret_cast<const uint8_t *>(W + static_cast<int64_t>(gr) * K + a_c * 8);
            b_dst[i] = BM * 8 + lidx(bslot<BN>(r), a_c);
        }
    } else {
        const int8_t *W = static_cast<const int8_t *>(Wv);
        const int c4 = tid & 3;
#pragma unroll
        for (int i = 0; i < C::B8_PER_T; ++i) {
            int r = (tid >> 2) + i * (C::NT / 4);
            int gr = min(n0 + r, N - 1);
            b_src[i] = reinterpret_cast<const uint8_t *>(W + static_cast<int64_t>(gr) * K + c4 * 16);
            s_src[i] = Ws + static_cast<int64_t>(gr) * (K / 32) + (c4 >> 1);
            b_dst[i] = BM * 8 + lidx(bslot<BN>(r), 2 * c4);
            b_dst2[i] = BM * 8 + lidx(bslot<BN>(r), 2 * c4 + 1);
        }
    }

    u32x4 ra[C::A_PER_T];
    u32x4 rb[W8 ? C::B8_PER_T : C::B_PER_T];
    uint16_t rs[W8 ? C::B8_PER_T : 1];

    auto load_tile = [&](int kt) {
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i)
            ra[i] = *reinterpret_cast<const u32x4 *>(a_src[i] + kt * BK);
        if constexpr (!W8) {
#pragma unroll
            for (int i = 0; i < C::B_PER_T; ++i)
                rb[i] = *reinterpret_cast<const u32x4 *>(b_src[i] + kt * BK * 2);
        } else {
#pragma unroll
            for (int i = 0; i < C::B8_PER_T; ++i) {
                rb[i] = *reinterpret_cast<const u32x4 *>(b_src[i] + kt * BK);
                rs[i] = s_src[i][kt * 2];
            }
        }
    };
    auto store_tile = [&](int buf) {
        u32x4 *L = lds + buf * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i) L[a_dst[i]] = ra[i];
        if constexpr (!W8) {
#pragma unroll
            for (int i = 0; i < C::B_PER_T; ++i) L[b_dst[i]] = rb[i];
        } else {
#pragma unroll
            for (int i = 0; i < C::B8_PER_T; ++i) {
                u32x4 lo, hi;
                dequant16(rb[i], bf16_to_f32(rs[i]), lo, hi);
                L[b_dst[i]] = lo;
                L[b_dst2[i]] = hi;
            }
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // operand slots of this lane
    int a_slot[TM], b_slot[TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) a_slot[tm] = wm * WM + tm * 16 + (lane & 15);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
        b_slot[tn] = (tn < TN / 2 ? 0 : BN / 2) + wn * (WN / 2) + (tn % (TN / 2)) * 16 + (lane & 15);

    const int KT = K / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_tile(kt + 1);
        const u32x4 *L = lds + cur * C::STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int ch = ks * 4 + (lane >> 4);
            bf16x8 af[TM], bfr[TN];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
                af[tm] = __builtin_bit_cast(bf16x8, L[lidx(a_slot[tm], ch)]);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                bfr[tn] = __builtin_bit_cast(bf16x8, L[BM * 8 + lidx(b_slot[tn], ch)]);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], bfr[tn], acc[tm][tn], 0, 0, 0);
        }
        if (kt + 1 < KT) store_tile(cur ^ 1);
        __syncthreads();
    }

    gemm_epilogue<EPI, TM>(acc, m0, n0, wm, wn, lane, M, N, ep);
}

// ---------------------------------------------------------------------------
// Ping-pong product for bf16 weights: 256x256x64 tiles, 8 waves in two groups
// of four (one wave of each group per SIMD).  The two waves of every SIMD
// alternate between a compute phase (64 MFMAs on fragments already in
// registers) and a memory phase (LDS -> register fragments for their next
// compute phase, plus their share of the global -> LDS loads).  One
// workgroup barrier ends every phase, so at any time one wave per SIMD feeds
// the matrix core while the other works on memory:
//
//   phase 2t   : group 0 computes k-tile t      | group 1 reads fragments of t
//   phase 2t+1 : group 0 reads fragments of t+1 | group 1 computes k-tile t
// ---------------------------------------------------------------------------
namespace {
constexpr int PP_BM = 256, PP_BN = 256;
typedef __attribute__((address_space(3))) void lds_void_t;

// Barriers and waits as volatile asm with a memory clobber (no LDS or
// global access moves across them).
__device__ __forceinline__ void pp_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm8() { asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); }
__device__ __forceinline__ void wait_vm7() { asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); }
__device__ __forceinline__ void wait_vm4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
}  // namespace

// Epilogue of the 256x256 ping-pong product, staged through the (then idle)
// LDS so that global memory sees 16-byte accesses: a lane's accumulators
// hold 4 rows of one column pair, which would otherwise leave as 2-, 4- or
// 8-byte pieces.  Wave (wm, wn) holds rows wm*64 + tm*16 + 4*(lane>>4) + r
// and column pairs (2P, 2P+1), P = wn*64 + tp*16 + (lane&15), of the tile.
// All 512 threads take part; LDS must be free (no loads in flight).
//  - SWIGLU: bf16 [256][128] tile, 256-byte rows, 16-byte chunks swizzled
//    by chunk ^ (row & 15);
//  - F32 / GATE_RES / QKV (q, k): fp32 [128][256] half tiles, 1 KB rows,
//    16-byte chunks swizzled by chunk ^ (((row >> 2) & 1) << 3); rows
//    0-127 are written by waves wm = 0, 1, rows 128-255 by wm = 2, 3.
//  - QKV values (v): written straight from the accumulators (four
//    consecutive rows of one feature are 8 contiguous bytes of vt).
template <int EPI, bool PRE = true>
__device__ __forceinline__ void pp_epilogue(f32x4 (&acc)[TM][TN], u32x4 *lds, int m0, int n0, int wm, int wn,
                                            int lane, int tid, int M, int N, const GemmEpi &ep) {
    const int pl = lane & 15, g = lane >> 4;
    char *L = reinterpret_cast<char *>(lds);
    if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * 64 + tm * 16 + 4 * g + r;
#pragma unroll
                for (int tp = 0; tp < TN / 2; ++tp) {
                    const int col = wn * 64 + tp * 16 + pl;          // output column 0..127
                    const float gt = acc[tm][tp][r], up = acc[tm][tp + TN / 2][r];
                    const int off = row * 256 + (((col >> 3) ^ (row & 15)) << 4) + ((col & 7) << 1);
                    *reinterpret_cast<uint16_t *>(L + off) = f32_to_bf16(silu_f(gt) * up);
                }
            }
        wait_lgkm0();
        pp_barrier();
        const int half = ep.ld_act ? ep.ld_act : N / 2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = tid + 512 * i, row = q >> 4, c = q & 15;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(L + row * 256 + ((c ^ (row & 15)) << 4));
            if (m0 + row < M)
                *reinterpret_cast<u32x4 *>(ep.act + static_cast<int64_t>(m0 + row) * half + n0 / 2 + c * 8) = v;
        }
    } else {
        // QKV: the tile's two heads share a region (q, k or v) when the
        // region width heads*128 is a multiple of 256 (checked at launch)
        int region = 0;
        float rs[TM][4];
        if constexpr (EPI == EPI_QKV) {
            region = (n0 / 128) / ep.heads;
            if (region == 2) {
                const int head = (n0 / 128) % ep.heads + wn;
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    const int row0 = m0 + wm * 64 + tm * 16 + 4 * g;
                    if (row0 >= M) continue;
#pragma unroll
                    for (int tp = 0; tp < TN / 2; ++tp) {
                        const int p = tp * 16 + pl;
                        uint16_t *d0 = ep.vt + (static_cast<int64_t>(head) * 128 + 2 * p) * ep.ldv + ep.row_base + row0;
                        const f32x4 e = acc[tm][tp], o = acc[tm][tp + TN / 2];
                        store_v4(d0, d0 + ep.ldv, e, o, ep.row_base + row0, M - row0);
                    }
                }
                return;
            }
            // per-row 1/rms over the wave's 128 columns (one head): the 16
            // lanes with equal lane>>4 share a row
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float ss = 0.f;
#pragma unroll
                    for (int tp = 0; tp < TN / 2; ++tp) {
                        const float e = acc[tm][tp][r], o = acc[tm][tp + TN / 2][r];
                        ss += e * e + o * o;
                    }
                    ss = row16_sum(ss);
                    rs[tm][r] = rsqrtf(ss * (1.0f / 128.0f) + ep.qk_eps);
                }
        }
        float2 wq[TN / 2];
        if constexpr (EPI == EPI_QKV) {
            const float *nw = region == 0 ? ep.qn : ep.kn;
#pragma unroll
            for (int tp = 0; tp < TN / 2; ++tp) wq[tp] = *reinterpret_cast<const float2 *>(nw + 2 * (tp * 16 + pl));
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            if (hf) pp_barrier();                    // half 0 has been read
            // QKV: this thread's rows' cos and sin (read back below), fetched
            // before the staging so that their latency passes meanwhile
            // (PRE; otherwise where they are used: fewer live registers)
            f32x4 csr[4], snr[4];
            auto fetch_cs = [&](int i) {
                const int64_t gr = min(m0 + hf * 128 + (tid >> 4) + 32 * i, M - 1);
                csr[i] = *reinterpret_cast<const f32x4 *>(ep.cos + gr * 64 + 4 * (tid & 15));
                snr[i] = *reinterpret_cast<const f32x4 *>(ep.sin + gr * 64 + 4 * (tid & 15));
            };
            if constexpr (EPI == EPI_QKV && PRE) {
#pragma unroll
                for (int i = 0; i < 4; ++i) fetch_cs(i);
            }
            if ((wm >> 1) == hf) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = (wm & 1) * 64 + tm * 16 + 4 * g + r;   // 0..127 in the half
#pragma unroll
                        for (int tp = 0; tp < TN / 2; ++tp) {
                            const int col = wn * 128 + 2 * (tp * 16 + pl);     // even column 0..254
                            float e = acc[tm][tp][r], o = acc[tm][tp + TN / 2][r];
                            if constexpr (EPI == EPI_QKV) {
                                e = e * rs[tm][r] * wq[tp].x;
                                o = o * rs[tm][r] * wq[tp].y;
                            }
                            const int off = row * 1024 + ((((col >> 2) ^ (((row >> 2) & 1) << 3))) << 4) + ((col & 3) << 2);
                            *reinterpret_cast<float2 *>(L + off) = make_float2(e, o);
                        }
                    }
            }
            wait_lgkm0();
            pp_barrier();
            if constexpr (EPI == EPI_QKV) {
                // thread -> 8 consecutive columns (4 rotation pairs) of one row
                // in each of the tile's two heads: one cos and sin fetch serves both
                const int c16 = tid & 15, p0 = 4 * c16;
                const int head0 = (n0 / 128) % ep.heads;
                uint16_t *dst = region == 0 ? ep.q : ep.k;
                const int64_t hstride = static_cast<int64_t>(ep.rows_total ? ep.rows_total : M) * 128;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = (tid >> 4) + 32 * i, grow = m0 + hf * 128 + row;
                    if (grow >= M) continue;
                    const int sw = ((row >> 2) & 1) << 3;
                    if constexpr (!PRE) fetch_cs(i);
                    const f32x4 cs = csr[i], sn = snr[i];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int cg = c16 + 16 * h2;
                        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(L + row * 1024 + (((2 * cg) ^ sw) << 4));
                        const f32x4 v1 = *reinterpret_cast<const f32x4 *>(L + row * 1024 + (((2 * cg + 1) ^ sw) << 4));
                        const u32x4 o = {rotate_pack(v0[0], v0[1], cs[0], sn[0]), rotate_pack(v0[2], v0[3], cs[1], sn[1]),
                                         rotate_pack(v1[0], v1[1], cs[2], sn[2]), rotate_pack(v1[2], v1[3], cs[3], sn[3])};
                        *reinterpret_cast<u32x4 *>(dst + (head0 + h2) * hstride + (ep.row_base + grow) * 128 + 2 * p0) = o;
                    }
                }
            } else {
                // thread -> 4 consecutive columns, rows tid/64 + 8i: one gate chunk
                const int cc = tid & 63;
                f32x4 gt = {0.f, 0.f, 0.f, 0.f};
                if constexpr (EPI == EPI_GATE_RES) gt = *reinterpret_cast<const f32x4 *>(ep.gate + n0 + 4 * cc);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = (tid >> 6) + 8 * i, grow = m0 + hf * 128 + row;
                    if (grow >= M) continue;
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(
                        L + row * 1024 + ((cc ^ (((row >> 2) & 1) << 3)) << 4));
                    if constexpr (EPI == EPI_BF16) {
                        *reinterpret_cast<u32x2 *>(ep.act + static_cast<int64_t>(grow) * (ep.ld_act ? ep.ld_act : N) + n0 +
                                                   4 * cc) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                        continue;
                    }
                    f32x4 *dst = reinterpret_cast<f32x4 *>(ep.out + static_cast<int64_t>(grow) * ep.ldo + n0 + 4 * cc);
                    if constexpr (EPI == EPI_F32) {
                        *dst = v;
                    } else {
                        f32x4 x = *dst;
                        x[0] += gt[0] * v[0];
                        x[1] += gt[1] * v[1];
                        x[2] += gt[2] * v[2];
                        x[3] += gt[3] * v[3];
                        *dst = x;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// The loads.  A memory phase interleaves its global -> LDS loads with its
// fragment reads (three 16-byte fragment reads, one 1 KB load, eight times)
// instead of issuing them after the reads: the LDS read port and the load
// path then work at the same time.  For that the
// loads must go to buffers that nobody reads in that phase, which two 64 KB
// buffers cannot give.  The LDS (160 KB) holds three A buffers and two W
// buffers; A(t) is read by group 0 in phase 2t-1 and group 1 in phase 2t,
// W's two 128-row halves separately (group 0 reads output columns 0-127 in
// phase 2t-1, group 1 columns 128-255 in phase 2t):
//   phase 2t   (group 1 reads t):   group 1 loads W half 0 and A rows 0-127
//                                   of k-tile t+2;
//   phase 2t+1 (group 0 reads t+1): group 0 loads W half 1 of t+2 and A
//                                   rows 128-255 of t+3.
// Every load has at least two phases to land, and every memory phase ends
// with a wait for all but the loads issued in it.  Within a W half, even
// rows fill the first 64 slots and odd rows the next 64, so a lane's
// accumulators again hold output columns 2p and 2p+1.
// ---------------------------------------------------------------------------
namespace {
constexpr int P3_NA = 3, P3_NW = 2;
constexpr int P3_BUF = 256 * 8;   // u32x4 per buffer: 256 rows of 128 bytes
// Raw buffer descriptor over [base, base + 2 GiB): no range clamping is
// relied on, the loads stay inside the operands by construction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), 0x7fffffff, 0x00020000);
}
// 16 bytes per lane, buffer -> LDS (slot = the wave's base plus lane*16)
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, u32x4 *l) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)l, 16, voff, soff, 0, 0);
}
}  // namespace

// I8: the W8A8 form.  A and W are INT8 rows; a 128-byte LDS row then holds
// 128 codes of K instead of 64 bf16, a lane's 16-byte fragment feeds
// v_mfma_i32_16x16x64_i8 where it fed v_mfma_f32_16x16x32_bf16 (A and W
// fragments take K in the same order, so the dot products are those of the
// rows), and the int32 sums are scaled by ep.a_scale[row] * ep.w_scale[col]
// before the epilogue.  Everything else is the bf16 kernel's.
//
// B32: int8 weights with one bf16 scale per 32 inputs ("Host contract --
// RGBA-Image-2.1-Turbo" s.1, int8 weights dequantised inside the graph,
// products in bf16), dequantised into LDS.  W reaches the chip as int8 (half
// the bytes of bf16): each wave moves its share of a k-tile's codes and their
// scales into a staging area of its own (buffer loads into LDS, one memory
// phase ahead), and at the start of its next memory phase each lane turns
// exactly the 32 codes it loaded (one row, one block of 32) into bf16,
// code * scale rounded to nearest even, written into the one bf16 W buffer
// in the layout the fragment reads expect.  A group converts the W half the
// other group reads, in the phase just before that read:
//   phase 2t   : group 1 converts half 0 of k-tile t+1 (read by group 0 in 2t+1)
//   phase 2t+1 : group 0 converts half 1 of k-tile t+1 (read by group 1 in 2t+2)
// so a single bf16 W buffer suffices (the half being written was last read
// the phase before).  The product code * scale is exact: with the code's
// sign bit flipped, u = code + 128 in 0..255 converts exactly, and
// u * s - 128 * s is (code) * s, at most 15 significant bits.  LDS: three A
// buffers (96 KB), one W buffer (32 KB), codes (16 KB) and scales (2 KB).
template <int EPI, bool KS, bool I8 = false, bool B32 = false>
__global__ void __launch_bounds__(512, 1)
k_gemm_p3(const uint16_t *__restrict__ A, const uint16_t *__restrict__ W, int M, int N, int K,
          GemmEpi ep, const uint16_t *__restrict__ A2, const uint16_t *__restrict__ W2, int M2, GemmEpi ep2) {
    static_assert(!(KS && I8), "the k-split form is bf16 only");
    static_assert(!(B32 && (KS || I8)), "the block-32 form is a plain one-weight product");
    constexpr int BM = PP_BM, BN = PP_BN;
    constexpr uint32_t ESZ = I8 ? 1 : 2;          // bytes per element
    constexpr int BKE = 128 / ESZ;                // elements per 128-byte k-tile row
    using FragT = std::conditional_t<I8, i32x4, bf16x8>;
    using AccT = std::conditional_t<I8, i32x4, f32x4>;
    __shared__ u32x4 lds[(P3_NA + P3_NW) * P3_BUF];   // 160 KB
    u32x4 *const Abuf = lds;
    u32x4 *const Wbuf = lds + P3_NA * P3_BUF;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = wave >> 2, wg = wave & 3;     // group 0: waves 0-3, group 1: waves 4-7
    const int wm = wg, wn = grp;                  // wave tile (wm*64, wn*128)

    // Two products can share a launch (the double-stream block's streams:
    // same N and K, their own rows, weights and epilogue): tiles past the
    // first product's are the second's.
    const int ntn = (N + BN - 1) / BN;
    const int T0 = ((M + BM - 1) / BM) * ntn;
    const int total = T0 + ((M2 + BM - 1) / BM) * ntn;
    int bid = blockIdx.x;
    {
        const int per = total / 8, rem = total % 8, xcd = bid % 8, loc = bid / 8;
        bid = xcd < rem ? xcd * (per + 1) + loc : rem * (per + 1) + (xcd - rem) * per + loc;
    }
    if (bid >= T0) {
        bid -= T0;
        A = A2;
        W = W2;
        M = M2;
        ep = ep2;
    }
    const int ntm = (M + BM - 1) / BM;
    constexpr int GM = 6;
    const int group = bid / (GM * ntn), first = group * GM;
    const int gsz = min(ntm - first, GM);
    const int tile_m = first + (bid % (GM * ntn)) % gsz;
    const int tile_n = (bid % (GM * ntn)) / gsz;
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int T = K / BKE;

    // Loads: a wave's instruction i (0..3) within a 128-row half writes the
    // half's LDS slots 8(4wg + i) .. +7: lane -> slot 8(4wg + i) + (lane>>3),
    // chunk position lane&7, which holds global chunk
    // (lane&7) ^ (slot>>1 & 7) = (lane&7) ^ (lane>>4) ^ 4(i&1).
    // The operands are read without row clamping: A has whole 256-row tiles
    // allocated and N % 256 == 0.  Buffer loads keep the three address parts
    // apart: the tile base in the descriptor, the lane's row and chunk in a
    // 32-bit vector offset, the k-tile and the instruction's row step in a
    // scalar offset.
    const int lrow = lane >> 3;
    const int cE = (lane & 7) ^ (lane >> 4), cO = cE ^ 4;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(reinterpret_cast<const char *>(A) + static_cast<int64_t>(m0) * K * ESZ);
    // The weight rows of this tile.  Two-weight products: the SwiGLU columns
    // of EPI_QKV_SWIGLU read the second weight; with KS the k-tiles past
    // k_split read the second weight's rows (row length K - k_split).
    bool swi = false;
    const char *Wt = reinterpret_cast<const char *>(W) + static_cast<int64_t>(n0) * K * ESZ;
    if constexpr (EPI == EPI_QKV_SWIGLU) {
        swi = n0 >= ep.n_split;
        if (swi) Wt = reinterpret_cast<const char *>(ep.w2) + static_cast<int64_t>(n0 - ep.n_split) * K * ESZ;
    }
    const int K1 = KS ? ep.k_split : K, K2 = K - K1, T1 = K1 / BKE;
    if constexpr (KS) Wt = reinterpret_cast<const char *>(W + static_cast<int64_t>(n0) * K1);
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(Wt);
    const __amdgpu_buffer_rsrc_t rW2 =
        make_rsrc(KS ? reinterpret_cast<const char *>(ep.w2 + static_cast<int64_t>(n0) * K2) : Wt);
    const int ah = grp ^ 1;                        // the A and W halves this group loads
    // instruction i reads rows 8i (A) or 16i (W, de-interleaved) further
    // down than instruction 0
    const int wrow0 = 128 * ah + (wg < 2 ? 2 * (32 * wg + lrow) : 2 * (32 * wg - 64 + lrow) + 1);
    // byte offsets: a row is K * ESZ bytes, a 16-byte chunk c starts at 16c
    const uint32_t a_offE = ESZ * static_cast<uint32_t>((128 * ah + 32 * wg + lrow) * K) + 16u * cE;
    const uint32_t a_offO = ESZ * static_cast<uint32_t>((128 * ah + 32 * wg + lrow) * K) + 16u * cO;
    const uint32_t w_offE = ESZ * static_cast<uint32_t>(wrow0 * K1) + 16u * cE;
    const uint32_t w_offO = ESZ * static_cast<uint32_t>(wrow0 * K1) + 16u * cO;
    const uint32_t w2_offE = ESZ * static_cast<uint32_t>(wrow0 * K2) + 16u * cE;
    const uint32_t w2_offO = ESZ * static_cast<uint32_t>(wrow0 * K2) + 16u * cO;
    // load i (0..3) of the W half or the A half this group loads (half
    // grp ^ 1 of both), of k-tile kt.  Past the last k-tile the source is
    // clamped to it: those loads land in a buffer nobody reads any more, and
    // every memory phase issues the same number of loads.
    auto issue_w = [&](int kt, int i) {
        const int ks = min(kt, T - 1);
        u32x4 *dst = Wbuf + (kt & 1) * P3_BUF + (128 * ah + 8 * (4 * wg + i)) * 8;
        if (KS && ks >= T1)
            bdma16(rW2, (i & 1) ? w2_offO : w2_offE, 128u * (ks - T1) + ESZ * static_cast<uint32_t>(i * 16 * K2), dst);
        else
            bdma16(rW, (i & 1) ? w_offO : w_offE, 128u * ks + ESZ * static_cast<uint32_t>(i * 16 * K1), dst);
    };
    auto issue_a = [&](int kt, int i) {
        const int ks = min(kt, T - 1);
        bdma16(rA, (i & 1) ? a_offO : a_offE, 128u * ks + ESZ * static_cast<uint32_t>(i * 8 * K),
               Abuf + (kt % 3) * P3_BUF + (128 * ah + 8 * (4 * wg + i)) * 8);
    };

    // fragment slots: A wm*64 + tm*16 + (lane&15) in A(kt % 3); W
    // 128*wn + {0, 64} + tp*16 + (lane&15) in W(kt & 1)
    const int l16 = lane & 15;
    const int c0 = (lane >> 4) ^ ((l16 >> 1) & 7);
    const int offA0 = (wm * WM + l16) * 8 + c0, offA1 = offA0 ^ 4;
    const int offB0 = (128 * wn + l16) * 8 + c0, offB1 = offB0 ^ 4;

    FragT af[2][TM], bfr[2][TN];
    auto frag = [&](const u32x4 *La, const u32x4 *Lw, int f) {   // fragment read f of 24
        if (f < 2 * TM) {
            const int ks = f & 1, tm = f >> 1;
            af[ks][tm] = __builtin_bit_cast(FragT, La[(ks ? offA1 : offA0) + tm * 128]);
        } else {
            const int ks = (f - 2 * TM) & 1, tn = (f - 2 * TM) >> 1;
            const int o = ((tn < TN / 2 ? 0 : 64) + (tn % (TN / 2)) * 16) * 8;
            bfr[ks][tn] = __builtin_bit_cast(FragT, Lw[(ks ? offB1 : offB0) + o]);
        }
    };
    // fragments of k-tile kt only (prologue)
    auto load_frags = [&](int kt) {
        const u32x4 *La = Abuf + (kt % 3) * P3_BUF, *Lw = Wbuf + (B32 ? 0 : (kt & 1)) * P3_BUF;
#pragma unroll
        for (int f = 0; f < 24; ++f) frag(La, Lw, f);
    };
    // memory phase: fragments of k-tile kt, with W loads 0-3 of k-tile kw
    // and A loads 0-3 of k-tile ka in between
    auto memory = [&](int kt, int kw, int ka) {
        const u32x4 *La = Abuf + (kt % 3) * P3_BUF, *Lw = Wbuf + (B32 ? 0 : (kt & 1)) * P3_BUF;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
#pragma unroll
            for (int q = 0; q < 3; ++q) frag(La, Lw, 3 * r + q);
            __builtin_amdgcn_sched_barrier(0);
            if (r < 4) issue_w(kw, r);
            else issue_a(ka, r - 4);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- B32 staging.  Wave (grp, wg) stages rows rr = 32wg + j, j < 32, of
    // the W half ah = grp^1: load i (0, 1) moves rows j = 2m + i, m < 16, four
    // lanes to a row (lane l: m = l>>2, bytes 16(l&3) of the row's 64 codes
    // of the k-tile), so each 1 KB load reads 16 contiguous 64-byte row
    // pieces; one dword load brings every row's two block scales (lanes 2j,
    // 2j+1: row j).  Lane l later converts exactly the 32 codes it loaded:
    // 16 of row 2m (chunks 2(l&3), 2(l&3)+1, block (l&3)>>1) and the same 16
    // of row 2m + 1, into W slots 128ah + 64i + 16wg + m (even rows first,
    // then odd rows, as the fragment reads expect; 16 consecutive lanes of a
    // chunk write 4 consecutive 128-byte slots at 4 chunk positions each).
    u32x4 *const Wst = lds + 4 * P3_BUF + (grp * 4 + wg) * 128;                    // codes: 2 x 64 chunks
    uint32_t *const Sst = reinterpret_cast<uint32_t *>(lds + 4 * P3_BUF + 8 * 128) + (grp * 4 + wg) * 64;
    const int b_m = lane >> 2, b_q = lane & 3;
    __amdgpu_buffer_rsrc_t rW8 = rW, rS = rW;
    uint32_t w8_off = 0, s_off = 0;
    if constexpr (B32) {
        // descriptors end at the weight's (and scales') last row: nothing
        // past them is ever read
        const int64_t rem = static_cast<int64_t>(N - n0);
        const int64_t wb = rem * K, sb = rem * (K / 32) * 2;
        rW8 = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(reinterpret_cast<const char *>(W) + static_cast<int64_t>(n0) * K),
                                                static_cast<short>(0), static_cast<int>(wb < 0x7fffffff ? wb : 0x7fffffff),
                                                0x00020000);
        rS = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(ep.w_bscale + static_cast<int64_t>(n0) * (K / 32)),
                                               static_cast<short>(0), static_cast<int>(sb < 0x7fffffff ? sb : 0x7fffffff),
                                               0x00020000);
        w8_off = static_cast<uint32_t>((128 * ah + 32 * wg + 2 * b_m) * K + 16 * b_q);
        s_off = static_cast<uint32_t>((128 * ah + 32 * wg + (lane >> 1)) * (K / 32) * 2);
    }
    // codes and scales of k-tile kt (clamped past the last: those land in a
    // staging area nobody converts any more; every memory phase issues the
    // same three loads, codes first)
    auto issue_stage = [&](int kt) {
        const uint32_t ks = static_cast<uint32_t>(min(kt, T - 1));
        bdma16(rW8, w8_off, 64u * ks, Wst);
        bdma16(rW8, w8_off + static_cast<uint32_t>(K), 64u * ks, Wst + 64);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rS, (lds_void_t *)Sst, 4, s_off, 4u * ks, 0, 0);
    };
    // chunk h (0, 1) of this lane's 16 codes of row 2m + i: the two dwords
    // w0, w1 holding them, times the row's scale sd (block b_q >> 1) -> bf16
    u32x4 *const b_dst = Wbuf + (128 * ah + 16 * wg + b_m) * 8;
    auto convert_chunk = [&](uint32_t w0, uint32_t w1, uint32_t sd, int i, int h) {
        const float sc = (b_q >> 1) ? bf16hi_to_f32(sd) : bf16lo_to_f32(sd);
        const float msc = -128.0f * sc;
        w0 ^= 0x80808080u;
        w1 ^= 0x80808080u;
        auto dq = [&](uint32_t w, int b) {   // (byte b of w) - 128, times the scale: exact
            return __builtin_fmaf(static_cast<float>((w >> (8 * b)) & 0xffu), sc, msc);
        };
        const int slot = 128 * ah + 64 * i + 16 * wg + b_m;
        b_dst[64 * i * 8 + ((2 * b_q + h) ^ ((slot >> 1) & 7))] =
            u32x4{pack_bf16x2(dq(w0, 0), dq(w0, 1)), pack_bf16x2(dq(w0, 2), dq(w0, 3)),
                  pack_bf16x2(dq(w1, 0), dq(w1, 1)), pack_bf16x2(dq(w1, 2), dq(w1, 3))};
    };
    auto convert = [&]() {
        const u32x4 c0 = Wst[lane], c1 = Wst[64 + lane];
        const uint32_t s0 = Sst[4 * b_m], s1 = Sst[4 * b_m + 2];
        convert_chunk(c0[0], c0[1], s0, 0, 0);
        convert_chunk(c0[2], c0[3], s0, 0, 1);
        convert_chunk(c1[0], c1[1], s1, 1, 0);
        convert_chunk(c1[2], c1[3], s1, 1, 1);
    };
    // B32 memory phase: the staged codes of k-tile kc (loaded at the start of
    // this wave's previous memory phase, before its 4 A loads) are read
    // first and converted a chunk at a time between the fragment reads of
    // k-tile kt; once they are consumed the codes of k-tile kc + 1 are
    // staged, then the A loads of k-tile ka go out between the remaining
    // reads.  Nothing is converted past the last k-tile.
    auto memory_b32 = [&](int kt, int kc, int ka) {
        wait_vm4();
        const u32x4 *La = Abuf + (kt % 3) * P3_BUF, *Lw = Wbuf;
        const u32x4 c0 = Wst[lane], c1 = Wst[64 + lane];
        const uint32_t s0 = Sst[4 * b_m], s1 = Sst[4 * b_m + 2];
        const bool conv = kc < T;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
#pragma unroll
            for (int q = 0; q < 3; ++q) frag(La, Lw, 3 * r + q);
            __builtin_amdgcn_sched_barrier(0);
            if (r < 4) {
                if (conv) {
                    const u32x4 &c = r < 2 ? c0 : c1;
                    convert_chunk(c[2 * (r & 1)], c[2 * (r & 1) + 1], r < 2 ? s0 : s1, r >> 1, r & 1);
                }
                if (r == 3) issue_stage(kc + 1);   // after the last use of the staged codes
            } else {
                issue_a(ka, r - 4);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    AccT acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = AccT{0, 0, 0, 0};
    auto compute = [&]() {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    if constexpr (I8)
                        acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[ks][tm], bfr[ks][tn], acc[tm][tn], 0, 0, 0);
                    else
                        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][tm], bfr[ks][tn], acc[tm][tn], 0, 0, 0);
                }
    };

    // prologue: k-tiles 0 and 1 whole, and A rows 128-255 of k-tile 2 (group
    // 0's load of the phase before the first); all land before the first read.
    // B32: the codes of k-tile 0 are converted here (each group its half
    // grp^1) and those of k-tile 1 staged.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            issue_a(kt, i);
            if constexpr (!B32) issue_w(kt, i);
        }
    if (grp == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) issue_a(2, i);
    }
    if constexpr (B32) {
        issue_stage(0);
        wait_vm0();
        convert();
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkm0();
        issue_stage(1);
    }
    wait_vm0();
    pp_barrier();
    if (grp == 0) {
        load_frags(0);
        wait_lgkm0();
    }
    pp_barrier();

    // Main loop.  At the end of a memory phase the group's loads issued two
    // memory phases earlier have landed:
    //   end of 2t:   group 1 its W half 0 and A rows 0-127 of t+1 (phase
    //                2t-2), read by group 0 in 2t+1 (A rows 128-255 of t+1
    //                came from group 0 in 2t-3, waited for at the end of 2t-1);
    //   end of 2t+1: group 0 its W half 1 of t+1 (2t-1), read by group 1 in
    //                2t+2.
    for (int t = 0; t < T; ++t) {
        // phase 2t: group 0 computes k-tile t; group 1 reads its fragments
        // of t and loads W half 0 and A rows 0-127 of t+2
        if (grp == 0) {
            compute();
            __builtin_amdgcn_sched_barrier(0);
        } else {
            if constexpr (B32) {
                memory_b32(t, t + 1, t + 2);
                wait_lgkm0();
                wait_vm7();
            } else {
                memory(t, t + 2, t + 2);
                wait_lgkm0();
                wait_vm8();
            }
        }
        pp_barrier();
        // phase 2t+1: group 0 reads its fragments of t+1 and loads W half 1
        // of t+2 and A rows 128-255 of t+3; group 1 computes t
        if (grp == 0) {
            if (t + 1 < T) {
                if constexpr (B32) {
                    memory_b32(t + 1, t + 1, t + 3);
                    wait_lgkm0();
                    wait_vm7();
                } else {
                    memory(t + 1, t + 2, t + 3);
                    wait_lgkm0();
                    wait_vm8();
                }
            }
        } else {
            compute();
            __builtin_amdgcn_sched_barrier(0);
        }
        pp_barrier();
    }
    wait_vm0();   // no load into LDS may be in flight when the block ends
    pp_barrier();

    if constexpr (I8) {
        // acc[tm][tn][r] is the int32 sum of row m0 + wm*64 + tm*16 +
        // 4*(lane>>4) + r and column 2P (tn < TN/2) or 2P + 1 (tn >= TN/2),
        // P = (n0 + wn*128)/2 + (tn % (TN/2))*16 + (lane & 15)
        f32x4 accf[TM][TN];
        float sw[TN];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
            sw[tn] = ep.w_scale[n0 + 128 * wn + 2 * ((tn % (TN / 2)) * 16 + l16) + (tn >= TN / 2 ? 1 : 0)];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm * WM + tm * 16 + 4 * (lane >> 4) + r;
                const float sa = row < M ? ep.a_scale[row] : 0.f;
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) accf[tm][tn][r] = static_cast<float>(acc[tm][tn][r]) * sa * sw[tn];
            }
        }
        pp_epilogue<EPI>(accf, lds, m0, n0, wm, wn, lane, tid, M, N, ep);
    } else if constexpr (EPI == EPI_QKV_SWIGLU) {
        if (swi) pp_epilogue<EPI_SWIGLU>(acc, lds, m0, n0 - ep.n_split, wm, wn, lane, tid, M, N - ep.n_split, ep);
        else pp_epilogue<EPI_QKV, !B32>(acc, lds, m0, n0, wm, wn, lane, tid, M, ep.n_split, ep);
    } else {
        pp_epilogue<EPI, !B32>(acc, lds, m0, n0, wm, wn, lane, tid, M, N, ep);
    }
}

template <int BM, int BN, bool W8>
static hipError_t launch_cfg(const uint16_t *A, const void *W, const uint16_t *Ws, int M, int N, int K,
                             const GemmEpi &ep, hipStream_t st) {
    using C = Cfg<BM, BN>;
    const int grid = static_cast<int>(cdiv(M, BM) * cdiv(N, BN));
    switch (ep.kind) {
        case EPI_F32:
            k_gemm<BM, BN, W8, EPI_F32><<<grid, C::NT, 0, st>>>(A, W, Ws, M, N, K, ep);
            break;
        case EPI_BF16:
            k_gemm<BM, BN, W8, EPI_BF16><<<grid, C::NT, 0, st>>>(A, W, Ws, M, N, K, ep);
            break;
        case EPI_GATE_RES:
            k_gemm<BM, BN, W8, EPI_GATE_RES><<<grid, C::NT, 0, st>>>(A, W, Ws, M, N, K, ep);
            break;
        case EPI_SWIGLU:
            k_gemm<BM, BN, W8, EPI_SWIGLU><<<grid, C::NT, 0, st>>>(A, W, Ws, M, N, K, ep);
            break;
        case EPI_QKV:
            k_gemm<BM, BN, W8, EPI_QKV><<<grid, C::NT, 0, st>>>(A, W, Ws, M, N, K, ep);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int EPI, bool KS = false, bool I8 = false, bool B32 = false>
static hipError_t launch_pp(const uint16_t *A, const uint16_t *W, int M, int N, int K, const GemmEpi &ep,
                            hipStream_t st) {
    const int grid = static_cast<int>(cdiv(M, PP_BM) * cdiv(N, PP_BN));
    k_gemm_p3<EPI, KS, I8, B32><<<grid, 512, 0, st>>>(A, W, M, N, K, ep, nullptr, nullptr, 0, ep);
    return hipGetLastError();
}

// Two products of one epilogue kind, same N and K, in one ping-pong launch.
template <int EPI, bool B32 = false>
static hipError_t launch_pp2(const uint16_t *A, const uint16_t *W, int M, const GemmEpi &ep, const uint16_t *A2,
                             const uint16_t *W2, int M2, const GemmEpi &ep2, int N, int K, hipStream_t st) {
    const int grid = static_cast<int>((cdiv(M, PP_BM) + cdiv(M2, PP_BM)) * cdiv(N, PP_BN));
    k_gemm_p3<EPI, false, false, B32><<<grid, 512, 0, st>>>(A, W, M, N, K, ep, A2, W2, M2, ep2);
    return hipGetLastError();
}

// Whether the ping-pong kernel's staged epilogue can serve ep: it moves
// 16-byte pieces and keeps the two heads of a QKV tile in one region.
static bool pp_epilogue_ok(const GemmEpi &ep, int N) {
    auto al16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool qkv_ok = ep.heads % 2 == 0 && al16(ep.q) && al16(ep.k) && al16(ep.cos) && al16(ep.sin);
    const bool act_ok = al16(ep.act) && ep.ld_act % 8 == 0;
    bool epi_ok = false;
    switch (ep.kind) {
        case EPI_F32: epi_ok = al16(ep.out) && ep.ldo % 4 == 0; break;
        case EPI_BF16: epi_ok = al16(ep.act) && ep.ld_act % 8 == 0; break;
        case EPI_GATE_RES: epi_ok = al16(ep.out) && ep.ldo % 4 == 0 && al16(ep.gate); break;
        case EPI_SWIGLU: epi_ok = act_ok; break;
        case EPI_QKV: epi_ok = qkv_ok; break;
        case EPI_QKV_SWIGLU:
            epi_ok = qkv_ok && act_ok && ep.w2 && ep.n_split > 0 && ep.n_split % 256 == 0 && ep.n_split < N;
            break;
        default: break;
    }
    return epi_ok;
}

bool gemm_pingpong_ok(int M, int N, int K, bool w8, const GemmEpi &ep, bool a_rows_padded) {
    // Large problems: 256x256 tiles (8 waves; ping-pong for bf16 weights when
    // A's allocation covers whole 256-row tiles and N is a multiple of 256).
    const int64_t big_tiles = cdiv(M, 256) * cdiv(N, 256);
    bool epi_ok = pp_epilogue_ok(ep, N);
    if (ep.k_split > 0)
        epi_ok = epi_ok && ep.kind == EPI_GATE_RES && ep.w2 && ep.k_split % BK == 0 && ep.k_split >= 128 &&
                 K - ep.k_split >= 128;
    // int8 block-32 weights: the plain one-weight products
    if (w8) epi_ok = epi_ok && ep.kind != EPI_QKV_SWIGLU && ep.k_split == 0;
    return big_tiles >= 128 && epi_ok && K >= 128 && N % 256 == 0 && (a_rows_padded || M % 256 == 0);
}

hipError_t launch_gemm2(const uint16_t *A, const void *W, const uint16_t *Ws, int M, const GemmEpi &ep,
                        const uint16_t *A2, const void *W2, const uint16_t *Ws2, int M2, const GemmEpi &ep2,
                        bool w8, int N, int K, hipStream_t st) {
    const bool one = M > 0 && M2 > 0 && ep.kind == ep2.kind && ep.kind != EPI_QKV_SWIGLU && ep.k_split == 0 &&
                     ep2.k_split == 0 && gemm_pingpong_ok(M + M2, N, K, w8, ep, true) &&
                     gemm_pingpong_ok(M + M2, N, K, w8, ep2, true);
    if (!one) {
        hipError_t e = hipSuccess;
        if (M > 0) e = launch_gemm(A, W, Ws, w8, M, N, K, ep, st, true);
        if (e == hipSuccess && M2 > 0) e = launch_gemm(A2, W2, Ws2, w8, M2, N, K, ep2, st, true);
        return e;
    }
    const uint16_t *Wb = static_cast<const uint16_t *>(W), *Wb2 = static_cast<const uint16_t *>(W2);
    if (w8) {
        GemmEpi e1 = ep, e2 = ep2;
        e1.w_bscale = Ws;
        e2.w_bscale = Ws2;
        switch (ep.kind) {
            case EPI_F32: return launch_pp2<EPI_F32, true>(A, Wb, M, e1, A2, Wb2, M2, e2, N, K, st);
            case EPI_GATE_RES: return launch_pp2<EPI_GATE_RES, true>(A, Wb, M, e1, A2, Wb2, M2, e2, N, K, st);
            case EPI_SWIGLU: return launch_pp2<EPI_SWIGLU, true>(A, Wb, M, e1, A2, Wb2, M2, e2, N, K, st);
            case EPI_QKV: return launch_pp2<EPI_QKV, true>(A, Wb, M, e1, A2, Wb2, M2, e2, N, K, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (ep.kind) {
        case EPI_F32: return launch_pp2<EPI_F32>(A, Wb, M, ep, A2, Wb2, M2, ep2, N, K, st);
        case EPI_GATE_RES: return launch_pp2<EPI_GATE_RES>(A, Wb, M, ep, A2, Wb2, M2, ep2, N, K, st);
        case EPI_SWIGLU: return launch_pp2<EPI_SWIGLU>(A, Wb, M, ep, A2, Wb2, M2, ep2, N, K, st);
        case EPI_QKV: return launch_pp2<EPI_QKV>(A, Wb, M, ep, A2, Wb2, M2, ep2, N, K, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_w8a8(const int8_t *A, const float *a_scale, const int8_t *W, const float *w_scale, int M,
                            int N, int K, const GemmEpi &ep_in, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    if (N % PP_BN || K % 128 || K < 128 || !a_scale || !w_scale) return hipErrorInvalidValue;
    if (ep_in.k_split > 0 || !pp_epilogue_ok(ep_in, N)) return hipErrorInvalidValue;
    GemmEpi ep = ep_in;
    ep.a_scale = a_scale;
    ep.w_scale = w_scale;
    const auto *a = reinterpret_cast<const uint16_t *>(A);
    const auto *w = reinterpret_cast<const uint16_t *>(W);
    switch (ep.kind) {
        case EPI_F32: return launch_pp<EPI_F32, false, true>(a, w, M, N, K, ep, st);
        case EPI_BF16: return launch_pp<EPI_BF16, false, true>(a, w, M, N, K, ep, st);
        case EPI_GATE_RES: return launch_pp<EPI_GATE_RES, false, true>(a, w, M, N, K, ep, st);
        case EPI_SWIGLU: return launch_pp<EPI_SWIGLU, false, true>(a, w, M, N, K, ep, st);
        case EPI_QKV: return launch_pp<EPI_QKV, false, true>(a, w, M, N, K, ep, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm(const uint16_t *A, const void *W, const uint16_t *Ws, bool w8, int M, int N,
                       int K, const GemmEpi &ep, hipStream_t st, bool a_rows_padded) {
    if (M <= 0) return hipSuccess;
    if (gemm_pingpong_ok(M, N, K, w8, ep, a_rows_padded)) {
        const uint16_t *Wb = static_cast<const uint16_t *>(W);
        if (w8) {
            GemmEpi e = ep;
            e.w_bscale = Ws;
            switch (ep.kind) {
                case EPI_F32: return launch_pp<EPI_F32, false, false, true>(A, Wb, M, N, K, e, st);
                case EPI_BF16: return launch_pp<EPI_BF16, false, false, true>(A, Wb, M, N, K, e, st);
                case EPI_GATE_RES: return launch_pp<EPI_GATE_RES, false, false, true>(A, Wb, M, N, K, e, st);
                case EPI_SWIGLU: return launch_pp<EPI_SWIGLU, false, false, true>(A, Wb, M, N, K, e, st);
                case EPI_QKV: return launch_pp<EPI_QKV, false, false, true>(A, Wb, M, N, K, e, st);
                default: return hipErrorInvalidValue;
            }
        }
        if (ep.k_split > 0) return launch_pp<EPI_GATE_RES, true>(A, Wb, M, N, K, ep, st);
        switch (ep.kind) {
            case EPI_F32: return launch_pp<EPI_F32>(A, Wb, M, N, K, ep, st);
            case EPI_BF16: return launch_pp<EPI_BF16>(A, Wb, M, N, K, ep, st);
            case EPI_GATE_RES: return launch_pp<EPI_GATE_RES>(A, Wb, M, N, K, ep, st);
            case EPI_SWIGLU: return launch_pp<EPI_SWIGLU>(A, Wb, M, N, K, ep, st);
            case EPI_QKV: return launch_pp<EPI_QKV>(A, Wb, M, N, K, ep, st);
            case EPI_QKV_SWIGLU: return launch_pp<EPI_QKV_SWIGLU>(A, Wb, M, N, K, ep, st);
            default: return hipErrorInvalidValue;
        }
    }
    // the two-weight forms exist only as the ping-pong kernel
    if (ep.kind == EPI_QKV_SWIGLU || ep.k_split > 0) return hipErrorInvalidValue;
    // otherwise 256x256 tiles with register staging, or for small problems
    // 128x128 (2 waves) so that the grid still spreads over the chip
    const int64_t big_tiles = cdiv(M, 256) * cdiv(N, 256);
    if (big_tiles >= 128) {
        return w8 ? launch_cfg<256, 256, true>(A, W, Ws, M, N, K, ep, st)
                  : launch_cfg<256, 256, false>(A, W, Ws, M, N, K, ep, st);
    }
    return w8 ? launch_cfg<128, 128, true>(A, W, Ws, M, N, K, ep, st)
              : launch_cfg<128, 128, false>(A, W, Ws, M, N, K, ep, st);
}

}  // namespace dit
