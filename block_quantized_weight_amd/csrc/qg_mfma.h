#pragma once
// qg_mfma.h -- co-batch product (several tokens, bf16 activations) on the
// gfx950 matrix cores, and the many-token product (qgemm) built on it.
//
// With M tokens the product reuses every decoded weight M times; past a few
// tokens the per-weight VALU work of the lane-per-block kernel (an unpack plus
// M dot products, each reading its activations from LDS) becomes the bound.
// Here one v_mfma_f32_16x16x32_bf16 takes a 32-weight block of 16 rows:
//   A (16 x 32)  the tokens' activations of that block (A row = token, rows
//                past M repeat the last token), bf16 exactly as given;
//   B (32 x 16)  the 16 rows' codes, converted to bf16 in registers (exact:
//                Q4_0 as (q-8)/16, E2M1 values, int8 codes);
//   C            zero;
//   D[t][r]      the block's dot product for token t and row r before the
//                block scale, which is applied in fp32: acc += d * D (16 d
//                for Q4_0); rows t >= M are computed and never stored.
// The sum over k inside the instruction is order-free, so any assignment of
// the 32 k values to operand slots works as long as A and B agree: lane l of
// both holds 8 consecutive k (octet l/16 of the block), A for token l%16 and
// B for row l%16; D gives lane l row l%16 and tokens 4*(l/16) .. +3.
//
// B needs 8 consecutive k of one row per lane, while the packed layout gives
// each lane a whole block (16-byte record: row r, block s for lane r*L + s).
// Weights are loaded exactly as in the lane-per-block kernel (coalesced
// 16-byte records, nontemporal), then each step's records pass through a
// small wave-private LDS area from which every lane reads its octets: dword g
// (4-bit codes) or dwords 2g, 2g+1 (Q8_0) of record r*L + s.  One record of
// padding after every eight keeps those reads at most two-way bank-conflicted.
//
// A "unit" is 16 rows x the whole K: one tile of 16 rows (L = 4), two
// half-tiles (L = 8, R = 8), four quarter-tiles (L = 16, R = 4), or 2 / 4
// row groups of a taller tile (L = 2, 1).  KS waves of a workgroup split a
// unit's steps; their partial sums are added in a fixed order through LDS,
// so results are deterministic.
//
// More than 16 tokens: each group of 16 is one A operand; a workgroup pass
// (grid row blockIdx.y) takes one group, or two that share each unpacked
// weight operand where a wave holds several 16-row groups; every pass reads
// the unit's weights again, and those repeats can be served by the device
// caches.
#include "qg_common.h"

namespace qg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int MFMA_MAX_L = 8;     // lanes per row served for co-batches of up to 8 tokens
constexpr int GEMM_MAX_L = 16;    // lanes per row served for token groups (qgemm)

struct MGeom {
    const uint8_t *w;
    int32_t n, k, nb, L, R, S, tiles;
    int64_t ctb, stb, soff;
    int32_t m;                       // tokens of the call; each blockIdx.y runs a group of up to 16
    int32_t units, KS, ksh, upi, ngroups;
    int32_t SW, nwin, wblk;
};

// Compile-time shape of a unit for lanes-per-row LL.
template <int LL> struct MShape {
    static constexpr int R = 64 / LL;
    static constexpr int TPW = LL >= 8 ? LL / 4 : 1;       // tiles per unit
    static constexpr int RG = LL >= 4 ? 1 : 4 / LL;        // 16-row groups per unit
    static constexpr int NM = LL >= 4 ? LL : 4;            // MFMAs per step
    static constexpr int NS = LL;                           // blocks per step
};

// Per-wave transpose area: one plane of 72 record slots per (tile, part),
// planes 1168 bytes apart (16 bytes of skew per plane), then the step's
// scales as fp32 [tile][lane].
constexpr int MPLANE = 1168;
inline __host__ __device__ int mfma_wave_bytes(int fmt, int LL)
{
    const int tpw = LL >= 8 ? LL / 4 : 1, P = fmt == QG_Q8_0 ? 2 : 1;
    return tpw * P * MPLANE + tpw * 64 * 4;
}

// Token groups of 16 per workgroup pass in the many-token product: two where
// a wave holds several 16-row groups (L <= 2) and there are more than 16
// tokens, so every unpacked weight operand serves two A operands; one
// elsewhere.  Measured on MI355X (Q4_0,
// 64 / 128 tokens): 24576x4096 at 2 lanes per row 72.4 / 119.2 us with one
// group, 60.1 / 98.7 with two; at 8 lanes per row two groups were slower
// (4096x12288: 73.7 -> 93.2 us at 128 tokens), four slower everywhere.
inline __host__ __device__ int gemm_groups(int LL, int64_t m) { return LL <= 2 && m > 16 ? 2 : 1; }

// Split-K partials (present only when KS > 1).
inline __host__ __device__ size_t mfma_red_bytes(int LL, int TG = 1, int nw = WAVES)
{
    const int RG = LL >= 4 ? 1 : 4 / LL;
    return (size_t)nw * TG * RG * 4 * 64 * 4;
}

inline __host__ __device__ size_t mfma_lds_bytes(int fmt, int m, int wblk, int LL, int KS, int TG = 1, int nw = WAVES)
{
    size_t b = (size_t)wblk * m * 64;                        // activations: [block][token][octet]
    if (KS > 1) b += mfma_red_bytes(LL, TG, nw);             // split-K partials
    b += (size_t)nw * mfma_wave_bytes(fmt, LL);              // transpose areas
    return b;
}

// Waves per workgroup of the co-batch kernel on 8 lanes per row where its
// units would otherwise run one wave per SIMD: eight, splitting each unit's
// steps (or two units) over twice the waves with the same activation staging
// (MI355X, Q4_0, 4 / 8 tokens: 6144x4096 9.69 -> 9.30 / 10.63 -> 9.77 us,
// 4096x12288 14.84 -> 13.79 / 19.15 -> 16.06; on 2 lanes per row, 24576x4096
// at 8 tokens, 19.6 -> 24.0, so not there).
constexpr int MFMA_WIDE_WAVES = 8;

template <int FMT, int LL, int TG = 1>
struct MEngine {
    using Sh = MShape<LL>;
    static constexpr int P = FMT == QG_Q8_0 ? 2 : 1;        // 16-byte parts per record
    static constexpr int TPW = Sh::TPW;
    static constexpr int NM = Sh::NM;
    // steps per load batch (16 lanes per row load 4 tiles per step: fewer steps)
    static constexpr int U = LL >= 16 ? (FMT == QG_Q8_0 ? 1 : 2) : (FMT == QG_Q8_0 ? 2 : 4);

    struct Regs {
        uint4 c[U][TPW][P];
        uint32_t s[U][TPW];
    };

    // Issues the loads of cnt (>= 1) steps jfirst, jfirst+KS, ... of the
    // unit's tiles: always U steps' worth (steps past cnt repeat the last
    // one), so the vmcnt waits stay exact.  tok[t] is false for a tile past
    // the end, which then reads the unit's first tile instead (never stored).
    static __device__ __forceinline__ void load(const MGeom &g, const uint8_t *cb, const uint8_t *sbase, int lane,
                                                int jfirst, int cnt, int KS, const int (&tofs)[TPW], Regs &r)
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = jfirst + min(u, cnt - 1) * KS;
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const uint8_t *cp = cb + (int64_t)tofs[tt] * g.ctb + (int64_t)j * (P * 1024) + lane * 16;
#pragma unroll
                for (int h = 0; h < P; ++h) r.c[u][tt][h] = ld_stream16(cp + h * 1024);
                const uint8_t *sp = sbase + (int64_t)tofs[tt] * g.stb;
                if (FMT == QG_MXFP4)
                    r.s[u][tt] = ld_stream_u8(sp + (int64_t)j * 64 + lane);
                else
                    r.s[u][tt] = ld_stream_u16((const uint16_t *)sp + (int64_t)j * 64 + lane);
            }
        }
    }

    static __device__ __forceinline__ int slot(int sl) { return (sl + (sl >> 3)) * 16; }

    // 8 codes (one octet) -> 8 bf16 values, element order.
    static __device__ __forceinline__ bf16x8_t unpack(const uint32_t *c)
    {
        uint32_t q[4];
        if (FMT == QG_Q4_0) {
            float v[8];
            q4_unpack8(c[0], v);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) q[kk] = __builtin_bit_cast(uint32_t, pk_bf16(v[2 * kk], v[2 * kk + 1]));
        } else if (FMT == QG_MXFP4) {
            q[0] = __builtin_bit_cast(uint32_t, fp4_pair_bf16<0>(c[0]));
            q[1] = __builtin_bit_cast(uint32_t, fp4_pair_bf16<1>(c[0]));
            q[2] = __builtin_bit_cast(uint32_t, fp4_pair_bf16<2>(c[0]));
            q[3] = __builtin_bit_cast(uint32_t, fp4_pair_bf16<3>(c[0]));
        } else {
            // int8 -> fp32 is exact and has at most 8 significant bits, so
            // its upper half is the exact bf16
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint32_t w = c[kk >> 1];
                const int b = 2 * (kk & 1);
                const uint32_t lo = __builtin_bit_cast(uint32_t, i8_at(w, b));
                const uint32_t hi = __builtin_bit_cast(uint32_t, i8_at(w, b + 1));
                q[kk] = (lo >> 16) | (hi & 0xFFFF0000u);
            }
        }
        return __builtin_bit_cast(bf16x8_t, make_uint4(q[0], q[1], q[2], q[3]));
    }

    static __device__ __forceinline__ float scale(uint32_t bits)
    {
        return FMT == QG_MXFP4 ? e8m0_to_f32(bits) : FMT == QG_Q4_0 ? q4_scale(bits) : f16_bits_to_f32(bits);
    }

    // What one block of the step reads from LDS: the rows' codes (one octet
    // per lane and 16-row group) and scales, and the token groups'
    // activations.
    struct Raw {
        uint32_t cw[Sh::RG][2];
        float sc[Sh::RG];
        bf16x8_t a[TG];
    };

    // Reads block s of the step (block index jL + s of every row of the unit)
    // from the transpose area and the staged activations.  A rows past mp
    // repeat the last token: a row of D depends only on its row of A, and
    // those rows are never stored.
    static __device__ __forceinline__ void fetch(int s, int j, int b0, const uint4 *xs, const uint8_t *wl,
                                                 const float *wsc, int mp, Raw &o)
    {
        const int lane = threadIdx.x & 63, i = lane & 15, oct = lane >> 4;
        const int bl = j * LL + s - b0;
#pragma unroll
        for (int G = 0; G < Sh::RG; ++G) {
            const int tt = LL >= 8 ? i / Sh::R : 0;
            const int rr = LL >= 8 ? i % Sh::R : 16 * G + i;
            const int sl = rr * LL + s;
            if (FMT == QG_Q8_0) {
                const uint2 v = *(const uint2 *)(wl + (tt * P + (oct >> 1)) * MPLANE + slot(sl) + 8 * (oct & 1));
                o.cw[G][0] = v.x;
                o.cw[G][1] = v.y;
            } else {
                o.cw[G][0] = *(const uint32_t *)(wl + tt * MPLANE + slot(sl) + 4 * oct);
                o.cw[G][1] = 0;
            }
            o.sc[G] = wsc[tt * 64 + sl];
        }
#pragma unroll
        for (int tg = 0; tg < TG; ++tg)
            o.a[tg] = __builtin_bit_cast(bf16x8_t, xs[(bl * mp + min(16 * tg + i, mp - 1)) * 4 + oct]);
    }

    static __device__ __forceinline__ void decode(const Raw &o, bf16x8_t (&bw)[Sh::RG])
    {
#pragma unroll
        for (int G = 0; G < Sh::RG; ++G) bw[G] = unpack(o.cw[G]);
    }

    // The MFMAs of one step for the mp (<= 16) tokens of the group, every
    // token group unconditionally.  wl: this wave's transpose area.  While
    // the matrix cores work on block s, block s + 1 is unpacked and the LDS
    // reads of block s + 2 are issued; block s's scale is applied after.
    static __device__ __forceinline__ void step(const MGeom &g, const Regs &r, int u, int j, int b0, const uint4 *xs,
                                                uint8_t *wl, f32x4_t (&acc)[TG][Sh::RG], int mp)
    {
        const int lane = threadIdx.x & 63;
        float *wsc = (float *)(wl + TPW * P * MPLANE);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
            for (int h = 0; h < P; ++h) *(uint4 *)(wl + (tt * P + h) * MPLANE + slot(lane)) = r.c[u][tt][h];
            wsc[tt * 64 + lane] = scale(r.s[u][tt]);
        }
        constexpr int NS = Sh::NS;
        Raw rw[NS];
        bf16x8_t bw[NS][Sh::RG];
        fetch(0, j, b0, xs, wl, wsc, mp, rw[0]);
        if (NS > 1) fetch(1, j, b0, xs, wl, wsc, mp, rw[NS > 1 ? 1 : 0]);
        decode(rw[0], bw[0]);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4_t d[TG][Sh::RG];
#pragma unroll
            for (int tg = 0; tg < TG; ++tg)
#pragma unroll
                for (int G = 0; G < Sh::RG; ++G)
                    d[tg][G] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rw[s].a[tg], bw[s][G], c, 0, 0, 0);
            if (s + 2 < NS) fetch(s + 2, j, b0, xs, wl, wsc, mp, rw[s + 2 < NS ? s + 2 : 0]);
            if (s + 1 < NS) decode(rw[s + 1 < NS ? s + 1 : 0], bw[s + 1 < NS ? s + 1 : 0]);
#pragma unroll
            for (int tg = 0; tg < TG; ++tg)
#pragma unroll
                for (int G = 0; G < Sh::RG; ++G)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[tg][G][q] = __builtin_fmaf(rw[s].sc[G], d[tg][G][q], acc[tg][G][q]);
        }
    }

    static __device__ __forceinline__ void compute(const MGeom &g, const Regs &r, int cnt, int jfirst, int KS, int b0,
                                                   const uint4 *xs, uint8_t *wl, f32x4_t (&acc)[TG][Sh::RG], int mp)
    {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (u < cnt) step(g, r, u, jfirst + u * KS, b0, xs, wl, acc, mp);
    }
};

// Stages window w of the mp tokens' activations (x already offset to the
// group's first token) as xs[(bl*mp + t)*4 + oct] (bf16 octets), i.e. 16-byte
// pieces p = (bl*mp + t)*4 + oct.  Thread p of each round of blockDim pieces
// loads piece p straight into LDS (global_load_lds_dwordx4: the wave's 64
// pieces land at the wave-uniform base + 16 * lane), so every round is in
// flight at once and no registers hold the data; pieces of blocks past the
// matrix are written as zeros.  Returns once this wave's pieces are in LDS
// (the caller's barrier then covers the workgroup).
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void mfma_stage(const MGeom &g, const uint16_t *x, int w, uint4 *xs, int mp)
{
    const int b0 = w * g.SW * g.L;
    const int pieces = g.wblk * mp * 4;
    const int T = (int)blockDim.x;
    const int wbase = (int)threadIdx.x & ~63;
    for (int base = 0; base < pieces; base += T) {
        const int p = base + (int)threadIdx.x;
        if (p < pieces) {
            const int idx = p >> 2, bl = idx / mp, t = idx - bl * mp, b = b0 + bl;
            if (b < g.nb)
                __builtin_amdgcn_global_load_lds((const void *)(x + (int64_t)t * g.k + (int64_t)b * QK + (p & 3) * 8),
                                                 (lds_void *)(xs + base + wbase), 16, 0, 0);
            else
                xs[p] = make_uint4(0, 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): this wave's LDS loads have landed
}

// blockIdx.y: a pass over TG token groups of 16 (tokens 16*TG*y .. of the
// call); the co-batch calls have one pass of one group.  LDS is planned for
// min(m, 16*TG) tokens.
template <int FMT, int LL, int TG, int NW = WAVES>
__global__ __launch_bounds__(64 * NW) void k_dense_mfma(MGeom g, const void *__restrict__ xv, float *__restrict__ yv)
{
    using E = MEngine<FMT, LL, TG>;
    using Sh = MShape<LL>;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tb = (int)blockIdx.y * 16 * TG;
    const int mp = min(16 * TG, g.m - tb);
    const int mplan = min(16 * TG, g.m);
    uint4 *xs = (uint4 *)smem;
    float *red = (float *)(smem + (size_t)g.wblk * mplan * 64);
    const uint16_t *x = (const uint16_t *)xv + (int64_t)tb * g.k;
    float *y = yv + (int64_t)tb * g.n;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint8_t *wl = (uint8_t *)red + (g.KS > 1 ? mfma_red_bytes(LL, TG, NW) : 0) + wave * mfma_wave_bytes(FMT, LL);
    const int usub = wave >> g.ksh, kpart = wave & (g.KS - 1);
    const int KS = g.KS;
    bool staged = false;
    for (int grp = blockIdx.x; grp < g.ngroups; grp += gridDim.x) {
        const int unit = grp * g.upi + usub;
        const bool active = unit < g.units;
        const int uu = active ? unit : 0;
        const uint8_t *cb = g.w + (int64_t)uu * Sh::TPW * g.ctb;
        const uint8_t *sbase = g.w + g.soff + (int64_t)uu * Sh::TPW * g.stb;
        int tofs[Sh::TPW];
#pragma unroll
        for (int tt = 0; tt < Sh::TPW; ++tt) tofs[tt] = uu * Sh::TPW + tt < g.tiles ? tt : 0;
        f32x4_t acc[TG][Sh::RG];
#pragma unroll
        for (int tg = 0; tg < TG; ++tg)
#pragma unroll
            for (int G = 0; G < Sh::RG; ++G) acc[tg][G] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        for (int w = 0; w < g.nwin; ++w) {
            const int j0 = w * g.SW;
            const int j1 = min(g.S, j0 + g.SW);
            const int jf = j0 + kpart;      // SW is a multiple of KS
            const int nsteps = (active && jf < j1) ? (j1 - jf + KS - 1) / KS : 0;
            const int jlast = nsteps > 0 ? jf + (nsteps - 1) * KS : 0;
            typename E::Regs ra, rb;
            E::load(g, cb, sbase, lane, nsteps > 0 ? jf : 0, max(1, min(nsteps, E::U)), KS, tofs, ra);
            if (g.nwin > 1 || !staged) {
                __syncthreads();
                mfma_stage(g, x, w, xs, mp);
                __syncthreads();
                staged = true;
            }
            const int b0 = j0 * g.L;
            int done = 0;
            while (done < nsteps) {
                const int cA = min(nsteps - done, E::U);
                const int rB = nsteps - done - cA;
                E::load(g, cb, sbase, lane, rB > 0 ? jf + (done + cA) * KS : jlast, rB > 0 ? min(rB, E::U) : 1, KS, tofs, rb);
                E::compute(g, ra, cA, jf + done * KS, KS, b0, xs, wl, acc, mp);
                done += cA;
                if (done >= nsteps) break;
                const int cB = min(nsteps - done, E::U);
                const int rA = nsteps - done - cB;
                E::load(g, cb, sbase, lane, rA > 0 ? jf + (done + cB) * KS : jlast, rA > 0 ? min(rA, E::U) : 1, KS, tofs, ra);
                E::compute(g, rb, cB, jf + done * KS, KS, b0, xs, wl, acc, mp);
                done += cB;
            }
        }
        // split-K partials, summed in kpart order
        if (KS > 1) {
#pragma unroll
            for (int tg = 0; tg < TG; ++tg)
#pragma unroll
                for (int G = 0; G < Sh::RG; ++G)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        red[(((wave * TG + tg) * Sh::RG + G) * 4 + q) * 64 + lane] = acc[tg][G][q];
            __syncthreads();
            if (kpart == 0) {
                for (int qq = 1; qq < KS; ++qq)
#pragma unroll
                    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
                        for (int G = 0; G < Sh::RG; ++G)
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                acc[tg][G][q] += red[((((wave + qq) * TG + tg) * Sh::RG + G) * 4 + q) * 64 + lane];
            }
            __syncthreads();
        }
        if (kpart == 0 && active) {
            const int i = lane & 15, oct = lane >> 4;
#pragma unroll
            for (int tg = 0; tg < TG; ++tg) {
#pragma unroll
                for (int G = 0; G < Sh::RG; ++G) {
                    const int64_t row = (int64_t)unit * 16 * Sh::RG + 16 * G + i;
                    if (row >= g.n) continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int t = 16 * tg + 4 * oct + q;
                        if (t < mp) y[(int64_t)t * g.n + row] = acc[tg][G][q];
                    }
                }
            }
        }
    }
}

typedef void (*mfma_fn)(MGeom, const void *, float *);

// tg: token groups per pass, 1 (co-batch calls, and qgemm where L > 2) or 2
// (qgemm, L <= 2: gemm_groups).  L = 16 serves only qgemm.
template <int FMT>
mfma_fn pick_mfma(int L, int tg = 1, int nw = WAVES)
{
    if (tg == 2) return L == 1 ? k_dense_mfma<FMT, 1, 2> : k_dense_mfma<FMT, 2, 2>;
    if (nw == MFMA_WIDE_WAVES) return k_dense_mfma<FMT, 8, 1, MFMA_WIDE_WAVES>;
    switch (L) {
    case 1: return k_dense_mfma<FMT, 1, 1>;
    case 2: return k_dense_mfma<FMT, 2, 1>;
    case 4: return k_dense_mfma<FMT, 4, 1>;
    case 8: return k_dense_mfma<FMT, 8, 1>;
    default: return k_dense_mfma<FMT, 16, 1>;
    }
}

mfma_fn mfma_kernel_q8_0(int L, int tg = 1, int nw = WAVES);
mfma_fn mfma_kernel_q4_0(int L, int tg = 1, int nw = WAVES);
mfma_fn mfma_kernel_mxfp4(int L, int tg = 1, int nw = WAVES);

} // namespace qg
