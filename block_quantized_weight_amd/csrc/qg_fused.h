#pragma once
// qg_fused.h -- the dense GEMV with the decode step's neighbours fused in:
// RMS normalisation of the activations in the staging, a SwiGLU gate or a
// residual add in the epilogue, fp32 or bf16 output.
//
// The pages report such fusions as hand-made, measured choices (Imparo
// README, "Design Rules"; "Bonsai CUDA Validation", where an extra RMS/Add
// tail fusion is listed as reviewed; imp release notes v0.4, a fused
// RMSNorm-gated + SiLU kernel) without defining the operations.  The
// definitions used are the published ones:
//   RMSNorm  x' = x * r * gamma,  r = 1 / sqrt(mean(x^2) + eps)
//            (Zhang and Sennrich, "Root Mean Square Layer Normalization")
//   SwiGLU   o = SiLU(g) * u, SiLU(v) = v / (1 + exp(-v)), g = rows [0, F)
//            of the product and u = rows [F, 2F) (Shazeer, "GLU Variants
//            Improve Transformer"; the gate-first split is a reading of the
//            pages' gate_up matrices, whose N is twice the down matrix's K).
//
// Design on gfx950:
//  * Normalisation.  The product is linear in x, so W (x r gamma) =
//    r * (W (x gamma)): x * gamma is formed in fp32 while staging (exact to
//    one rounding, and kept in fp32 -- a bf16 copy would cost up to 2^-9 of
//    each activation) and r is applied to the row totals.  r comes from a
//    sum of squares over the whole row that every workgroup forms itself,
//    while staging when one window holds the row (fixed order: per-thread
//    partials, a xor butterfly, then the waves in order), with the first
//    weight loads already in flight; all workgroups hold the same r and no
//    extra launch is needed.
//  * SwiGLU.  F is a multiple of the tile's rows, so the up tile of gate
//    tile t is t + F/R.  A wave takes half a gate tile in its lanes 0..31 and
//    the same half of the up tile in lanes 32..63, so the work units are as
//    many as the tiles and the grid is the plain product's; the gate and up
//    totals of a row meet by one lane swap, and only F outputs are written.
//    (Layouts of 64 lanes per row have one-row tiles: there eight-wave
//    workgroups split gate and up tiles and meet through LDS.)
//  * Residual and bf16 output in the store.
#include <type_traits>

#include "qg_common.h"

namespace qg {

// Arguments of the fused epilogue.
struct EpiArgs {
    const float *gamma;          // RMSNorm weights [k] (16-B aligned) when normalising
    float eps;
    const float *residual;       // [m][n_out] fp32 or null
    void *y;                     // [m][n_out] fp32 or bf16
    int32_t n_out;               // output rows: n, or n / 2 with SwiGLU
    int32_t half_tiles;          // SwiGLU: tiles of the gate half (up tile = gate tile + half_tiles); 0 without
    int32_t y_bf16;
};

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + expf(-v)); }

// Stager of normalised activations: window w of x * gamma in the engine's
// fp32 form, and the per-wave partial sums of x^2 of each token slot in
// s_part[wave][t] (read after the engine's barrier that follows the
// staging; the epilogue turns them into 1/rms).  With a single window the
// sums are formed while staging, each element once; with several, a
// separate pass over the row on the first call forms them.
template <bool XBF16>
struct NormStage {
    const float *gamma;
    float *s_part;               // LDS [WAVES][QG_MAX_M]
    bool have;

    template <int M>
    static __device__ __forceinline__ void publish(float (&ss)[M], float *s_part)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int t = 0; t < M; ++t)
            for (int off = 32; off >= 1; off >>= 1) ss[t] += __shfl_xor(ss[t], off, 64);
        if (lane == 0) {
#pragma unroll
            for (int t = 0; t < M; ++t) s_part[wave * QG_MAX_M + t] = ss[t];
        }
    }

    template <int M>
    __device__ __forceinline__ void rms_pass(const Geom &g, const void *x, const Slots &sl)
    {
        constexpr int PER = XBF16 ? 8 : 4;           // elements per 16-B load
        const int nq = g.k / PER;
        float ss[M];
#pragma unroll
        for (int t = 0; t < M; ++t) ss[t] = 0.0f;
        for (int i = threadIdx.x; i < nq; i += (int)blockDim.x) {
#pragma unroll
            for (int t = 0; t < M; ++t) {
                const uint4 v = ld_global16((const uint8_t *)x + ((int64_t)sl.xrow[t] * g.k + (int64_t)i * PER) * (XBF16 ? 2 : 4));
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (XBF16) {
                        const float a = __builtin_bit_cast(float, w4[j] << 16);
                        const float b = __builtin_bit_cast(float, w4[j] & 0xFFFF0000u);
                        ss[t] = fmaf(a, a, ss[t]);
                        ss[t] = fmaf(b, b, ss[t]);
                    } else {
                        const float a = __builtin_bit_cast(float, w4[j]);
                        ss[t] = fmaf(a, a, ss[t]);
                    }
                }
            }
        }
        publish<M>(ss, s_part);
    }

    template <int M, int FMT>
    __device__ __forceinline__ void run(const Geom &g, const void *x, const Slots &sl, int w, uint4 *xs)
    {
        const bool sums_here = g.nwin == 1;
        if (!sums_here && !have) rms_pass<M>(g, x, sl);
        have = true;
        constexpr int QPB = x_quads(FMT, false);
        const int b0 = w * g.SW * g.L;
        // one half block (16 activations) per thread and iteration
        const int total = 2 * M * g.wblk;
        float ss[M];
#pragma unroll
        for (int t = 0; t < M; ++t) ss[t] = 0.0f;
        for (int idx = threadIdx.x; idx < total; idx += (int)blockDim.x) {
            const int half = idx & 1, item = idx >> 1;
            const int t = item / g.wblk, bl = item - t * g.wblk, b = b0 + bl;
            const int64_t xo = (int64_t)sl.xrow[t] * g.k + (int64_t)b * QK + half * 16;
            uint4 *dst = xs + (t * QPB + half * 4) * g.wblk + bl;
            float sq = 0.0f;
            if (b < g.nb) {
                uint4 raw[4];
                if (XBF16) {
                    const uint4 *src = (const uint4 *)((const uint16_t *)x + xo);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const uint4 v = ld_global16(src + i);
                        raw[2 * i] = make_uint4(v.x << 16, v.x & 0xFFFF0000u, v.y << 16, v.y & 0xFFFF0000u);
                        raw[2 * i + 1] = make_uint4(v.z << 16, v.z & 0xFFFF0000u, v.w << 16, v.w & 0xFFFF0000u);
                    }
                } else {
                    const uint4 *src = (const uint4 *)((const float *)x + xo);
#pragma unroll
                    for (int i = 0; i < 4; ++i) raw[i] = ld_global16(src + i);
                }
                const uint4 *gs = (const uint4 *)(gamma + (int64_t)b * QK + half * 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 gv = ld_global16(gs + i);
                    const float x0 = __builtin_bit_cast(float, raw[i].x), x1 = __builtin_bit_cast(float, raw[i].y);
                    const float x2 = __builtin_bit_cast(float, raw[i].z), x3 = __builtin_bit_cast(float, raw[i].w);
                    sq = fmaf(x0, x0, sq);
                    sq = fmaf(x1, x1, sq);
                    sq = fmaf(x2, x2, sq);
                    sq = fmaf(x3, x3, sq);
                    const float p0 = x0 * __builtin_bit_cast(float, gv.x), p1 = x1 * __builtin_bit_cast(float, gv.y);
                    const float p2 = x2 * __builtin_bit_cast(float, gv.z), p3 = x3 * __builtin_bit_cast(float, gv.w);
                    dst[i * g.wblk] = make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                                                 __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[i * g.wblk] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int tt = 0; tt < M; ++tt) ss[tt] += tt == t ? sq : 0.0f;
        }
        if (sums_here) publish<M>(ss, s_part);
    }
};

// Plain stager for the fused kernel without normalisation (the engine's own).
template <bool XBF16, bool DOT>
struct PlainStage {
    template <int M, int FMT>
    __device__ __forceinline__ void run(const Geom &g, const void *x, const Slots &sl, int w, uint4 *xs)
    {
        XStage<XBF16, DOT>::template run<M, FMT>(g, x, sl, w, xs);
    }
};

// 1/rms of token slot t from the per-wave partial sums (waves in order).
template <int NW>
__device__ __forceinline__ float rinv_of(const float *s_part, int t, int k, float eps)
{
    float tot = 0.0f;
#pragma unroll
    for (int q = 0; q < NW; ++q) tot += s_part[q * QG_MAX_M + t];
    return 1.0f / sqrtf(tot / (float)k + eps);
}

__device__ __forceinline__ void store_out(const EpiArgs &e, int64_t o, float v)
{
    if (e.residual) v += e.residual[o];
    if (e.y_bf16)
        ((uint16_t *)e.y)[o] = bf16_rne(v);
    else
        ((float *)e.y)[o] = v;
}

// Without a gate: TPB threads, the plain product's tile grouping.
template <int FMT, bool XBF16, bool DOT, int M, bool NORM>
__global__ __launch_bounds__(TPB) void k_dense_ep(Geom g, EpiArgs e, const void *__restrict__ x)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int QPB = x_quads(FMT, DOT);
    uint4 *xs = (uint4 *)smem;
    float *red = (float *)(smem + (size_t)M * QPB * g.wblk * 16);
    __shared__ int32_t s_rows[QG_MAX_M];
    __shared__ float s_part[WAVES * QG_MAX_M];
    if (threadIdx.x < QG_MAX_M) s_rows[threadIdx.x] = threadIdx.x;   // read only after the first barrier
    Slots sl{s_rows, s_rows};
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tsub = wave >> g.ksh, kpart = wave & (g.KS - 1);
    const int rsub = lane >> g.lsh, slot = lane & (g.L - 1);
    typedef typename std::conditional<NORM, NormStage<XBF16>, PlainStage<XBF16, DOT>>::type Stager;
    Stager st;
    if constexpr (NORM) {
        st.gamma = e.gamma;
        st.s_part = s_part;
        st.have = false;
    }
    bool staged = false;
    for (int grp = blockIdx.x; grp < g.ngroups; grp += gridDim.x) {
        const int tile = grp * g.tpi + tsub;
        float acc[M];
        Engine<FMT, XBF16, DOT, M>::pass_st(g, x, sl, tile, staged, xs, acc, st);
        reduce_partials<M>(g, red, acc);
        const int64_t row = (int64_t)tile * g.R + rsub;
        if (kpart == 0 && tile < g.tiles && row < e.n_out) {
            const float ts = tensor_scale<FMT>(g);
#pragma unroll
            for (int t = 0; t < M; ++t) {
                if ((t & (g.L - 1)) != slot) continue;
                float v = NORM ? acc[t] * rinv_of<WAVES>(s_part, t, g.k, e.eps) : acc[t];
                if (FMT == QG_NVFP4) v *= ts;
                store_out(e, (int64_t)t * e.n_out + row, v);
            }
        }
    }
}

// Without normalisation or gate, where the plain product takes its one-batch
// form (one_batch_u): the same pass, then the residual / output-type epilogue.
template <int FMT, bool XBF16, bool DOT, int M, int U>
__global__ __launch_bounds__(TPB, one_waves(FMT, XBF16, U)) void k_dense_one_ep(Geom g, EpiArgs e,
                                                                                 const void *__restrict__ x)
{
    float acc[M];
    dense_one_pass<FMT, XBF16, DOT, M, U>(g, x, acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tile = blockIdx.x * g.tpi + (wave >> g.ksh);
    const int64_t row = (int64_t)tile * g.R + (lane >> g.lsh);
    if ((wave & (g.KS - 1)) == 0 && tile < g.tiles && row < e.n_out) {
        const float ts = tensor_scale<FMT>(g);
#pragma unroll
        for (int t = 0; t < M; ++t)
            if ((t & (g.L - 1)) == (lane & (g.L - 1)))
                store_out(e, (int64_t)t * e.n_out + row, FMT == QG_NVFP4 ? acc[t] * ts : acc[t]);
    }
}

// With the SwiGLU gate, layouts of at most 32 lanes per row: the plain
// product's grid of TPB-thread workgroups over work units u = 2 t + h, one
// per tile count.  A wave's lanes 0..31 read records 32 h .. 32 h + 31 of gate
// tile t (rows 32 h / L .. of the tile), lanes 32..63 the same records of up
// tile t + half_tiles; each load instruction reads two contiguous 512-byte
// halves.  After the split-K and row reductions (within 32-lane halves, as
// L <= 32) a row's gate and up totals are 32 lanes apart, one lane swap.
template <int FMT, bool XBF16, bool DOT, int M, bool NORM>
__global__ __launch_bounds__(TPB) void k_dense_glu_lanes(Geom g, EpiArgs e, const void *__restrict__ x)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int QPB = x_quads(FMT, DOT);
    uint4 *xs = (uint4 *)smem;
    float *red = (float *)(smem + (size_t)M * QPB * g.wblk * 16);
    __shared__ int32_t s_rows[QG_MAX_M];
    __shared__ float s_part[WAVES * QG_MAX_M];
    if (threadIdx.x < QG_MAX_M) s_rows[threadIdx.x] = threadIdx.x;   // read only after the first barrier
    Slots sl{s_rows, s_rows};
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tsub = wave >> g.ksh, kpart = wave & (g.KS - 1);
    const int slot = lane & (g.L - 1);
    const bool upl = lane >= 32;
    typedef typename std::conditional<NORM, NormStage<XBF16>, PlainStage<XBF16, DOT>>::type Stager;
    Stager st;
    if constexpr (NORM) {
        st.gamma = e.gamma;
        st.s_part = s_part;
        st.have = false;
    }
    bool staged = false;
    for (int grp = blockIdx.x; grp < g.ngroups; grp += gridDim.x) {
        const int u = grp * g.tpi + tsub;
        const int t = u >> 1, h = u & 1;
        const bool active = t < e.half_tiles;
        const int tile = active ? t + (upl ? e.half_tiles : 0) : 0;
        const int rl = 32 * h + (lane & 31);
        float acc[M];
        Engine<FMT, XBF16, DOT, M>::pass_core(g, x, sl, g.w + (int64_t)tile * g.ctb, g.w + g.soff + (int64_t)tile * g.stb,
                                              rl, active, staged, xs, acc, st);
        reduce_partials<M>(g, red, acc);
        float up[M];
#pragma unroll
        for (int q = 0; q < M; ++q) up[q] = __shfl_xor(acc[q], 32, 64);
        const int64_t row = (int64_t)t * g.R + rl / g.L;
        if (!upl && kpart == 0 && active && row < e.n_out) {
            const float ts = tensor_scale<FMT>(g);
#pragma unroll
            for (int q = 0; q < M; ++q) {
                if ((q & (g.L - 1)) != slot) continue;
                float gv = acc[q], uv = up[q];
                if (FMT == QG_NVFP4) {
                    gv *= ts;
                    uv *= ts;
                }
                if (NORM) {
                    const float r = rinv_of<WAVES>(s_part, q, g.k, e.eps);
                    gv *= r;
                    uv *= r;
                }
                store_out(e, (int64_t)q * e.n_out + row, silu(gv) * uv);
            }
        }
    }
}

// With the SwiGLU gate, 64 lanes per row (one-row tiles): workgroups of GLU_WAVES waves.  The first half of the
// waves runs g.tpi / 2 gate tiles (KS waves each), the second half the up
// tiles of the same rows (gate tile + half_tiles); the up waves hand their
// row totals to the gate waves through LDS, which finish the outputs.
constexpr int GLU_WAVES = 8;

template <int FMT, bool XBF16, bool DOT, int M, bool NORM>
__global__ __launch_bounds__(64 * GLU_WAVES) void k_dense_glu(Geom g, EpiArgs e, const void *__restrict__ x)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int QPB = x_quads(FMT, DOT);
    uint4 *xs = (uint4 *)smem;
    float *red = (float *)(smem + (size_t)M * QPB * g.wblk * 16);
    __shared__ int32_t s_rows[QG_MAX_M];
    __shared__ float s_part[GLU_WAVES * QG_MAX_M];
    __shared__ float s_up[GLU_WAVES / 2][QG_MAX_M][64];
    if (threadIdx.x < QG_MAX_M) s_rows[threadIdx.x] = threadIdx.x;   // read only after the first barrier
    Slots sl{s_rows, s_rows};
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tsub = wave >> g.ksh, kpart = wave & (g.KS - 1);
    const int rsub = lane >> g.lsh, slot = lane & (g.L - 1);
    const int pp = g.tpi >> 1;                      // gate/up pairs per workgroup
    const bool up = tsub >= pp;
    const int p = up ? tsub - pp : tsub;
    typedef typename std::conditional<NORM, NormStage<XBF16>, PlainStage<XBF16, DOT>>::type Stager;
    Stager st;
    if constexpr (NORM) {
        st.gamma = e.gamma;
        st.s_part = s_part;
        st.have = false;
    }
    bool staged = false;
    for (int grp = blockIdx.x; grp < g.ngroups; grp += gridDim.x) {
        const int pair = grp * pp + p;
        const bool active = pair < e.half_tiles;
        const int tile = active ? (up ? pair + e.half_tiles : pair) : g.tiles;
        float acc[M];
        Engine<FMT, XBF16, DOT, M>::pass_st(g, x, sl, tile, staged, xs, acc, st);
        reduce_partials<M>(g, red, acc);
        if (up && kpart == 0 && active) {
#pragma unroll
            for (int t = 0; t < M; ++t)
                if ((t & (g.L - 1)) == slot) s_up[p][t][rsub] = acc[t];
        }
        __syncthreads();
        const int64_t row = (int64_t)pair * g.R + rsub;
        if (!up && kpart == 0 && active && row < e.n_out) {
            const float ts = tensor_scale<FMT>(g);
#pragma unroll
            for (int t = 0; t < M; ++t) {
                if ((t & (g.L - 1)) != slot) continue;
                float gv = acc[t], uv = s_up[p][t][rsub];
                if (FMT == QG_NVFP4) {
                    gv *= ts;
                    uv *= ts;
                }
                if (NORM) {
                    const float r = rinv_of<GLU_WAVES>(s_part, t, g.k, e.eps);
                    gv *= r;
                    uv *= r;
                }
                store_out(e, (int64_t)t * e.n_out + row, silu(gv) * uv);
            }
        }
        __syncthreads();                             // s_up is rewritten by the next group
    }
}

typedef void (*dense_ep_fn)(Geom, EpiArgs, const void *);

// GLU: 0 none, 1 lanes (<= 32 lanes per row), 2 eight-wave workgroups.
template <int FMT, bool XBF16, bool DOT, bool NORM, int GLU, int M>
dense_ep_fn ep_kernel()
{
    if constexpr (GLU == 1)
        return k_dense_glu_lanes<FMT, XBF16, DOT, M, NORM>;
    else if constexpr (GLU == 2)
        return k_dense_glu<FMT, XBF16, DOT, M, NORM>;
    else
        return k_dense_ep<FMT, XBF16, DOT, M, NORM>;
}

template <int FMT, bool XBF16, bool DOT, bool NORM, int GLU>
dense_ep_fn pick_dense_ep(int m)
{
    switch (m) {
    case 1: return ep_kernel<FMT, XBF16, DOT, NORM, GLU, 1>();
    case 2: return ep_kernel<FMT, XBF16, DOT, NORM, GLU, 2>();
    case 3: return ep_kernel<FMT, XBF16, DOT, NORM, GLU, 3>();
    case 4: return ep_kernel<FMT, XBF16, DOT, NORM, GLU, 4>();
    case 5: return ep_kernel<FMT, XBF16, DOT, NORM, GLU, 5>();
    case 6: return ep_kernel<FMT, XBF16, DOT, NORM, GLU, 6>();
    case 7: return ep_kernel<FMT, XBF16, DOT, NORM, GLU, 7>();
    default: return ep_kernel<FMT, XBF16, DOT, NORM, GLU, 8>();
    }
}

template <int FMT, int GLU>
dense_ep_fn pick_dense_ep_glu(int xt, int m, bool norm)
{
    constexpr bool DOTB = FMT != QG_Q8_0;
    if (norm)
        return xt == QG_BF16 ? pick_dense_ep<FMT, true, false, true, GLU>(m) : pick_dense_ep<FMT, false, false, true, GLU>(m);
    return xt == QG_BF16 ? pick_dense_ep<FMT, true, DOTB, false, GLU>(m) : pick_dense_ep<FMT, false, false, false, GLU>(m);
}

// Normalising kernels stage fp32 (x * gamma); the others stage as the plain
// product does (bf16 pairs for 4-bit codes with bf16 activations).
template <int FMT>
dense_ep_fn pick_dense_ep_fmt(int xt, int m, bool norm, int glu)
{
    return glu == 1 ? pick_dense_ep_glu<FMT, 1>(xt, m, norm)
           : glu == 2 ? pick_dense_ep_glu<FMT, 2>(xt, m, norm) : pick_dense_ep_glu<FMT, 0>(xt, m, norm);
}

template <int FMT, bool XBF16, bool DOT, int M>
dense_ep_fn pick_dense_one_ep_u(int u)
{
    return u == 8 ? k_dense_one_ep<FMT, XBF16, DOT, M, 8>
                  : u == 12 ? k_dense_one_ep<FMT, XBF16, DOT, M, 12> : k_dense_one_ep<FMT, XBF16, DOT, M, ONE_MAX_U>;
}

// m tokens, u steps in flight, as pick_dense_one.
template <int FMT>
dense_ep_fn pick_dense_one_ep(int xt, int m, int u)
{
    if constexpr (FMT == QG_Q8_0) {
        if (u == 10)
            return xt == QG_BF16 ? k_dense_one_ep<FMT, true, false, 1, 10> : k_dense_one_ep<FMT, false, false, 1, 10>;
        return xt == QG_BF16 ? k_dense_one_ep<FMT, true, false, 1, 8> : k_dense_one_ep<FMT, false, false, 1, 8>;
    } else {
        if (xt == QG_BF16)
            return m == 1 ? pick_dense_one_ep_u<FMT, true, true, 1>(u)
                   : m == 2 ? pick_dense_one_ep_u<FMT, true, true, 2>(u) : pick_dense_one_ep_u<FMT, true, true, 3>(u);
        return m == 1 ? pick_dense_one_ep_u<FMT, false, false, 1>(u)
               : m == 2 ? pick_dense_one_ep_u<FMT, false, false, 2>(u) : pick_dense_one_ep_u<FMT, false, false, 3>(u);
    }
}

dense_ep_fn dense_ep_kernel_q8_0(int xt, int m, bool norm, int glu);
dense_ep_fn dense_ep_kernel_q4_0(int xt, int m, bool norm, int glu);
dense_ep_fn dense_ep_kernel_mxfp4(int xt, int m, bool norm, int glu);
dense_ep_fn dense_ep_kernel_nvfp4(int xt, int m, bool norm, int glu);
dense_ep_fn dense_one_ep_kernel_q8_0(int xt, int m, int u);
dense_ep_fn dense_one_ep_kernel_q4_0(int xt, int m, int u);
dense_ep_fn dense_one_ep_kernel_mxfp4(int xt, int m, int u);
dense_ep_fn dense_one_ep_kernel_nvfp4(int xt, int m, int u);

} // namespace qg
