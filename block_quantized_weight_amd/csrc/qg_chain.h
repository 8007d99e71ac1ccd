// qg_chain.h -- a chain of dense GEMVs run by one persistent kernel.
//
// A decode step streams its weight matrices one after another, each product
// depending on the previous one; with one kernel per product every matrix
// pays a launch, a ramp-up and a drain of a few microseconds, which at
// 1.4-7 us of traffic per matrix costs more than half the bandwidth.  Imparo
// answers the same problem on Metal with one persistent dispatch per decode
// layer and a grid barrier in place of each dispatch boundary (Imparo README,
// "Megakernel Decode").  Here one cooperative kernel walks the whole chain,
// one workgroup per compute unit:
//
//  * every workgroup owns a balanced range of tiles of every link;
//  * product i+1 starts on a workgroup only after all workgroups finished
//    product i (grid barrier on per-workgroup epoch flags; each wait is
//    bounded and records a timeout instead of hanging);
//  * eight compute wavefronts only stream weights and compute.  Each keeps
//    its next batch of weights in flight at all times, across passes and
//    across link boundaries (weights do not depend on the barrier);
//  * one control wavefront does everything that must wait on memory it
//    wrote or read across the device: it polls the barrier, stages the
//    activations into LDS, writes the outputs and publishes completion.  On
//    gfx9 one counter tracks all of a wave's vector loads and stores in
//    order, so these waits in a compute wave would also wait for the weight
//    batches it has in flight.
#pragma once
#include "qg_common.h"

namespace qg {

constexpr int CWAVES = 8;                 // compute wavefronts per workgroup
constexpr int CTPB = 64 * (CWAVES + 1);   // + one control wavefront
constexpr int CHAIN_MAX_WG = 1024;        // flag slots
constexpr uint32_t CHAIN_MAGIC = 0x51474332u;
constexpr long CHAIN_SPIN_LIMIT = 400000;

// Device-resident barrier state.  Flags only grow: a launch reads the epoch
// base from qg_chain_gen, workgroup g publishes base + i + 1 after link i, and
// workgroup 0 advances qg_chain_gen after the final barrier.  Launches that
// overlap on one device would race on these words.  (Each translation unit
// that instantiates chain kernels has its own copy.)
static __device__ uint32_t qg_chain_flags[CHAIN_MAX_WG];
static __device__ uint32_t qg_chain_gen;
static __device__ uint32_t qg_chain_err;

// Reads (and optionally clears) this translation unit's barrier-timeout word.
inline int chain_error_read(bool clear)
{
    uint32_t v = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(qg_chain_err), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess)
        return -1;
    if (clear && v) {
        const uint32_t z = 0;
        if (hipMemcpyToSymbol(HIP_SYMBOL(qg_chain_err), &z, sizeof(z), 0, hipMemcpyHostToDevice) != hipSuccess)
            return -1;
    }
    return (int)v;
}

struct ChainLink {
    Geom g;              // layout of the link; KS / tpi chosen for CWAVES waves
    const void *x;
    float *y;
};

struct ChainHdr {
    uint32_t magic;
    int32_t fmt, xt, m, count, grid;
    int64_t lds;
};

// Steps per weight batch.  Two batches stay live across a whole pass (one in
// flight, one computing) beside the control wave's staging registers, so the
// wider compute variants (fp32 activations, more than 4 tokens) take smaller
// batches to stay within the 168 registers this launch shape allows without
// spilling (Q4_0 with fp32 activations and one token spills even at 2).
template <int FMT, bool XBF16, bool DOT, int M> struct ChainBatch {
    static constexpr int U = !XBF16 && FMT == QG_Q4_0 && M == 1 ? 1
                             : !XBF16 || (FMT == QG_Q8_0 && M > 4) ? 2
                             : FMT == QG_Q8_0                      ? 4
                             : DOT                                 ? (M > 4 ? 4 : 8)
                                                                   : 4;
};

// LDS carve-up of one link: staged activations, split-K partials, and a
// double-buffered block of finished rows for the control wave.
template <int M, bool DOT>
struct ChainLds {
    uint4 *xs;
    float *red, *out;
    __device__ ChainLds(uint8_t *smem, const Geom &g)
    {
        constexpr int QPB = DOT ? 4 : 8;
        xs = (uint4 *)smem;
        red = (float *)(smem + (size_t)M * QPB * g.wblk * 16);
        out = red + CWAVES * M * 64;
    }
};

inline size_t chain_lds_bytes(int M, bool dot, int wblk, int rows_per_pass)
{
    const int QPB = dot ? 4 : 8;
    return (size_t)M * QPB * wblk * 16 + (size_t)CWAVES * M * 64 * 4 + (size_t)2 * M * rows_per_pass * 4;
}

// ------------------------------------------------------------ control wave
// Wait until every workgroup published at least `target`.
__device__ __forceinline__ void chain_poll(uint32_t target)
{
    const int lane = threadIdx.x & 63;
    const int P = gridDim.x;
    long spins = 0;
    while (true) {
        bool ok = true;
        for (int q = lane; q < P; q += 64) {
            const uint32_t f = __hip_atomic_load(&qg_chain_flags[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = ok && (int32_t)(f - target) >= 0;
        }
        if (__all(ok)) break;
        if (++spins > CHAIN_SPIN_LIMIT) {
            if (lane == 0) __hip_atomic_store(&qg_chain_err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

__device__ __forceinline__ void chain_publish(uint32_t value)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_store(&qg_chain_flags[blockIdx.x], value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stages x (M tokens) of one link into LDS with the 64 lanes of the control
// wave; each lane issues the loads of CH blocks before writing any of them.
template <int M, int FMT, bool XBF16, bool DOT>
__device__ __forceinline__ void chain_stage(const Geom &g, const void *x, uint4 *xs)
{
    constexpr int QPB = DOT ? 4 : 8;
    constexpr int CH = XBF16 ? 2 : 1;       // blocks per lane in flight (fp32 blocks are twice the registers)
    constexpr int NLD = XBF16 ? 4 : 8;       // 16-byte loads per block
    const int lane = threadIdx.x & 63;
    const int total = M * g.wblk;
    for (int base = 0; base < total; base += 64 * CH) {
        uint4 raw[CH][NLD];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = base + c * 64 + lane;
            const int t = idx / g.wblk, b = idx - t * g.wblk;
            const bool ok = idx < total && b < g.nb;
            const uint8_t *src = (const uint8_t *)x +
                                 ((int64_t)(ok ? t : 0) * g.k + (int64_t)(ok ? b : 0) * QK) * (XBF16 ? 2 : 4);
#pragma unroll
            for (int i = 0; i < NLD; ++i) raw[c][i] = ld_global16(src + 16 * i);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = base + c * 64 + lane;
            if (idx >= total) continue;
            const int t = idx / g.wblk, bl = idx - t * g.wblk;
            const bool ok = bl < g.nb;
            uint4 q[8];
            stage_block<XBF16, DOT>(raw[c], q);
            if (!ok) {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < QPB; ++i) xs[(t * QPB + i) * g.wblk + bl] = q[i];
        }
    }
}

// ------------------------------------------------------------ compute waves
// Work of a compute wave inside one pass of one link.
struct PassWork {
    const uint8_t *ct, *st;   // code / scale base of the wave's tile (a valid tile even when idle)
    int jf, nsteps, tile, KS;
};

__device__ __forceinline__ void wg_tiles(const Geom &g, int grp, int P, int64_t &t0, int64_t &t1)
{
    t0 = (int64_t)grp * g.tiles / P;
    t1 = (int64_t)(grp + 1) * g.tiles / P;
}

__device__ __forceinline__ PassWork pass_work(const Geom &g, int64_t t0, int64_t t1, int p)
{
    const int wave = threadIdx.x >> 6;
    const int tsub = wave >> g.ksh, kpart = wave & (g.KS - 1);
    PassWork w;
    const int64_t tile = t0 + (int64_t)p * g.tpi + tsub;
    const bool active = tile < t1;
    const int64_t tl = active ? tile : (t0 < g.tiles ? t0 : 0);
    w.tile = (int)tile;
    w.ct = g.w + tl * g.ctb;
    w.st = g.w + g.soff + tl * g.stb;
    w.jf = kpart;
    w.KS = g.KS;
    w.nsteps = (active && kpart < g.S) ? (g.S - kpart + g.KS - 1) / g.KS : 0;
    return w;
}

// The first pass after (i, p) in which this wave has work; false at the end.
__device__ __forceinline__ bool next_work(const ChainLink *links, int nlinks, int grp, int P, int i, int p,
                                          PassWork &out)
{
    while (true) {
        Geom g = links[i].g;
        int64_t t0, t1;
        wg_tiles(g, grp, P, t0, t1);
        const int npass = (int)((t1 - t0 + g.tpi - 1) / g.tpi);
        if (++p >= npass) {
            if (++i >= nlinks) return false;
            p = -1;
            continue;
        }
        out = pass_work(g, t0, t1, p);
        if (out.nsteps > 0) return true;
    }
}

// Streams the wave's batches of one pass: `A` holds the first batch (already
// in flight); each step loads the following batch -- or the first batch of
// the wave's next working pass (`nx`) -- into the other buffer before
// computing.  Returns true if the next pass's first batch ended up in `B`.
template <typename E, int M>
__device__ __forceinline__ bool chain_pass_loop(const Geom &g, const PassWork &w, const PassWork &nx, int slot,
                                                const uint4 *xs, float acc[M],
                                                typename E::Regs &A, typename E::Regs &B)
{
    constexpr int U = E::U;
    const int nb = (w.nsteps + U - 1) / U;
    const int ncnt = max(1, min(nx.nsteps, U));
    int b = 0;
    while (true) {
        {
            const bool more = b + 1 < nb;
            const int c = more ? min(w.nsteps - (b + 1) * U, U) : ncnt;
            E::load(g, more ? w.ct : nx.ct, more ? w.st : nx.st, threadIdx.x & 63,
                    more ? w.jf + (b + 1) * U * w.KS : nx.jf, c, more ? w.KS : nx.KS, B);
        }
        E::compute(g, A, min(w.nsteps - b * U, U), w.jf + b * U * w.KS, w.KS, slot, 0, xs, acc);
        if (++b >= nb) return true;
        {
            const bool more = b + 1 < nb;
            const int c = more ? min(w.nsteps - (b + 1) * U, U) : ncnt;
            E::load(g, more ? w.ct : nx.ct, more ? w.st : nx.st, threadIdx.x & 63,
                    more ? w.jf + (b + 1) * U * w.KS : nx.jf, c, more ? w.KS : nx.KS, A);
        }
        E::compute(g, B, min(w.nsteps - b * U, U), w.jf + b * U * w.KS, w.KS, slot, 0, xs, acc);
        if (++b >= nb) return false;
    }
}

template <int FMT, bool XBF16, bool DOT, int M>
__global__ __launch_bounds__(CTPB) void k_chain(const ChainLink *__restrict__ links, int nlinks)
{
    using E = Engine<FMT, XBF16, DOT, M, ChainBatch<FMT, XBF16, DOT, M>::U>;
    using LdsT = ChainLds<M, DOT>;
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ uint32_t s_base;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool control = wave == CWAVES;
    const int P = gridDim.x, grp = blockIdx.x;
    if (threadIdx.x == 0) s_base = __hip_atomic_load(&qg_chain_gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t base = s_base;

    typename E::Regs ra, rb;
    bool phase = false;             // false: the next working pass's first batch is in ra
    if (!control) {
        PassWork first;
        if (next_work(links, nlinks, grp, P, 0, -1, first))
            E::load(links[0].g, first.ct, first.st, lane, first.jf, max(1, min(first.nsteps, E::U)), first.KS, ra);
    }

    for (int i = 0; i < nlinks; ++i) {
        const Geom g = links[i].g;
        int64_t t0, t1;
        wg_tiles(g, grp, P, t0, t1);
        const int npass = (int)((t1 - t0 + g.tpi - 1) / g.tpi);
        const int rows_pp = g.tpi * g.R;
        LdsT lds(smem, g);

        if (control) {
            if (i > 0) chain_poll(base + (uint32_t)i);   // product i-1 complete everywhere
            chain_stage<M, FMT, XBF16, DOT>(g, links[i].x, lds.xs);
        }
        __syncthreads();                                   // activations of link i staged

        const int tsub = wave >> g.ksh, kpart = wave & (g.KS - 1);
        const int rsub = lane >> g.lsh, slot = lane & (g.L - 1);
        for (int p = 0; p < npass; ++p) {
            float *outp = lds.out + (p & 1) * M * rows_pp;
            float acc[M];
#pragma unroll
            for (int t = 0; t < M; ++t) acc[t] = 0.0f;
            if (!control) {
                const PassWork w = pass_work(g, t0, t1, p);
                if (w.nsteps > 0) {
                    PassWork nx;
                    if (!next_work(links, nlinks, grp, P, i, p, nx)) {
                        nx = w;             // nothing left: repeat this pass's first step
                        nx.nsteps = 1;
                    }
                    const bool flip = phase ? chain_pass_loop<E, M>(g, w, nx, slot, lds.xs, acc, rb, ra)
                                            : chain_pass_loop<E, M>(g, w, nx, slot, lds.xs, acc, ra, rb);
                    if (flip) phase = !phase;
                }
                if (g.KS > 1) {
#pragma unroll
                    for (int t = 0; t < M; ++t) lds.red[(wave * M + t) * 64 + lane] = acc[t];
                }
            }
            if (g.KS > 1) __syncthreads();                // split-K partials in LDS
            if (!control) {
                if (g.KS > 1 && kpart == 0) {
                    for (int qq = 1; qq < g.KS; ++qq)
#pragma unroll
                        for (int t = 0; t < M; ++t) acc[t] += lds.red[((wave + qq) * M + t) * 64 + lane];
                }
                for (int off = 1; off < g.L; off <<= 1) {
#pragma unroll
                    for (int t = 0; t < M; ++t) acc[t] += __shfl_xor(acc[t], off, 64);
                }
                if (kpart == 0) {
#pragma unroll
                    for (int t = 0; t < M; ++t)
                        if ((t & (g.L - 1)) == slot) outp[t * rows_pp + tsub * g.R + rsub] = acc[t];
                }
            }
            __syncthreads();                               // rows of pass p in LDS
            if (control) {
                const int64_t row0 = (t0 + (int64_t)p * g.tpi) * g.R;
                const int64_t rend = t1 * g.R < g.n ? t1 * g.R : g.n;
                for (int idx = lane; idx < M * rows_pp; idx += 64) {
                    const int t = idx / rows_pp, rl = idx - t * rows_pp;
                    const int64_t row = row0 + rl;
                    if (row < rend) st_global_f32(links[i].y + (int64_t)t * g.n + row, outp[idx]);
                }
            }
        }
        if (control) chain_publish(base + (uint32_t)i + 1);
    }
    // final barrier, then workgroup 0 moves the epoch base for the next launch
    if (control && grp == 0) {
        chain_poll(base + (uint32_t)nlinks);
        if (lane == 0)
            __hip_atomic_store(&qg_chain_gen, base + (uint32_t)nlinks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int FMT, bool XBF16, bool DOT>
const void *pick_chain(int m)
{
    switch (m) {
    case 1: return (const void *)k_chain<FMT, XBF16, DOT, 1>;
    case 2: return (const void *)k_chain<FMT, XBF16, DOT, 2>;
    case 3: return (const void *)k_chain<FMT, XBF16, DOT, 3>;
    case 4: return (const void *)k_chain<FMT, XBF16, DOT, 4>;
    case 5: return (const void *)k_chain<FMT, XBF16, DOT, 5>;
    case 6: return (const void *)k_chain<FMT, XBF16, DOT, 6>;
    case 7: return (const void *)k_chain<FMT, XBF16, DOT, 7>;
    default: return (const void *)k_chain<FMT, XBF16, DOT, 8>;
    }
}

// per-format tables (defined in qg_<fmt>.hip)
const void *chain_kernel_q8_0(int xt, int m);
const void *chain_kernel_q4_0(int xt, int m);
const void *chain_kernel_mxfp4(int xt, int m);
int chain_error_q8_0(bool clear);
int chain_error_q4_0(bool clear);
int chain_error_mxfp4(bool clear);

} // namespace qg
