// qg_chain.h -- a chain of dense GEMVs run by one persistent kernel.
//
// A decode step streams its weight matrices one after another, each product
// depending on the previous one.  With one kernel per product every matrix
// pays a launch, a ramp-up of its memory stream and a drain: at 1.4-7 us of
// traffic per matrix that costs more than half the bandwidth.  Imparo answers
// the same problem on Metal with one persistent dispatch per decode layer and
// a grid barrier in place of each dispatch boundary (Imparo README,
// "Megakernel Decode").  Here one cooperative kernel walks the whole chain,
// one workgroup per compute unit, and the weight stream does not stop at the
// barriers:
//
//  * Work split.  Workgroup g owns tiles [g T / P, (g+1) T / P) of a link
//    (T tiles, P workgroups).  Its tiles' (tile, step) items, tile-major, are
//    cut into CW equal contiguous ranges, one per compute wave, so every wave
//    streams the same number of 16-byte records whatever the shape.  A wave
//    keeps one partial sum per tile it touches and leaves it in LDS; after a
//    workgroup barrier each tile's partials are added in wave order and across
//    the tile's L lanes of a row (a fixed order: bitwise reproducible).
//  * Weight prefetch.  A compute wave reads its items in batches of U, two
//    batches in flight ahead of the arithmetic, across link boundaries: weights
//    do not depend on the barrier, so while a workgroup waits for the others
//    its next product's first batches are already on their way from HBM.
//  * Barrier.  One control wave per workgroup writes the link's rows with
//    device-scope stores, waits for them, publishes the workgroup's epoch flag,
//    polls all workgroups' flags, and stages the next link's activations with
//    device-scope loads.  Device scope (the sc1 cache policy) makes those
//    accesses coherent across the MI355X's eight XCDs without writing back or
//    invalidating a whole L2, which is what an agent-scope fence does.  The
//    compute waves touch no barrier memory, so their waits on the memory
//    counter never include a barrier round trip, and the control wave has no
//    weight loads of its own to wait behind.
//  * Every barrier wait is bounded by a wall-clock limit (the 100 MHz
//    real-time counter): a wait that gives up records a timeout, and the
//    workgroup's rows of the links it computes afterwards are written as NaN,
//    so the kernel always finishes and a stale result cannot pass a check.
#pragma once
#include "qg_common.h"

namespace qg {

constexpr int CW = 7;                      // compute wavefronts per workgroup
constexpr int CTPB = 64 * (CW + 1);        // + one control wavefront
constexpr int CHAIN_MAX_WG = 256;          // flag slots (workgroups of a chain launch at most)
constexpr uint32_t CHAIN_MAGIC = 0x51474333u;
constexpr uint64_t CHAIN_WAIT_TICKS = 2000000;   // 20 ms of the 100 MHz real-time counter
constexpr size_t CHAIN_LDS_MAX = 150 * 1024;

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

// One link of the plan (device copy): the layout of its packed matrix (one
// activation window over the whole K: g.wblk = S * L), its activations and
// outputs, and the most tiles any workgroup owns.
struct ChainLink {
    Geom g;
    const void *x;
    float *y;
    int32_t tmax;
};

// LDS carve-up for M tokens: staged activations (the widest link's), the
// compute waves' partial sums [tile][wave][token][lane], then the finished
// rows [token][tmax * R].
struct ChainHdr {
    uint32_t magic;
    int32_t fmt, xt, m, count, grid;
    int64_t lds, part_off, out_off;
};

inline size_t chain_xs_bytes(int M, bool dot, int wblk) { return (size_t)M * (dot ? 4 : 8) * wblk * 16; }
inline size_t chain_part_bytes(int M, int tmax) { return (size_t)tmax * CW * M * 64 * 4; }
inline size_t chain_out_bytes(int M, int tmax, int R) { return (size_t)M * tmax * R * 4; }

// Items per weight batch: 6 Q8_0 records (2 KiB each per wave) or 12 4-bit
// ones (1 KiB), two batches in flight: 24 KiB per wave, 168 KiB per compute
// unit, enough to cover a barrier and the staging after it at the per-unit
// share of the HBM bandwidth.  4-bit co-batches of 4 or more tokens take 8
// (their wider arithmetic would otherwise spill registers).
template <int FMT, int M> struct ChainBatch { static constexpr int U = FMT == QG_Q8_0 ? 6 : M <= 3 ? 12 : 8; };

__device__ __forceinline__ void wg_tiles(int tiles, int grp, int P, int &t0, int &t1)
{
    t0 = (int)((int64_t)grp * tiles / P);
    t1 = (int)((int64_t)(grp + 1) * tiles / P);
}

// Items [lo, hi) of compute wave w among I items of its workgroup.
__device__ __forceinline__ void wave_items(int I, int w, int &lo, int &hi)
{
    lo = (int)((int64_t)w * I / CW);
    hi = (int)((int64_t)(w + 1) * I / CW);
}

// Device-scope (sc1) accesses: coherent across the XCDs without L2 fences.
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_dev_f32(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_dev_u32(uint32_t *p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until every vector memory access this wave issued has completed
// (loads returned, stores acknowledged at their scope).  The signal fences
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void wait_vmem()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0), expcnt(7), lgkmcnt(15)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ------------------------------------------------------------ control wave
// Waits until every workgroup published at least `target`.  Returns false if
// the wait gave up (the timeout is recorded in qg_chain_err).
__device__ __forceinline__ bool chain_poll(uint32_t target)
{
    const int lane = threadIdx.x & 63;
    const int P = gridDim.x;
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + CHAIN_WAIT_TICKS;
    constexpr int NF = CHAIN_MAX_WG / 64;   // flags per lane, all loaded in one round trip
    while (true) {
        uint32_t f[NF];
#pragma unroll
        for (int r = 0; r < NF; ++r) f[r] = lane + 64 * r < P ? ld_dev_u32(&qg_chain_flags[lane + 64 * r]) : target;
        bool ok = true;
#pragma unroll
        for (int r = 0; r < NF; ++r) ok &= (int32_t)(f[r] - target) >= 0;
        if (__all(ok)) return true;
        if (__builtin_amdgcn_s_memrealtime() > t_end) {
            if (lane == 0) st_dev_u32(&qg_chain_err, 1u);
            return false;
        }
    }
}

// Stages x (M tokens) of one link into LDS in the engine's form, with the 64
// lanes of the control wave: each lane issues the device-scope loads of up to
// CH blocks before writing any of them (one memory round trip per 64 * CH
// blocks).
template <int M, bool XBF16, bool DOT>
__device__ __forceinline__ void chain_stage(const Geom &g, const void *x, uint4 *xs)
{
    constexpr int QPB = DOT ? 4 : 8;
    constexpr int NW = XBF16 ? 8 : 16;      // 8-byte loads per block
    constexpr int CH = XBF16 ? 5 : 3;       // blocks per lane per round
    const int lane = threadIdx.x & 63;
    const int total = M * g.wblk;
    for (int base = 0; base < total; base += 64 * CH) {
        uint64_t raw[CH][NW];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = base + c * 64 + lane;
            const int t = idx / g.wblk, b = idx - t * g.wblk;
            const bool ok = idx < total && b < g.nb;
            const uint64_t *src = (const uint64_t *)((const uint8_t *)x +
                                                     ((int64_t)(ok ? t : 0) * g.k + (int64_t)(ok ? b : 0) * QK) *
                                                         (XBF16 ? 2 : 4));
#pragma unroll
            for (int i = 0; i < NW; ++i) raw[c][i] = ld_dev_u64(src + i);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = base + c * 64 + lane;
            if (idx >= total) continue;
            const int t = idx / g.wblk, bl = idx - t * g.wblk;
            uint4 r8[8], q[8];
#pragma unroll
            for (int i = 0; i < NW / 2; ++i)
                r8[i] = make_uint4((uint32_t)raw[c][2 * i], (uint32_t)(raw[c][2 * i] >> 32), (uint32_t)raw[c][2 * i + 1],
                                   (uint32_t)(raw[c][2 * i + 1] >> 32));
            stage_block<XBF16, DOT>(r8, q);
            if (bl >= g.nb) {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < QPB; ++i) xs[(t * QPB + i) * g.wblk + bl] = q[i];
        }
    }
}

// ------------------------------------------------------------ compute waves
// Position of a compute wave in its stream of items: link `li`, the next item
// `q` of its range [q, qe) of that link, and that item's tile (local to the
// workgroup) `tl` and step `j`.  Wave-uniform: kept in scalar registers.
struct ChainCursor {
    int li, q, qe, tl, j;
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The cursor at the first item, at or after link `li`, of a link in which
// this wave has items (li = nlinks at the end).
__device__ __forceinline__ ChainCursor cursor_at(const ChainLink *links, int nlinks, int grp, int P, int w, int li)
{
    ChainCursor c{nlinks, 0, 0, 0, 0};
    for (; li < nlinks; ++li) {
        const int tiles = links[li].g.tiles, S = links[li].g.S;
        int t0, t1, lo, hi;
        wg_tiles(tiles, grp, P, t0, t1);
        wave_items((t1 - t0) * S, w, lo, hi);
        if (lo < hi) {
            c.li = li;
            c.q = lo;
            c.qe = hi;
            c.tl = lo / S;
            c.j = lo - c.tl * S;
            break;
        }
    }
    c.li = uni(c.li);
    c.q = uni(c.q);
    c.qe = uni(c.qe);
    c.tl = uni(c.tl);
    c.j = uni(c.j);
    return c;
}

// A batch of up to U items of one link, in registers.
template <int FMT, int U>
struct ChainRegs {
    static constexpr int P = FMT == QG_Q8_0 ? 2 : 1;
    uint4 c[U][P];
    uint32_t s[U];
    int li, cnt, tl0, j0;          // link, items, first item's local tile and step
};

// Issues the loads of the next batch at the cursor and returns the cursor
// after it.  Every call issues U items' worth of loads (items past the batch
// repeat its last one, a cache hit), so the compiler's memory-counter waits
// stay exact; past the end of the stream it re-reads a valid record that is
// never used.  Addresses are a scalar base per item plus the lane's offset.
template <int FMT, int U>
__device__ __forceinline__ ChainCursor chain_issue(const ChainLink *links, int nlinks, int grp, int P, int w,
                                                   const ChainCursor c, ChainRegs<FMT, U> &b)
{
    constexpr int PP = ChainRegs<FMT, U>::P;
    constexpr int SB = FMT == QG_MXFP4 ? 1 : 2;
    const int lane = threadIdx.x & 63;
    const bool live = c.li < nlinks;
    const Geom &g = links[live ? c.li : nlinks - 1].g;
    const int S = g.S;
    int t0, t1;
    wg_tiles(g.tiles, grp, P, t0, t1);
    const int cnt = live ? min(U, c.qe - c.q) : 0;
    b.li = c.li;
    b.cnt = cnt;
    b.tl0 = c.tl;
    b.j0 = c.j;
    int tl = c.tl, j = c.j;
    const uint32_t coff = (uint32_t)lane * 16, soff = (uint32_t)lane * SB;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int tile = live ? t0 + tl : 0;
        const int jj = live ? j : 0;
        const uint8_t *cb = g.w + (int64_t)tile * g.ctb + (int64_t)jj * (PP * 1024);
        const uint8_t *sb = g.w + g.soff + (int64_t)tile * g.stb + (int64_t)jj * 64 * SB;
#pragma unroll
        for (int h = 0; h < PP; ++h) b.c[u][h] = ld_stream16(cb + h * 1024 + coff);
        if (FMT == QG_MXFP4)
            b.s[u] = ld_stream_u8(sb + soff);
        else
            b.s[u] = ld_stream_u16((const uint16_t *)(sb + soff));
        if (u + 1 < cnt && ++j == S) {       // position of the batch's next item
            j = 0;
            ++tl;
        }
    }
    if (!live) return c;
    if (c.q + cnt >= c.qe) return cursor_at(links, nlinks, grp, P, w, c.li + 1);
    if (++j == S) {                          // the item after the batch's last one
        j = 0;
        ++tl;
    }
    return ChainCursor{c.li, uni(c.q + cnt), c.qe, uni(tl), uni(j)};
}

// This wave's partial sums: the tile being summed (-1: none) and its values.
template <int M>
struct ChainAcc {
    int tl;
    float a[M];
};

template <int M>
__device__ __forceinline__ void acc_flush(ChainAcc<M> &acc, float *part, int w)
{
    const int lane = threadIdx.x & 63;
    if (acc.tl >= 0) {
#pragma unroll
        for (int t = 0; t < M; ++t) part[((acc.tl * CW + w) * M + t) * 64 + lane] = acc.a[t];
    }
#pragma unroll
    for (int t = 0; t < M; ++t) acc.a[t] = 0.0f;
}

// Adds the batch's items (all of one link) into the accumulators, flushing a
// tile's partials to LDS when an item starts another tile.
template <int FMT, bool XBF16, bool DOT, int M, int U>
__device__ __forceinline__ void chain_compute(const Geom &g, const ChainRegs<FMT, U> &b, const uint4 *xs,
                                              float *part, int w, ChainAcc<M> &acc)
{
    using E = Engine<FMT, XBF16, DOT, M, U>;
    const int slot = (threadIdx.x & 63) & (g.L - 1);
    int tl = b.tl0, j = b.j0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (u < b.cnt) {
            if (tl != acc.tl) {
                acc_flush<M>(acc, part, w);
                acc.tl = tl;
            }
            E::step(g, b.c[u], b.s[u], xs, j * g.L + slot, acc.a);
            // one item at a time: the scheduler may not hoist the next item's
            // activation reads (32 registers each) above this one's arithmetic
            __builtin_amdgcn_sched_barrier(0);
            if (++j == g.S) {
                j = 0;
                ++tl;
            }
        }
    }
}

template <int FMT, bool XBF16, bool DOT, int M>
__global__ __launch_bounds__(CTPB) void k_chain(const ChainLink *__restrict__ links, int nlinks, int part_off,
                                                int out_off)
{
    constexpr int U = ChainBatch<FMT, M>::U;
    using BR = ChainRegs<FMT, U>;
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ uint32_t s_base;
    // the wave index is uniform over the wave: keep it (and the whole item
    // cursor derived from it) in scalar registers
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int P = gridDim.x, grp = blockIdx.x;
    uint4 *xs = (uint4 *)smem;
    float *part = (float *)(smem + part_off);
    float *out = (float *)(smem + out_off);
    if (threadIdx.x == 0) s_base = ld_dev_u32(&qg_chain_gen);
    __syncthreads();
    const uint32_t base = s_base;

    if (wave == CW) {
        // ---------------------------------------------------- control wave
        chain_stage<M, XBF16, DOT>(links[0].g, links[0].x, xs);
        bool stale = false;                  // a barrier wait gave up: rows from here on are NaN
        for (int i = 0; i < nlinks; ++i) {
            const Geom &g = links[i].g;
            const int ostride = links[i].tmax * g.R;
            __syncthreads();                 // #1 activations of link i staged
            __syncthreads();                 // #2 partial sums in LDS
            __syncthreads();                 // #3 finished rows in LDS
            int t0, t1;
            wg_tiles(g.tiles, grp, P, t0, t1);
            const int r0 = t0 * g.R, nr = min(t1 * g.R, g.n) - r0;
            for (int idx = lane; idx < M * nr; idx += 64) {
                const int t = idx / nr, r = idx - t * nr;
                st_dev_f32(links[i].y + (int64_t)t * g.n + r0 + r, stale ? __builtin_nanf("") : out[t * ostride + r]);
            }
            wait_vmem();                     // this workgroup's rows of link i are visible device-wide
            if (lane == 0) st_dev_u32(&qg_chain_flags[grp], base + (uint32_t)i + 1);
            if (i + 1 < nlinks) {
                if (!chain_poll(base + (uint32_t)i + 1)) stale = true;    // link i complete everywhere
                chain_stage<M, XBF16, DOT>(links[i + 1].g, links[i + 1].x, xs);
            }
        }
        if (grp == 0) {
            chain_poll(base + (uint32_t)nlinks);
            if (lane == 0) st_dev_u32(&qg_chain_gen, base + (uint32_t)nlinks);
        }
        return;
    }

    // -------------------------------------------------------- compute waves
    ChainCursor cur = cursor_at(links, nlinks, grp, P, wave, 0);
    BR ra, rb;
    cur = chain_issue<FMT, U>(links, nlinks, grp, P, wave, cur, ra);
    cur = chain_issue<FMT, U>(links, nlinks, grp, P, wave, cur, rb);
    bool a_first = true;                     // the older batch in flight is ra
    for (int i = 0; i < nlinks; ++i) {
        const Geom &g = links[i].g;
        ChainAcc<M> acc;
        acc.tl = -1;
#pragma unroll
        for (int t = 0; t < M; ++t) acc.a[t] = 0.0f;
        __syncthreads();                     // #1 activations of link i staged
        // this wave's batches of link i, oldest first; a computed buffer is
        // refilled with the next batch of the stream before the other is used
        while (true) {
            if (a_first) {
                if (ra.li != i) break;
                chain_compute<FMT, XBF16, DOT, M, U>(g, ra, xs, part, wave, acc);
                cur = chain_issue<FMT, U>(links, nlinks, grp, P, wave, cur, ra);
            } else {
                if (rb.li != i) break;
                chain_compute<FMT, XBF16, DOT, M, U>(g, rb, xs, part, wave, acc);
                cur = chain_issue<FMT, U>(links, nlinks, grp, P, wave, cur, rb);
            }
            a_first = !a_first;
        }
        acc_flush<M>(acc, part, wave);
        __syncthreads();                     // #2 partial sums in LDS
        // each local tile: the partials of the waves that touched it, in wave
        // order, then the L lanes of each row
        int t0, t1;
        wg_tiles(g.tiles, grp, P, t0, t1);
        const int nt = t1 - t0, I = nt * g.S, ostride = links[i].tmax * g.R;
        for (int tl = wave; tl < nt; tl += CW) {
            float v[M];
#pragma unroll
            for (int t = 0; t < M; ++t) v[t] = 0.0f;
            for (int w = 0; w < CW; ++w) {
                int lo, hi;
                wave_items(I, w, lo, hi);
                if (lo < hi && lo < (tl + 1) * g.S && hi > tl * g.S) {      // wave w touched tile tl
#pragma unroll
                    for (int t = 0; t < M; ++t) v[t] += part[((tl * CW + w) * M + t) * 64 + lane];
                }
            }
            for (int off = 1; off < g.L; off <<= 1) {
#pragma unroll
                for (int t = 0; t < M; ++t) v[t] += __shfl_xor(v[t], off, 64);
            }
            if ((lane & (g.L - 1)) == 0) {
#pragma unroll
                for (int t = 0; t < M; ++t) out[t * ostride + tl * g.R + (lane >> g.lsh)] = v[t];
            }
        }
        __syncthreads();                     // #3 finished rows in LDS
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
