#pragma once
// qg_moe_stream.h -- top-k expert product, streaming form.
//
// Each workgroup reads the routing ids once, lists the distinct selected
// experts in ascending order (imp keeps routing on the device so the decode
// graph holds no host round trip: imp release notes v0.7.0, known issues),
// and splits every expert's slots into "items" of at most MS slots.  All the
// activation rows the call needs are staged once.  IS waves share a row tile
// of the expert shape and split its items (wave p takes items p, p+IS, ...);
// each wave streams all steps of its items back to back, the first weight
// batch of its next item being loaded while the current one is computed, so
// the weight stream does not drain at expert boundaries and no barrier sits
// inside it.
//   gate_up:      after each item the wave reduces across its row's lanes
//                 and stores the item's slot rows.
//   down-combine: the wave folds router-weighted slot results into per-token
//                 registers; at the end the IS waves of a tile add their
//                 partials in a fixed order through LDS.
// Only selected experts are read, each once per tile; the result is
// deterministic (fixed item assignment and reduction order).
#include "qg_common.h"

namespace qg {

constexpr int MOE_STREAM_LDS = 96 * 1024;   // staged activations + partials per workgroup

// Work items (expert, up to MS slots), built in LDS by wave 0.
struct MoeItems {
    int count;
    int e[64];
    int n[64];
    int s[64][QG_MAX_M];
};

// Slot -> staged activation row of one item (uniform over the wave).
template <int MS>
struct SlotMap {
    int r[MS];
    int n;
    __device__ __forceinline__ int operator()(int t) const { return r[t]; }
    __device__ __forceinline__ int count() const { return n; }
};

// Splits the distinct experts' slots into items of at most ms slots, in
// ascending expert order and ascending slot order.  Called by the whole
// workgroup after distinct_experts; ends with a barrier.
__device__ __forceinline__ void build_items(const int *s_ids, const int *s_list, int nexp, int nslots, int ms,
                                            MoeItems *it)
{
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int ni = 0;
        for (int d = 0; d < nexp; ++d) {
            const int e = s_list[d];
            const bool match = lane < nslots && s_ids[lane] == e;
            const uint64_t mask = __ballot(match);
            const int cnt = __popcll(mask);
            const int rank = __popcll(mask & ((1ull << lane) - 1));
            for (int c0 = 0; c0 < cnt; c0 += ms, ++ni) {
                if (match && rank >= c0 && rank < c0 + ms) it->s[ni][rank - c0] = lane;
                if (lane == 0) {
                    it->e[ni] = e;
                    it->n[ni] = min(ms, cnt - c0);
                }
            }
        }
        if (lane == 0) it->count = ni;
    }
    __syncthreads();
}

// Where a wave's tile of one item lives.
struct ItemWork {
    const uint8_t *ct, *st;
    int jf, nsteps, KS;
};

// Streams one item: A holds its first batch (in flight).  Each round loads
// the following batch -- or the first batch of the next item (nx) -- into the
// other buffer before computing.  Returns true if nx's first batch is in B.
template <typename E, int MS, typename XMap>
__device__ __forceinline__ bool stream_item(const Geom &g, const ItemWork &w, const ItemWork &nx, int slot,
                                            const uint4 *xs, const float *corr, float acc[MS], const XMap &xm,
                                            typename E::Regs &A, typename E::Regs &B)
{
    constexpr int U = E::U;
    const int lane = threadIdx.x & 63;
    const int nb = (w.nsteps + U - 1) / U;
    const int ncnt = max(1, min(nx.nsteps, U));
    int b = 0;
    while (true) {
        {
            const bool more = b + 1 < nb;
            const int c = more ? min(w.nsteps - (b + 1) * U, U) : ncnt;
            E::load(g, more ? w.ct : nx.ct, more ? w.st : nx.st, lane, more ? w.jf + (b + 1) * U * w.KS : nx.jf, c,
                    w.KS, B);
        }
        E::compute(g, A, min(w.nsteps - b * U, U), w.jf + b * U * w.KS, w.KS, slot, 0, xs, corr, acc, xm);
        if (++b >= nb) return true;
        {
            const bool more = b + 1 < nb;
            const int c = more ? min(w.nsteps - (b + 1) * U, U) : ncnt;
            E::load(g, more ? w.ct : nx.ct, more ? w.st : nx.st, lane, more ? w.jf + (b + 1) * U * w.KS : nx.jf, c,
                    w.KS, A);
        }
        E::compute(g, B, min(w.nsteps - b * U, U), w.jf + b * U * w.KS, w.KS, slot, 0, xs, corr, acc, xm);
        if (++b >= nb) return false;
    }
}

inline __host__ __device__ size_t moe_stream_lds(int fmt, bool dot, int nrows, int wblk, int mode)
{
    size_t b = (size_t)nrows * x_quads(fmt, dot) * wblk * 16;
    if (x_aux(fmt)) b += (size_t)nrows * wblk * 4;
    if (mode == QG_MOE_DOWN_COMBINE) b += (size_t)WAVES * QG_MAX_M * 64 * 4;
    return b;
}

// grid = ceil(tiles / tpi) workgroups, tpi = WAVES / IS tiles each; one
// (tile, item subset) per wave.  Geom: KS = 1, one activation window over K.
template <int FMT, bool XBF16, bool DOT, int MS, int MODE>
__global__ __launch_bounds__(TPB) void k_moe_stream(Geom g, MoeArgs a, const void *__restrict__ x, float *__restrict__ y)
{
    using E = Engine<FMT, XBF16, DOT, MS>;
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_ids[64];
    __shared__ int s_list[64];
    __shared__ int s_count;
    __shared__ MoeItems it;
    constexpr int QPB = x_quads(FMT, DOT);
    const int nslots = a.m * a.top_k;
    const int nrows = MODE == QG_MOE_GATE_UP ? a.m : nslots;
    uint4 *xs = (uint4 *)smem;
    float *corr = (float *)(smem + (size_t)nrows * QPB * g.wblk * 16);
    float *red = corr + (x_aux(FMT) ? nrows * g.wblk : 0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int IS = a.isplit;
    const int tsub = wave / IS, ipart = wave - tsub * IS;
    const int rsub = lane >> g.lsh, slot = lane & (g.L - 1);

    distinct_experts(a.ids, nslots, a.n_experts, s_ids, s_list, &s_count);
    build_items(s_ids, s_list, s_count, nslots, MS, &it);
    const int ni = it.count;

    const int tile = blockIdx.x * g.tpi + tsub;
    const int tl = tile < g.tiles ? tile : 0;
    const int nsteps = (tile < g.tiles && ipart < ni) ? g.S : 0;
    auto work = [&](int i) {
        const uint8_t *w = a.experts + (int64_t)it.e[i] * a.expert_bytes;
        ItemWork iw;
        iw.ct = w + (int64_t)tl * g.ctb;
        iw.st = w + g.soff + (int64_t)tl * g.stb;
        iw.jf = 0;
        iw.nsteps = nsteps;
        iw.KS = 1;
        return iw;
    };
    typename E::Regs ra, rb;
    if (nsteps > 0) {
        const ItemWork w0 = work(ipart);
        E::load(g, w0.ct, w0.st, lane, w0.jf, min(nsteps, E::U), 1, ra);
    }

    // stage every activation row of the call (row r = token for gate_up,
    // slot for down), one window over all of K
    {
        const int total = nrows * g.wblk;
        for (int idx = threadIdx.x; idx < total; idx += (int)blockDim.x) {
            const int r = idx / g.wblk, bl = idx - r * g.wblk;
            uint4 raw[8], q[8];
            float av = 0.0f;
            if (bl < g.nb) {
                const int64_t off = (int64_t)r * g.k + (int64_t)bl * QK;
                if (XBF16) {
                    const uint4 *src = (const uint4 *)((const uint16_t *)x + off);
#pragma unroll
                    for (int i = 0; i < 4; ++i) raw[i] = ld_global16(src + i);
                } else {
                    const uint4 *src = (const uint4 *)((const float *)x + off);
#pragma unroll
                    for (int i = 0; i < 8; ++i) raw[i] = ld_global16(src + i);
                }
                av = stage_block<FMT, XBF16, DOT>(raw, q);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < QPB; ++i) xs[(r * QPB + i) * g.wblk + bl] = q[i];
            if (x_aux(FMT)) corr[r * g.wblk + bl] = av;
        }
    }
    __syncthreads();

    const int64_t row = (int64_t)tile * g.R + rsub;
    float tok[QG_MAX_M];
#pragma unroll
    for (int t = 0; t < QG_MAX_M; ++t) tok[t] = 0.0f;
    bool in_a = true;               // the current item's first batch is in ra
    for (int i = ipart; i < ni; i += IS) {
        SlotMap<MS> sm;
        sm.n = it.n[i];
#pragma unroll
        for (int t = 0; t < MS; ++t) {
            const int sid = it.s[i][min(t, sm.n - 1)];
            sm.r[t] = MODE == QG_MOE_GATE_UP ? sid / a.top_k : sid;
        }
        float acc[MS];
#pragma unroll
        for (int t = 0; t < MS; ++t) acc[t] = 0.0f;
        if (nsteps > 0) {
            const ItemWork w = work(i);
            ItemWork nx = w;
            if (i + IS < ni) {
                nx = work(i + IS);
            } else {
                nx.nsteps = 1;      // nothing follows: repeat this item's first step
            }
            const bool flip = in_a ? stream_item<E, MS>(g, w, nx, slot, xs, corr, acc, sm, ra, rb)
                                   : stream_item<E, MS>(g, w, nx, slot, xs, corr, acc, sm, rb, ra);
            if (flip) in_a = !in_a;
        }
        if (MODE == QG_MOE_GATE_UP) {
            for (int off = 1; off < g.L; off <<= 1) {
#pragma unroll
                for (int t = 0; t < MS; ++t) acc[t] += __shfl_xor(acc[t], off, 64);
            }
            if (nsteps > 0 && row < g.n) {
#pragma unroll
                for (int t = 0; t < MS; ++t)
                    if (t < sm.n && (t & (g.L - 1)) == slot) y[(int64_t)it.s[i][t] * g.n + row] = acc[t];
            }
        } else {
#pragma unroll
            for (int t = 0; t < MS; ++t) {
                if (t >= sm.n) break;
                const int sid = it.s[i][t];
                const float gw = a.gw[sid];
                const int tk = sid / a.top_k;
#pragma unroll
                for (int q = 0; q < QG_MAX_M; ++q)
                    if (q == tk) tok[q] = __builtin_fmaf(gw, acc[t], tok[q]);
            }
        }
    }
    if (MODE == QG_MOE_DOWN_COMBINE) {
        // the IS waves' partials of the tile, added in ipart order
        if (IS > 1) {
#pragma unroll
            for (int t = 0; t < QG_MAX_M; ++t) red[(wave * QG_MAX_M + t) * 64 + lane] = tok[t];
            __syncthreads();
            if (ipart == 0) {
                for (int q = 1; q < IS; ++q)
#pragma unroll
                    for (int t = 0; t < QG_MAX_M; ++t) tok[t] += red[((wave + q) * QG_MAX_M + t) * 64 + lane];
            }
        }
        for (int off = 1; off < g.L; off <<= 1) {
#pragma unroll
            for (int t = 0; t < QG_MAX_M; ++t) tok[t] += __shfl_xor(tok[t], off, 64);
        }
        if (ipart == 0 && tile < g.tiles && row < g.n) {
#pragma unroll
            for (int t = 0; t < QG_MAX_M; ++t)
                if (t < a.m && (t & (g.L - 1)) == slot) y[(int64_t)t * g.n + row] = tok[t];
        }
    }
}

typedef void (*moe_stream_fn)(Geom, MoeArgs, const void *, float *);

template <int FMT, bool XBF16, bool DOT>
moe_stream_fn pick_moe_stream(int mode, int ms)
{
    if (mode == QG_MOE_GATE_UP) {
        switch (ms) {
        case 1: return k_moe_stream<FMT, XBF16, DOT, 1, QG_MOE_GATE_UP>;
        case 2: return k_moe_stream<FMT, XBF16, DOT, 2, QG_MOE_GATE_UP>;
        case 4: return k_moe_stream<FMT, XBF16, DOT, 4, QG_MOE_GATE_UP>;
        default: return k_moe_stream<FMT, XBF16, DOT, 8, QG_MOE_GATE_UP>;
        }
    }
    switch (ms) {
    case 1: return k_moe_stream<FMT, XBF16, DOT, 1, QG_MOE_DOWN_COMBINE>;
    case 2: return k_moe_stream<FMT, XBF16, DOT, 2, QG_MOE_DOWN_COMBINE>;
    case 4: return k_moe_stream<FMT, XBF16, DOT, 4, QG_MOE_DOWN_COMBINE>;
    default: return k_moe_stream<FMT, XBF16, DOT, 8, QG_MOE_DOWN_COMBINE>;
    }
}

moe_stream_fn moe_stream_kernel_q8_0(int xt, int mode, int ms);
moe_stream_fn moe_stream_kernel_q4_0(int xt, int mode, int ms);
moe_stream_fn moe_stream_kernel_mxfp4(int xt, int mode, int ms);

} // namespace qg
