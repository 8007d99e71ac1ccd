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
//
// Fused neighbours (the definitions of qg_fused.h): gate_up may normalise
// the token rows (x * gamma staged in fp32, sum of x^2 formed while staging,
// 1/rms applied to the row totals) and gate its output (SwiGLU: a workgroup
// holds tpi / 2 gate/up tile pairs; the waves of each tile stream their
// items and leave their per-slot row totals in LDS, and after one barrier
// the workgroup combines gate and up and writes F outputs per slot);
// down-combine may add a residual; either writes fp32 or bf16.
#include "qg_fused.h"

namespace qg {

constexpr int MOE_STREAM_LDS = 96 * 1024;   // staged activations + partials per workgroup
constexpr int MOE_STREAM_LDS_GLU = 144 * 1024;   // the same plus the gate's per-slot row totals

// Work items (expert, up to MS slots), built in LDS by wave 0.
struct MoeItems {
    int count;
    int e[64];
    int n[64];
    int s[64][QG_MAX_M];
    int tk[64][QG_MAX_M];       // the token of each slot (slot / top_k), divided once here
    float g[64][QG_MAX_M];      // down-combine: each slot's router weight, read with the ids
};

// Slot -> staged activation row of one item (uniform over the wave).
template <int MS>
struct SlotMap {
    int r[MS];
    int n;
    __device__ __forceinline__ int operator()(int t) const { return r[t]; }
    __device__ __forceinline__ int count() const { return n; }
};

// The work list, built by wave 0 from the routing ids held in registers
// (lane s holds slot s's id): the distinct valid experts in ascending order,
// each expert's slots split into items of at most ms slots in ascending slot
// order.  Two passes of lane reads (v_readlane) in which every lane works out
// its own slot's place -- one over the slots, one over the distinct experts
// -- so no step waits on LDS.  The caller synchronises afterwards.
__device__ __forceinline__ void route_items(int id, float gw, int nslots, int n_experts, int ms, int top_k,
                                            MoeItems *it)
{
    const int lane = threadIdx.x & 63;
    const bool valid = lane < nslots && id >= 0 && id < n_experts;
    const int e = valid ? id : 0x7FFFFFFF;
    // pass over the slots: slots of the same expert before this one, and in all
    int before = 0, same = 0;
    for (int q = 0; q < nslots; ++q) {
        const bool eq = __builtin_amdgcn_readlane(e, q) == e;
        same += eq ? 1 : 0;
        before += (eq && q < lane) ? 1 : 0;
    }
    const bool first = valid && before == 0;
    const int nit = (same + ms - 1) / ms;                // items of this lane's expert
    // pass over the distinct experts: items of smaller experts come first
    int base = 0, total = 0;
    for (uint64_t b = __ballot(first); b; b &= b - 1) {
        const int q = __builtin_ctzll(b);
        const int eq = __builtin_amdgcn_readlane(e, q);
        const int nq = __builtin_amdgcn_readlane(nit, q);
        base += eq < e ? nq : 0;
        total += nq;
    }
    if (valid) {
        const int item = base + before / ms, pos = before - (before / ms) * ms;
        it->s[item][pos] = lane;
        it->tk[item][pos] = lane / top_k;
        it->g[item][pos] = gw;
        if (pos == 0) {
            it->e[item] = e;
            it->n[item] = min(ms, same - before);
        }
    }
    if (lane == 0) it->count = total;
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
                                            const uint4 *xs, float acc[MS], const XMap &xm,
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
        E::compute(g, A, min(w.nsteps - b * U, U), w.jf + b * U * w.KS, w.KS, slot, 0, xs, acc, xm);
        if (++b >= nb) return true;
        {
            const bool more = b + 1 < nb;
            const int c = more ? min(w.nsteps - (b + 1) * U, U) : ncnt;
            E::load(g, more ? w.ct : nx.ct, more ? w.st : nx.st, lane, more ? w.jf + (b + 1) * U * w.KS : nx.jf, c,
                    w.KS, A);
        }
        E::compute(g, B, min(w.nsteps - b * U, U), w.jf + b * U * w.KS, w.KS, slot, 0, xs, acc, xm);
        if (++b >= nb) return false;
    }
}

// Dynamic LDS: staged rows, then down-combine's split partials or, with the
// gate, the per-slot row totals of the tile pairs.
inline __host__ __device__ size_t moe_stream_lds(int fmt, bool dot, int nrows, int wblk, int mode, int glu_slots = 0,
                                                 int rows_per_tile = 0, int nw = WAVES)
{
    size_t b = (size_t)nrows * x_quads(fmt, dot) * wblk * 16;
    if (mode == QG_MOE_DOWN_COMBINE) b += (size_t)nw * QG_MAX_M * 64 * 4;
    if (glu_slots) b += (size_t)WAVES * glu_slots * rows_per_tile * 4;
    return b;
}

// grid = ceil(tiles / tpi) workgroups, tpi = NW / IS tiles each (with
// the gate: gate tiles, e.half_tiles of them); one (tile, item subset) per
// wave.  Geom: KS = 1, one activation window over K.  NORM (gate_up only):
// stage x * gamma in fp32 (DOT false).  GLU (gate_up only): SwiGLU.
template <int FMT, bool XBF16, bool DOT, int MS, int MODE, bool NORM, bool GLU, int UB = Batch<FMT, DOT>::U,
          int NW = WAVES>
__global__ __launch_bounds__(64 * NW) void k_moe_stream(Geom g, MoeArgs a, EpiArgs e, const void *__restrict__ x)
{
    static_assert(!NORM || !DOT, "normalised rows are staged in fp32");
    static_assert(MODE == QG_MOE_GATE_UP || (!NORM && !GLU), "down-combine fuses only the residual");
    static_assert(NW == WAVES || MODE == QG_MOE_DOWN_COMBINE, "wider workgroups serve down-combine only");
    using E = Engine<FMT, XBF16, DOT, MS, UB>;
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ MoeItems it;
    __shared__ float s_part[NW * QG_MAX_M];
    constexpr int QPB = x_quads(FMT, DOT);
    const int nslots = a.m * a.top_k;
    const int nrows = MODE == QG_MOE_GATE_UP ? a.m : nslots;
    uint4 *xs = (uint4 *)smem;
    float *red = (float *)(smem + (size_t)nrows * QPB * g.wblk * 16);
    float *res = red;               // GLU: [2][PP][nslots][R] row totals (gate_up has no down partials)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int IS = a.isplit;
    const int tsub = wave / IS, ipart = wave - tsub * IS;
    const int rsub = lane >> g.lsh, slot = lane & (g.L - 1);

    // Activations do not depend on the routing: every thread issues the loads
    // of its first PF staging units before the ids are even known.  (LDS
    // already limits this kernel to one workgroup per compute unit, so the
    // registers cost no occupancy.)
    constexpr int PF = XBF16 ? 4 : 2;
    constexpr int NLD = XBF16 ? 4 : 8;
    const int total = nrows * g.wblk;
    auto unit_src = [&](int idx) {
        const int r = idx / g.wblk, bl = idx - r * g.wblk;
        return (const uint8_t *)x + ((int64_t)r * g.k + (int64_t)min(bl, g.nb - 1) * QK) * (XBF16 ? 2 : 4);
    };
    const int my_id = a.ids[min(lane, nslots - 1)];    // lanes past the slots are ignored by the routing
    // down-combine: the slot's router weight, loaded here beside its id (read
    // inside the weight stream, it would wait for the weight batch in flight)
    const float my_gw = MODE == QG_MOE_DOWN_COMBINE ? a.gw[min(lane, nslots - 1)] : 0.0f;
    // keep these loads ahead of the activation loads (the memory counter is in
    // order, so the routing would otherwise wait for all of them)
    __builtin_amdgcn_sched_barrier(0);
    // a fixed number of loads (units past the end repeat the last one), so
    // the wait for the ids below does not also wait for these
    uint4 pre[PF][8];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const uint8_t *src = unit_src(min((int)threadIdx.x + p * (int)blockDim.x, total - 1));
#pragma unroll
        for (int i = 0; i < NLD; ++i) pre[p][i] = ld_global16(src + 16 * i);
    }

    if (wave == 0) route_items(my_id, my_gw, nslots, a.n_experts, MS, a.top_k, &it);
    __syncthreads();
    const int ni = it.count;
    // with the gate (PP = tpi / 2 pairs per workgroup): tile slots [0, PP)
    // hold gate tiles, [PP, 2 PP) the matching up tiles, IS waves each
    const int PP = g.tpi / 2;
    const int gpair = blockIdx.x * PP + (tsub % PP);
    const bool upw = GLU && tsub >= PP;
    const int tile = GLU ? (gpair < e.half_tiles ? gpair + (upw ? e.half_tiles : 0) : g.tiles)
                         : blockIdx.x * g.tpi + tsub;
    const int tl = tile < g.tiles ? tile : 0;
    const int nsteps = (tile < g.tiles && ipart < ni) ? g.S : 0;
    auto work = [&](int i) {
        // i past the list (a wave with nothing to stream): expert 0, never used
        const uint8_t *w = a.experts + (int64_t)(i < ni ? it.e[i] : 0) * a.expert_bytes;
        ItemWork iw;
        iw.ct = w + (int64_t)tl * g.ctb;
        iw.st = w + g.soff + (int64_t)tl * g.stb;
        iw.jf = 0;
        iw.nsteps = nsteps;
        iw.KS = 1;
        return iw;
    };
    // The first batch is loaded by every wave (waves with nothing to stream
    // load one step of expert 0 and ignore it): with the load unconditional,
    // the staging below waits for the activations only, not for these weights.
    typename E::Regs ra, rb;
    {
        const ItemWork w0 = work(ipart);
        E::load(g, w0.ct, w0.st, lane, w0.jf, max(1, min(nsteps, E::U)), 1, ra);
    }

    // stage every activation row of the call (row r = token for gate_up,
    // slot for down), one window over all of K
    float ss[QG_MAX_M];             // NORM: this thread's sums of x^2 per token row
#pragma unroll
    for (int t = 0; t < QG_MAX_M; ++t) ss[t] = 0.0f;
    auto stage_unit = [&](int idx, const uint4 (&raw)[8]) {
        const int r = idx / g.wblk, bl = idx - r * g.wblk;
        uint4 q[8];
        if (bl < g.nb) {
            if constexpr (NORM) {
                // x (exact in fp32) times gamma, in the fp32 form; x^2 summed per row
                uint4 xf[8];
                if (XBF16) {
                    const uint32_t *rw = (const uint32_t *)raw;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        xf[i] = make_uint4(rw[2 * i] << 16, rw[2 * i] & 0xFFFF0000u, rw[2 * i + 1] << 16,
                                           rw[2 * i + 1] & 0xFFFF0000u);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) xf[i] = raw[i];
                }
                const uint4 *gs = (const uint4 *)(e.gamma + (int64_t)bl * QK);
                float sq = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint4 gv = ld_global16(gs + i);
                    const float x0 = __builtin_bit_cast(float, xf[i].x), x1 = __builtin_bit_cast(float, xf[i].y);
                    const float x2 = __builtin_bit_cast(float, xf[i].z), x3 = __builtin_bit_cast(float, xf[i].w);
                    sq = fmaf(x0, x0, sq);
                    sq = fmaf(x1, x1, sq);
                    sq = fmaf(x2, x2, sq);
                    sq = fmaf(x3, x3, sq);
                    xf[i] = make_uint4(__builtin_bit_cast(uint32_t, x0 * __builtin_bit_cast(float, gv.x)),
                                       __builtin_bit_cast(uint32_t, x1 * __builtin_bit_cast(float, gv.y)),
                                       __builtin_bit_cast(uint32_t, x2 * __builtin_bit_cast(float, gv.z)),
                                       __builtin_bit_cast(uint32_t, x3 * __builtin_bit_cast(float, gv.w)));
                }
#pragma unroll
                for (int t = 0; t < QG_MAX_M; ++t) ss[t] += t == r ? sq : 0.0f;
                stage_block<false, false>(xf, q);
            } else {
                stage_block<XBF16, DOT>(raw, q);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < QPB; ++i) xs[(r * QPB + i) * g.wblk + bl] = q[i];
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        const int idx = (int)threadIdx.x + p * (int)blockDim.x;
        if (idx < total) stage_unit(idx, pre[p]);
    }
    for (int idx = (int)threadIdx.x + PF * (int)blockDim.x; idx < total; idx += (int)blockDim.x) {
        uint4 raw[8];
        const uint8_t *src = unit_src(idx);
#pragma unroll
        for (int i = 0; i < NLD; ++i) raw[i] = ld_global16(src + 16 * i);
        stage_unit(idx, raw);
    }
    if constexpr (NORM) NormStage<XBF16>::template publish<QG_MAX_M>(ss, s_part);
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
            const int q = min(t, sm.n - 1);
            sm.r[t] = MODE == QG_MOE_GATE_UP ? it.tk[i][q] : it.s[i][q];
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
            const bool flip = in_a ? stream_item<E, MS>(g, w, nx, slot, xs, acc, sm, ra, rb)
                                   : stream_item<E, MS>(g, w, nx, slot, xs, acc, sm, rb, ra);
            if (flip) in_a = !in_a;
        }
        if (MODE == QG_MOE_GATE_UP) {
            for (int off = 1; off < g.L; off <<= 1) {
#pragma unroll
                for (int t = 0; t < MS; ++t) acc[t] += __shfl_xor(acc[t], off, 64);
            }
            if constexpr (GLU) {
                // row totals of this wave's tile per slot: res[up][pair][slot][row in tile]
                if (nsteps > 0) {
#pragma unroll
                    for (int t = 0; t < MS; ++t)
                        if (t < sm.n && (t & (g.L - 1)) == slot)
                            res[(((upw ? PP : 0) + tsub % PP) * nslots + it.s[i][t]) * g.R + rsub] = acc[t];
                }
            } else if (nsteps > 0 && row < e.n_out) {
#pragma unroll
                for (int t = 0; t < MS; ++t) {
                    if (t < sm.n && (t & (g.L - 1)) == slot) {
                        const float v = NORM ? acc[t] * rinv_of<WAVES>(s_part, sm.r[t], g.k, e.eps) : acc[t];
                        store_out(e, (int64_t)it.s[i][t] * e.n_out + row, v);
                    }
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < MS; ++t) {
                if (t >= sm.n) break;
                const float gw = it.g[i][t];
                const int tk = it.tk[i][t];
#pragma unroll
                for (int q = 0; q < QG_MAX_M; ++q)
                    if (q == tk) tok[q] = __builtin_fmaf(gw, acc[t], tok[q]);
            }
        }
    }
    if constexpr (GLU) {
        // every wave has left its totals; the workgroup writes SiLU(g) * u
        __syncthreads();
        const int per = nslots * g.R;
        for (int idx = threadIdx.x; idx < PP * per; idx += (int)blockDim.x) {
            const int pr = idx / per, rem = idx - pr * per;
            const int sid = rem / g.R, rs = rem - sid * g.R;
            const int pair = blockIdx.x * PP + pr;
            const int id = a.ids[sid];
            if (pair >= e.half_tiles || id < 0 || id >= a.n_experts) continue;     // no such pair, or no output
            float gv = res[(pr * nslots + sid) * g.R + rs], uv = res[((PP + pr) * nslots + sid) * g.R + rs];
            if (NORM) {
                const float r = rinv_of<WAVES>(s_part, sid / a.top_k, g.k, e.eps);
                gv *= r;
                uv *= r;
            }
            store_out(e, (int64_t)sid * e.n_out + (int64_t)pair * g.R + rs, silu(gv) * uv);
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
                if (t < a.m && (t & (g.L - 1)) == slot) store_out(e, (int64_t)t * g.n + row, tok[t]);
        }
    }
}

typedef void (*moe_stream_fn)(Geom, MoeArgs, EpiArgs, const void *);

template <int FMT, bool XBF16, bool DOT, int MODE, bool NORM, bool GLU, int UB = Batch<FMT, DOT>::U, int NW = WAVES>
moe_stream_fn pick_moe_stream_ms(int ms)
{
    switch (ms) {
    case 1: return k_moe_stream<FMT, XBF16, DOT, 1, MODE, NORM, GLU, UB, NW>;
    case 2: return k_moe_stream<FMT, XBF16, DOT, 2, MODE, NORM, GLU, UB, NW>;
    case 4: return k_moe_stream<FMT, XBF16, DOT, 4, MODE, NORM, GLU, UB, NW>;
    default: return k_moe_stream<FMT, XBF16, DOT, 8, MODE, NORM, GLU, UB, NW>;
    }
}

// gate_up: the plain form, or normalised and/or gated (normalised rows are
// staged in fp32, so those kernels take DOT false); down-combine: one form
// (residual and output type are arguments).  short_items: the plain gate_up
// over items of at most 4 steps per lane, in batches of 4 steps; wide:
// down-combine in workgroups of WIDE_WAVES waves.
constexpr int WIDE_WAVES = 8;
template <int FMT, bool XBF16, bool DOT>
moe_stream_fn pick_moe_stream(int mode, int ms, bool norm, bool glu, bool short_items, bool wide)
{
    if (mode == QG_MOE_DOWN_COMBINE)
        return wide ? pick_moe_stream_ms<FMT, XBF16, DOT, QG_MOE_DOWN_COMBINE, false, false, Batch<FMT, DOT>::U,
                                         WIDE_WAVES>(ms)
                    : pick_moe_stream_ms<FMT, XBF16, DOT, QG_MOE_DOWN_COMBINE, false, false>(ms);
    if (norm)
        return glu ? pick_moe_stream_ms<FMT, XBF16, false, QG_MOE_GATE_UP, true, true>(ms)
                   : pick_moe_stream_ms<FMT, XBF16, false, QG_MOE_GATE_UP, true, false>(ms);
    if (glu) return pick_moe_stream_ms<FMT, XBF16, DOT, QG_MOE_GATE_UP, false, true>(ms);
    return short_items ? pick_moe_stream_ms<FMT, XBF16, DOT, QG_MOE_GATE_UP, false, false, 4>(ms)
                       : pick_moe_stream_ms<FMT, XBF16, DOT, QG_MOE_GATE_UP, false, false>(ms);
}

moe_stream_fn moe_stream_kernel_q8_0(int xt, int mode, int ms, bool norm, bool glu, bool short_items,
                                     bool wide);
moe_stream_fn moe_stream_kernel_q4_0(int xt, int mode, int ms, bool norm, bool glu, bool short_items,
                                     bool wide);
moe_stream_fn moe_stream_kernel_mxfp4(int xt, int mode, int ms, bool norm, bool glu, bool short_items,
                                     bool wide);

} // namespace qg
