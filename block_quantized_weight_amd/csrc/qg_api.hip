// qg_api.hip -- C ABI of libqgemv.so: argument validation, layout, launch
// plans, the packer kernels and the dequantization test aid.
#include <mutex>

#include "qg_chain.h"
#include "qg_mfma.h"
#include "qg_moe_stream.h"
#include "qg_fused.h"

namespace qg {
namespace {

// ---------------------------------------------------------------- dequant
// Test aid: one thread per (tile, step, lane) record writes its 32 weights.
__global__ void k_dequant(LayoutArgs a, const uint8_t *__restrict__ packed, float *__restrict__ w, int64_t k, int64_t nrec)
{
    for (int64_t rec = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; rec < nrec; rec += (int64_t)gridDim.x * blockDim.x) {
        int64_t row, blk, co, so;
        record_geom(a, rec, &row, &blk, &co, &so);
        if (row >= a.n || blk >= a.nb) continue;
        const uint4 c0 = *(const uint4 *)(packed + co);
        float *out = w + row * k + blk * QK;
        if (is_kq(a.fmt)) {
            // each weight the single rounding of its exact value
            const uint32_t sb = packed[so] | (packed[so + 1] << 8);
            const uint32_t swd = *(const uint32_t *)(packed + a.sboff + (row * a.nsb + (blk >> 3)) * 4);
            uint32_t c[4] = {c0.x, c0.y, c0.z, c0.w};
            if (a.fmt == QG_Q4_K) {
                const float D = f16_bits_to_f32(swd & 0xFFFF) * (float)(sb & 63);
                const float Mn = -(f16_bits_to_f32(swd >> 16) * (float)((sb >> 8) & 63));
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v[8];
                    q4_unpack8(c[i], v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) out[8 * i + e] = __builtin_fmaf(D, __builtin_fmaf(16.0f, v[e], 8.0f), Mn);
                }
            } else {
                const float d = f16_bits_to_f32(swd & 0xFFFF);
                const float Da = d * (float)(int8_t)(sb & 0xFF), Db = d * (float)(int8_t)(sb >> 8);
                const uint2 hh = *(const uint2 *)(packed + kq_high_off(a, rec));
                const uint32_t hw[2] = {hh.x, hh.y};
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int f = 2 * (q & 1) + e;
                        const uint32_t H = hw[q >> 1];
                        const uint32_t hp = f == 0 ? H << 4 : f == 1 ? H << 2 : f == 2 ? H : H >> 2;
                        uint32_t Q = ((c[q] >> (4 * e)) & 0x0F0F0F0Fu) | (hp & 0x30303030u);
                        const uint32_t sg = Q & 0x20202020u;
                        Q |= (sg << 1) | (sg << 2);
#pragma unroll
                        for (int b = 0; b < 4; ++b) out[8 * q + 4 * e + b] = (q < 2 ? Da : Db) * i8_at(Q, b);
                    }
            }
        } else if (a.fmt == QG_Q8_0) {
            const uint4 c1 = *(const uint4 *)(packed + co + 1024);
            uint32_t s = packed[so] | (packed[so + 1] << 8);
            float d = f16_bits_to_f32(s);
            uint32_t c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int p = 0; p < 4; ++p) out[4 * i + p] = d * i8_at(c[i], p);
        } else if (a.fmt == QG_Q4_0) {
            uint32_t s = packed[so] | (packed[so + 1] << 8);
            float d = q4_scale(s);
            uint32_t c[4] = {c0.x, c0.y, c0.z, c0.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v[8];
                q4_unpack8(c[i], v);
#pragma unroll
                for (int e = 0; e < 8; ++e) out[8 * i + e] = d * v[e];
            }
        } else if (a.fmt == QG_NVFP4) {
            const float ts = *(const float *)(packed + a.tsoff);
            const float s0 = e4m3_to_f32(packed[so]), s1 = e4m3_to_f32(packed[so + 1]);
            uint32_t c[4] = {c0.x, c0.y, c0.z, c0.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x2_t pr[4] = {fp4_pair_bf16<0>(c[i]), fp4_pair_bf16<1>(c[i]), fp4_pair_bf16<2>(c[i]),
                                  fp4_pair_bf16<3>(c[i])};
                const float sc = i < 2 ? s0 : s1;
                // E2M1 * E4M3 is exact in fp32 (at most 6 significant bits), so
                // each weight is the single rounding of its exact value
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t v = __builtin_bit_cast(uint32_t, pr[p]);
                    out[8 * i + 2 * p] = (sc * __builtin_bit_cast(float, v << 16)) * ts;
                    out[8 * i + 2 * p + 1] = (sc * __builtin_bit_cast(float, v & 0xFFFF0000u)) * ts;
                }
            }
        } else {
            float sc = e8m0_to_f32(packed[so]);
            uint32_t c[4] = {c0.x, c0.y, c0.z, c0.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16x2_t pr[4] = {fp4_pair_bf16<0>(c[i]), fp4_pair_bf16<1>(c[i]), fp4_pair_bf16<2>(c[i]),
                                  fp4_pair_bf16<3>(c[i])};
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t v = __builtin_bit_cast(uint32_t, pr[p]);
                    out[8 * i + 2 * p] = sc * __builtin_bit_cast(float, v << 16);
                    out[8 * i + 2 * p + 1] = sc * __builtin_bit_cast(float, v & 0xFFFF0000u);
                }
            }
        }
    }
}


__global__ void k_pack(LayoutArgs a, const uint8_t *__restrict__ canon, uint8_t *__restrict__ packed, int64_t nrec)
{
    const int64_t tid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x, nthr = (int64_t)gridDim.x * blockDim.x;
    for (int64_t o = a.end + tid; o < a.total; o += nthr) packed[o] = tail_byte(a, canon, o);
    for (int64_t r = tid; r < nrec; r += nthr)
        pack_record(a, canon, packed, r);
}

__global__ void k_unpack(LayoutArgs a, const uint8_t *__restrict__ packed, uint8_t *__restrict__ canon, int64_t nrec)
{
    const int64_t tid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (a.fmt == QG_NVFP4 && tid < 4) canon[a.cts + tid] = packed[a.tsoff + tid];      // the tensor scale
    if (is_kq(a.fmt)) {             // one thread per super-block (its eight records share scale bytes)
        for (int64_t u = tid; u < a.n * a.nsb; u += (int64_t)gridDim.x * blockDim.x)
            unpack_superblock_kq(a, packed, canon, u / a.nsb, u % a.nsb);
        return;
    }
    for (int64_t r = tid; r < nrec; r += (int64_t)gridDim.x * blockDim.x)
        unpack_record(a, packed, canon, r);
}

// ------------------------------------------------------- streaming ceiling
// Read-only probe of the device's achievable HBM read rate, the ceiling the
// GEMV kernels are measured against (decode is bound by memory bandwidth:
// imp README, "Known limitations").  Every 16-byte chunk of the buffer is
// loaded once, nontemporally, with the GEMV's access shape (a wavefront load
// instruction reads 1 KiB of consecutive bytes); each wave XOR-folds what it
// read into one word of the sink so no load can be dropped.
constexpr int STREAM_WGS = QG_STREAM_SINK / WAVES;   // one sink word per wave
constexpr int STREAM_U = 4;                          // loads in flight per lane

__global__ __launch_bounds__(TPB) void k_read_stream(const uint8_t *__restrict__ p, int64_t n16,
                                                     uint32_t *__restrict__ sink)
{
    uint32_t acc = 0;
    const int64_t nthr = (int64_t)gridDim.x * TPB;
    int64_t i = (int64_t)blockIdx.x * TPB + threadIdx.x;
    for (; i + (STREAM_U - 1) * nthr < n16; i += STREAM_U * nthr) {
        uint4 v[STREAM_U];
#pragma unroll
        for (int u = 0; u < STREAM_U; ++u) v[u] = ld_stream16(p + (i + u * nthr) * 16);
#pragma unroll
        for (int u = 0; u < STREAM_U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += nthr) {
        const uint4 v = ld_stream16(p + i * 16);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * WAVES + (threadIdx.x >> 6)] = acc;
}

// ----------------------------------------------------------------- router
// Top-k routing on the device, one wavefront per token.  Each logit becomes a
// 64-bit key: the float's bits in an order-preserving unsigned form (NaN taken
// as -inf), then the complement of the expert id, so the largest key is the
// largest logit with the lower id first among equals.  top_k rounds of a
// wave-wide key maximum (within rows of 16 lanes by DPP rotations, across
// the four rows by lane reads) pick the experts in order; the softmax of the
// selected logits is taken in fp32.
constexpr int ROUTER_MAX_EXPERTS = 1024;
constexpr int ROUTER_MAX_K = 64;

__device__ __forceinline__ uint32_t order_bits(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if (f != f) u = 0xFF800000u;                            // NaN ranks as -inf
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_float(uint32_t o)
{
    return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t max_key(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Maximum over the wave, returned to every lane.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k)
{
    // rows of 16 lanes: rotate by 8, 4, 2, 1 (row_ror:n is DPP control 0x120 + n)
#define QG_ROR(N)                                                                                          \
    {                                                                                                      \
        const uint32_t lo = __builtin_amdgcn_update_dpp(0, (uint32_t)k, 0x120 + (N), 0xF, 0xF, false);     \
        const uint32_t hi = __builtin_amdgcn_update_dpp(0, (uint32_t)(k >> 32), 0x120 + (N), 0xF, 0xF, false); \
        k = max_key(k, ((uint64_t)hi << 32) | lo);                                                         \
    }
    QG_ROR(8) QG_ROR(4) QG_ROR(2) QG_ROR(1)
#undef QG_ROR
    uint64_t r = 0;
#pragma unroll
    for (int row = 0; row < 4; ++row) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, 16 * row);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), 16 * row);
        r = max_key(r, ((uint64_t)hi << 32) | lo);
    }
    return r;
}

template <int NV>
__global__ __launch_bounds__(64) void k_router(const float *__restrict__ logits, int ne, int topk,
                                               int32_t *__restrict__ ids, float *__restrict__ w)
{
    const int lane = threadIdx.x;
    const int64_t t = blockIdx.x;
    const float *lt = logits + t * ne;
    uint64_t key[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = lane + 64 * i;
        const float f = lt[e < ne ? e : 0];
        key[i] = e < ne ? (((uint64_t)order_bits(f) << 32) | (uint32_t)~e) : 0;   // 0: not an expert
    }
    int my_id = 0;
    float my_v = 0.0f;
    for (int j = 0; j < topk; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < NV; ++i) best = max_key(best, key[i]);
        best = wave_max_key(best);
        const int e = (int)~(uint32_t)best;
        if (lane == j) {
            my_id = e;
            my_v = order_float((uint32_t)(best >> 32));
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (key[i] == best) key[i] = 0;                // taken (keys are unique)
    }
    const float top = __shfl(my_v, 0, 64);
    const float ex = lane < topk ? expf(my_v - top) : 0.0f;
    float sum = ex;
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane < topk) {
        ids[t * topk + lane] = my_id;
        w[t * topk + lane] = ex / sum;
    }
}

// ------------------------------------------------------------ host side
hipStream_t as_stream(void *s) { return (hipStream_t)s; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Packed weights start on a 256-byte boundary, so every tile, every 1 KiB
// wavefront load of codes and every expert (whose sizes are multiples of 256
// bytes) starts on a whole cache line: a 16-byte-aligned base would split each
// 1 KiB load over nine 128-byte lines instead of eight.
constexpr uintptr_t W_ALIGN = 256;

int check_shape(int fmt, int64_t n, int64_t k)
{
    if (!valid_fmt(fmt) || n <= 0 || k <= 0 || (k % QK) != 0) return QG_EINVAL;
    if (is_kq(fmt) && (k % 256) != 0) return QG_EINVAL;         // whole super-blocks
    if (n > 0x7FFFFFFF || k > 0x7FFFFFFF) return QG_EUNSUPPORTED;
    return QG_OK;
}

// Launch plan: split-K factor KS (waves per tile) and the activation window.
Plan make_plan(const Layout &lo, int M, bool dot, int maxslots_lds)
{
    Plan p{};
    Geom &g = p.g;
    g.n = (int32_t)lo.n;
    g.k = (int32_t)lo.k;
    g.nb = (int32_t)lo.nb;
    g.L = lo.L;
    g.lsh = lo.lsh;
    g.R = lo.R;
    g.S = (int32_t)lo.S;
    g.tiles = (int32_t)lo.tiles;
    g.ctb = lo.ctb;
    g.stb = lo.stb;
    g.soff = lo.soff;
    g.tsoff = lo.tsoff;
    g.hoff = lo.hoff;
    g.htb = lo.htb;
    g.sboff = lo.sboff;
    g.nsb = (int32_t)lo.nsb;
    // activation window: as many steps as fit XBUDGET (at least one)
    const size_t per_block = (size_t)maxslots_lds * x_quads(lo.fmt, dot) * 16;
    int64_t sw_max = (int64_t)(XBUDGET / per_block) / lo.L;
    if (sw_max < 1) sw_max = 1;
    // split-K factor: more waves per tile when tiles are few; never more than
    // the steps of a tile or of a window.  A single token over short rows (at
    // most 20 steps per lane) runs unsplit: the cross-wave reduction then
    // costs more than it saves (MI355X: -0.7 to -1.0 us per launch on the
    // 2560..6144-row decode matrices).  The 4-bit formats with bf16
    // activations (dot) keep the split from 16 steps per lane on (one token,
    // us unsplit / split: Q4_0 2560x9728
    // 8.14 / 7.63, 2048x8192 7.07 / 5.91, 4096x4096 7.05 / 5.80; NVFP4
    // 2560x9728 8.67 / 7.63; at 12 steps mixed, 3072x6144 Q4_0 6.39 / 6.51).
    // Co-batches keep the split, which also spreads their heavier per-step
    // arithmetic.
    int KS = 1;
    if (lo.tiles < 4096) KS = 2;
    if (lo.tiles < 2048) KS = 4;
    const bool four_bit = lo.fmt != QG_Q8_0 && !is_kq(lo.fmt);
    if (M == 1 && lo.S <= 20 && !(four_bit && dot && lo.S >= 16)) KS = 1;
    while (KS > 1 && (lo.S < KS || sw_max < KS)) KS >>= 1;
    g.KS = KS;
    g.ksh = ilog2(KS);
    g.tpi = WAVES / KS;
    g.ngroups = (int32_t)((lo.tiles + g.tpi - 1) / g.tpi);
    int64_t sw = sw_max / KS * KS;                         // a multiple of KS
    if (sw >= lo.S) sw = ((lo.S + KS - 1) / KS) * KS;
    g.SW = (int32_t)sw;
    g.nwin = (int32_t)((lo.S + sw - 1) / sw);
    g.wblk = (int32_t)(sw * lo.L);
    p.lds = lds_bytes(maxslots_lds, dot, lo.fmt, g.wblk);
    int grid = g.ngroups;
    if (grid > 65535) grid = 65535;
    p.grid = grid;
    p.threads = TPB;
    return p;
}

// Workgroup size of an unsplit plan (one tile per wave): as many waves as
// put about one workgroup on every compute unit, at most WAVES.  Measured on
// MI355X, one token, bf16 x, graph replay over rotated copies, us per launch
// at 4 / 3 / 2 / 1 waves per workgroup:
//   768 tiles (qkv 6144x2560)   Q8_0 6.97 / 6.75 / 7.49 / 7.13   Q4_0 6.11 / 5.88 / 6.98 / 5.94
//   640 tiles (down 2560x9728)  Q8_0 10.03 / 9.65 / 11.33 / 10.86  MXFP4 7.40 / 7.19 / 8.97 / 8.27
//   896 tiles (3584x2048)       Q8_0 5.00 / 5.79 / 5.13 / 5.02   Q4_0 4.19 / 5.05 / 4.68 / 4.32
//   512 tiles (2048x2048)       Q8_0 4.62 / 4.37 / 4.17 / 4.24   MXFP4 3.71 / 3.63 / 3.57 / 3.78
//   256 tiles (2048x1792)       Q8_0 5.12 / 4.95 / 4.69 / 4.50   MXFP4 4.27 / 3.97 / 3.92 / 3.75
// (NVFP4 alike.)  A grid of more workgroups than compute units loses where
// some units get two (896 tiles at three waves, 640-768 at two).
void fit_workgroups(Plan &p)
{
    Geom &g = p.g;
    if (g.KS != 1) return;
    int64_t w = (g.tiles + QG_CUS - 1) / QG_CUS;
    if (w >= WAVES) return;
    if (w < 1) w = 1;
    g.tpi = (int32_t)w;
    g.ngroups = (int32_t)((g.tiles + w - 1) / w);
    p.grid = g.ngroups > 65535 ? 65535 : g.ngroups;
    p.threads = (int)(64 * w);
}

inline bool uses_dot(int fmt, int xt) { return fmt != QG_Q8_0 && fmt != QG_Q4_K && xt == QG_BF16; }

// Co-batches of at least this many bf16 tokens may run on the matrix cores
// (dense_kind: unless the one-batch vector kernel applies).
inline int mfma_min_m(int) { return 2; }

// LDS per co-batch workgroup is kept within 80 KiB, so two fit on a CU; a
// co-batch grid of at most one workgroup per CU may use all 160 KiB, which
// fits longer activation windows (4 tokens, 8 lanes per row, split in 4: K up
// to 18432 in one window instead of 8192).
constexpr int MFMA_WG_LDS = 80 * 1024;
constexpr int MFMA_WG_LDS_ONE = 160 * 1024;

struct MPlan {
    MGeom g;
    size_t lds;
    int grid;
    int nw;                      // waves per workgroup
};

// The matrix-core kernel serves bf16 activations, layouts of 1 to 8 lanes per
// row, and tiles whose per-lane offsets fit in 32 bits.
bool mfma_fits(const Layout &lo, int xt, int64_t m)
{
    if (lo.fmt == QG_NVFP4 || is_kq(lo.fmt) || xt != QG_BF16 || m < mfma_min_m(lo.fmt) || lo.L > MFMA_MAX_L)
        return false;
    const int64_t tpw = lo.L >= 8 ? lo.L / 4 : 1;
    return lo.ctb * tpw < ((int64_t)1 << 31) && lo.stb * tpw < ((int64_t)1 << 31);
}

// m: tokens the LDS holds (one pass); TG: token groups of 16 per pass;
// passes > 0 (the many-token product): the split-K factor is the smallest
// that still gives more than one workgroup per CU (>= 300 over all passes),
// since each workgroup stages the activations once for its WAVES / KS units
// (more units per workgroup means fewer re-reads of the activations).
// Measured on MI355X, Q4_0 at 64 tokens: 6144x4096 28.6 us unsplit (384
// workgroups) against 35.6 split in two; 4096x12288 52.0 us split in two
// against 59.0 unsplit (256 workgroups).
MPlan make_mplan(const Layout &lo, int m, int passes = 0, int TG = 1, int waves = WAVES)
{
    MPlan p{};
    p.nw = waves;
    MGeom &g = p.g;
    g.n = (int32_t)lo.n;
    g.k = (int32_t)lo.k;
    g.nb = (int32_t)lo.nb;
    g.L = lo.L;
    g.R = lo.R;
    g.S = (int32_t)lo.S;
    g.tiles = (int32_t)lo.tiles;
    g.ctb = lo.ctb;
    g.stb = lo.stb;
    g.soff = lo.soff;
    g.m = m;
    const int64_t tpw = lo.L >= 8 ? lo.L / 4 : 1;
    g.units = (int32_t)((lo.tiles + tpw - 1) / tpw);
    const size_t per_block = (size_t)m * 64;
    int64_t budget = MFMA_WG_LDS;
    // activation window: as many steps as fit beside the fixed areas (at least one)
    auto sw_for = [&](int ks) {
        const int64_t xbudget = budget - (int64_t)mfma_lds_bytes(lo.fmt, m, 0, lo.L, ks, TG, waves);
        const int64_t v = (xbudget / (int64_t)per_block) / lo.L;
        return v < 1 ? (int64_t)1 : v;
    };
    auto groups = [&](int ks) { return (g.units + waves / ks - 1) / (waves / ks); };
    int KS = 1;
    if (passes > 0) {
        while (KS < WAVES && groups(KS) * passes < 300) KS <<= 1;
    } else {
        if (g.units < 4096) KS = 2;
        if (g.units < 2048) KS = 4;
        // Past 4 tokens each workgroup stages twice the activations: two
        // units per workgroup halve that traffic once the units fill the
        // CUs.  Measured on MI355X at 8 tokens, split 2 / 4: Q4_0 6144x4096
        // 10.35 / 11.00 us, 24576x4096 20.28 / 21.14, Q8_0 11.10 / 15.82 and
        // 27.80 / 31.68; 4096x12288 (256 units) 27.99 / 22.25 keeps 4.
        if (m > 4 && g.units >= 384 && KS > 2) KS = 2;
        // eight-wave workgroups: a unit's steps over all eight waves where the
        // units fit the compute units once, else two units of four waves each
        if (waves == MFMA_WIDE_WAVES) KS = g.units <= QG_CUS ? 8 : 4;
        if (groups(KS) <= QG_CUS) budget = MFMA_WG_LDS_ONE;   // fewer KS only means fewer groups
    }
    while (KS > 1 && (lo.S < KS || sw_for(KS) < KS)) KS >>= 1;
    const int64_t sw_max = sw_for(KS);
    g.KS = KS;
    g.ksh = ilog2(KS);
    g.upi = waves / KS;
    g.ngroups = (int32_t)((g.units + g.upi - 1) / g.upi);
    int64_t sw = sw_max / KS * KS;
    if (sw >= lo.S) sw = ((lo.S + KS - 1) / KS) * KS;
    // windows of equal length (never longer than the largest that fits): a
    // short last window leaves its staging and barriers exposed (MI355X, Q4_0
    // 4096x12288 at 8 tokens: windows of 36 + 12 steps 21.2 us, 24 + 24 18.7)
    const int64_t nw = (lo.S + sw - 1) / sw;
    sw = ((lo.S + nw - 1) / nw + KS - 1) / KS * KS;
    g.SW = (int32_t)sw;
    g.nwin = (int32_t)((lo.S + sw - 1) / sw);
    g.wblk = (int32_t)(sw * lo.L);
    p.lds = mfma_lds_bytes(lo.fmt, m, g.wblk, lo.L, KS, TG, waves);
    p.grid = g.ngroups > 65535 ? 65535 : g.ngroups;
    return p;
}

// Steps in flight of the one-batch kernel for this plan, or 0 where it does
// not apply: few tokens (one_batch_u), one activation window held by the
// workgroup's threads, at most ONE_MAX_U steps per wave, one tile group per
// workgroup, and every workgroup resident at once (its registers allow
// one_waves per compute unit, its LDS may allow fewer).  A grid that needs
// two rounds loses to the batched pass (MI355X, Q4_0 24576x4096 at two
// tokens, 768 workgroups of 16 steps per wave: 18.9 us batched, 21.2 one
// batch at 2 per compute unit).  One exception, measured: Q8_0 with bf16
// activations at one token takes up to 1.25x the resident grid (19456x2560,
// 608 workgroups of 10 steps per wave at 2 per unit: 13.56 -> 13.15 us; 36
// decode layers 1284 -> 1269 us; bitwise the same results).
int one_batch(int fmt, int xt, const Plan &p, int64_t m)
{
    const Geom &g = p.g;
    if (g.nwin != 1 || m * g.wblk > (int64_t)ONE_XR * p.threads || g.ngroups != p.grid) return 0;
    const int u = one_batch_u(fmt, (int)m, (g.S + g.KS - 1) / g.KS);
    if (!u) return 0;
    // workgroups per compute unit: by registers (one_waves per SIMD) and by LDS
    int per_cu = one_waves(fmt, xt == QG_BF16, u) * WAVES / (p.threads / 64);
    const int lds_cu = p.lds > 0 ? (int)((160 * 1024) / p.lds) : per_cu;
    if (lds_cu < per_cu) per_cu = lds_cu;
    const int64_t resident = (int64_t)per_cu * QG_CUS;
    if (fmt == QG_Q8_0 && xt == QG_BF16 && m == 1) return 4 * (int64_t)p.grid <= 5 * resident ? u : 0;
    return p.grid <= resident ? u : 0;
}

// The kernel family of a dense call.  bf16 co-batches run on the matrix
// cores (mfma_fits) unless the one-batch vector kernel applies (4-bit formats,
// 2 or 3 tokens, grids resident at once), which is faster there; everything
// else on the vector kernel, one-batch where it applies.  p receives the
// vector plan, u its steps in flight (0: the batched pass).  Measured on
// MI355X, Q4_0 vector / matrix cores (us): 2 tokens 6144x4096 (one-batch)
// 7.62 / 8.74, 4096x12288 (one-batch) 11.87 / 12.09, 24576x4096 (batched)
// 19.68 / 17.44; 3 tokens 6144x4096 (one-batch) 8.59 / 9.11, 24576x4096
// (batched) 21.63 / 16.50, 4096x12288 (batched) 17.64 / 12.88.
int dense_kind(int fmt, const Layout &lo, int xt, int64_t m, Plan &p, int &u)
{
    p = make_plan(lo, (int)m, uses_dot(fmt, xt), (int)m);
    fit_workgroups(p);
    u = one_batch(fmt, xt, p, m);
    if (!u && mfma_fits(lo, xt, m)) return QG_PATH_MFMA;
    return u ? QG_PATH_VALU_ONE : QG_PATH_VALU;
}

int launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? QG_OK : QG_EHIP;
}

int dense(int fmt, const void *w, int64_t n, int64_t k, const void *x, int xt, int64_t m, float *y, void *stream)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!w || !x || !y) return QG_EINVAL;
    if (xt != QG_F32 && xt != QG_BF16) return QG_EINVAL;
    if (m < 1 || m > QG_MAX_M) return QG_EINVAL;
    if (!aligned(w, W_ALIGN) || !aligned(x, 16) || !aligned(y, 4)) return QG_EALIGN;
    const Layout lo = make_layout(fmt, n, k);
    Plan p;
    int u = 0;
    if (dense_kind(fmt, lo, xt, m, p, u) == QG_PATH_MFMA) {
        const int nw = lo.L == 8 && m >= 4 ? MFMA_WIDE_WAVES : WAVES;
        MPlan mp = make_mplan(lo, (int)m, 0, 1, nw);
        mp.g.w = (const uint8_t *)w;
        mfma_fn f = fmt == QG_Q8_0 ? mfma_kernel_q8_0(lo.L, 1, nw)
                    : fmt == QG_Q4_0 ? mfma_kernel_q4_0(lo.L, 1, nw) : mfma_kernel_mxfp4(lo.L, 1, nw);
        void *args[] = {(void *)&mp.g, (void *)&x, (void *)&y};
        if (allow_lds((const void *)f, mp.lds) != hipSuccess) return QG_EHIP;
        hipError_t e = hipLaunchKernel((const void *)f, dim3(mp.grid), dim3(64 * mp.nw), args, mp.lds,
                                       as_stream(stream));
        return e == hipSuccess ? launch_status() : QG_EHIP;
    }
    p.g.w = (const uint8_t *)w;
    dense_fn f = u ? (fmt == QG_Q8_0 ? dense_one_kernel_q8_0(xt, (int)m, u)
                      : fmt == QG_Q4_0 ? dense_one_kernel_q4_0(xt, (int)m, u)
                      : fmt == QG_MXFP4 ? dense_one_kernel_mxfp4(xt, (int)m, u)
                      : fmt == QG_NVFP4 ? dense_one_kernel_nvfp4(xt, (int)m, u) : dense_one_kernel_kq(fmt, xt, (int)m, u))
                   : (fmt == QG_Q8_0 ? dense_kernel_q8_0(xt, (int)m)
                      : fmt == QG_Q4_0 ? dense_kernel_q4_0(xt, (int)m)
                      : fmt == QG_MXFP4 ? dense_kernel_mxfp4(xt, (int)m)
                      : fmt == QG_NVFP4 ? dense_kernel_nvfp4(xt, (int)m) : dense_kernel_kq(fmt, xt, (int)m));
    void *args[] = {(void *)&p.g, (void *)&x, (void *)&y};
    if (allow_lds((const void *)f, p.lds) != hipSuccess) return QG_EHIP;
    hipError_t e = hipLaunchKernel((const void *)f, dim3(p.grid), dim3(p.threads), args, p.lds, as_stream(stream));
    return e == hipSuccess ? launch_status() : QG_EHIP;
}

int64_t nrecords(const Layout &lo) { return lo.tiles * lo.S * 64; }

int grid_for(int64_t items, int block)
{
    int64_t g = (items + block - 1) / block;
    if (g > 65535 * 8) g = 65535 * 8;
    if (g < 1) g = 1;
    return (int)g;
}

// Chain plan of one link: the layout with one activation window over the
// whole K, and the most tiles any of the P workgroups owns.  The LDS the link
// needs (staged x, partial sums, finished rows) is returned in *xs, *part and
// *out bytes.
int chain_link_plan(int fmt, int xt, int m, int P, const qg_chain_link_t &in, ChainLink *out, size_t *xs,
                    size_t *part, size_t *outb)
{
    int st = check_shape(fmt, in.n, in.k);
    if (st) return st;
    if (!in.w_packed || !in.x || !in.y) return QG_EINVAL;
    if (!aligned(in.w_packed, W_ALIGN) || !aligned(in.x, 16) || !aligned(in.y, 4)) return QG_EALIGN;
    const Layout lo = make_layout(fmt, in.n, in.k);
    const bool dot = uses_dot(fmt, xt);
    Geom &g = out->g;
    memset(out, 0, sizeof(*out));
    g.w = (const uint8_t *)in.w_packed;
    g.n = (int32_t)lo.n;
    g.k = (int32_t)lo.k;
    g.nb = (int32_t)lo.nb;
    g.L = lo.L;
    g.lsh = lo.lsh;
    g.R = lo.R;
    g.S = (int32_t)lo.S;
    g.tiles = (int32_t)lo.tiles;
    g.ctb = lo.ctb;
    g.stb = lo.stb;
    g.soff = lo.soff;
    g.KS = 1;
    g.ksh = 0;
    g.tpi = 1;
    g.ngroups = 0;
    g.SW = (int32_t)lo.S;
    g.nwin = 1;
    g.wblk = (int32_t)(lo.S * lo.L);
    // items of a workgroup are counted in int: tiles * S per workgroup
    const int64_t tmax = (lo.tiles + P - 1) / P;
    if (tmax * lo.S > 0x3FFFFFFF) return QG_EUNSUPPORTED;
    out->tmax = (int32_t)tmax;
    out->x = in.x;
    out->y = in.y;
    *xs = chain_xs_bytes(m, dot, g.wblk);
    *part = chain_part_bytes(m, (int)tmax);
    *outb = chain_out_bytes(m, (int)tmax, lo.R);
    return QG_OK;
}

const void *chain_kernel(int fmt, int xt, int m)
{
    return fmt == QG_Q8_0 ? chain_kernel_q8_0(xt, m) : fmt == QG_Q4_0 ? chain_kernel_q4_0(xt, m)
                                                                     : chain_kernel_mxfp4(xt, m);
}

// Launches a built plan whose device copy is at plan_device.
int chain_launch(const ChainHdr *h, const void *plan_device, hipStream_t stream)
{
    const ChainLink *links = (const ChainLink *)((const uint8_t *)plan_device + sizeof(ChainHdr) + 16);
    int nlinks = h->count;
    const void *fn = chain_kernel(h->fmt, h->xt, h->m);
    if (allow_lds(fn, (size_t)h->lds) != hipSuccess) return QG_EHIP;
    int part_off = (int)h->part_off, out_off = (int)h->out_off;
    void *args[] = {(void *)&links, (void *)&nlinks, (void *)&part_off, (void *)&out_off};
    hipError_t e = hipLaunchCooperativeKernel(fn, dim3(h->grid), dim3(CTPB), args, (unsigned)h->lds, stream);
    return e == hipSuccess ? launch_status() : QG_EHIP;
}

// Plan buffer of qgemv_chain_noalloc: one per device, held until the process
// ends.  Host code never uses this name as an address: the device address of
// each device's copy is looked up once (scratch_on_device) and passed on.
static __device__ __align__(256) uint8_t scratch[QG_CHAIN_STATIC_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_ptr[SCRATCH_MAX_DEVICES];

// Device address of the current device's scratch copy, looked up on the
// first call on that device (the device is current), or QG_* on failure.
int scratch_on_device(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QG_EHIP;
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return QG_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QG_EHIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return QG_OK;
}

} // namespace
} // namespace qg

using namespace qg;


// ================================================================ C ABI
extern "C" {

const char *qg_status_str(int status)
{
    switch (status) {
    case QG_OK: return "ok";
    case QG_EINVAL: return "invalid argument";
    case QG_EUNSUPPORTED: return "unsupported shape or size";
    case QG_EALIGN: return "misaligned device pointer";
    case QG_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int64_t qg_packed_bytes(int fmt, int64_t n, int64_t k)
{
    if (check_shape(fmt, n, k)) return -1;
    return make_layout(fmt, n, k).total;
}

int qg_layout(int fmt, int64_t n, int64_t k, qg_layout_t *out)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!out) return QG_EINVAL;
    const Layout lo = make_layout(fmt, n, k);
    memset(out, 0, sizeof(*out));
    out->fmt = fmt;
    out->lanes_per_row = lo.L;
    out->rows_per_tile = lo.R;
    out->parts_per_step = lo.P;
    out->scale_bytes = lo.sb;
    out->n = n;
    out->k = k;
    out->steps = lo.S;
    out->tiles = lo.tiles;
    out->code_tile_bytes = lo.ctb;
    out->scale_tile_bytes = lo.stb;
    out->scale_offset = lo.soff;
    out->packed_bytes = lo.total;
    out->tensor_scale_offset = lo.tsoff;
    out->high_offset = lo.hoff;
    out->superblock_offset = lo.sboff;
    return QG_OK;
}

int qg_pack_host(int fmt, const void *canon, int64_t n, int64_t k, void *packed)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!canon || !packed) return QG_EINVAL;
    const Layout lo = make_layout(fmt, n, k);
    const LayoutArgs a = layout_args(lo);
    const int64_t nrec = nrecords(lo);
    for (int64_t o = a.end; o < a.total; ++o) ((uint8_t *)packed)[o] = tail_byte(a, (const uint8_t *)canon, o);
    for (int64_t r = 0; r < nrec; ++r) pack_record(a, (const uint8_t *)canon, (uint8_t *)packed, r);
    return QG_OK;
}

int qg_unpack_host(int fmt, const void *packed, int64_t n, int64_t k, void *canon)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!canon || !packed) return QG_EINVAL;
    const Layout lo = make_layout(fmt, n, k);
    const LayoutArgs a = layout_args(lo);
    const int64_t nrec = nrecords(lo);
    if (fmt == QG_NVFP4) memcpy((uint8_t *)canon + a.cts, (const uint8_t *)packed + a.tsoff, 4);
    if (is_kq(fmt)) {
        for (int64_t r = 0; r < n; ++r)
            for (int64_t sbi = 0; sbi < a.nsb; ++sbi)
                unpack_superblock_kq(a, (const uint8_t *)packed, (uint8_t *)canon, r, sbi);
        return QG_OK;
    }
    for (int64_t r = 0; r < nrec; ++r) unpack_record(a, (const uint8_t *)packed, (uint8_t *)canon, r);
    return QG_OK;
}

int qg_pack(int fmt, const void *canon, int64_t n, int64_t k, void *packed, void *stream)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!canon || !packed) return QG_EINVAL;
    if (!aligned(packed, W_ALIGN)) return QG_EALIGN;
    const Layout lo = make_layout(fmt, n, k);
    const int64_t nrec = nrecords(lo);
    hipLaunchKernelGGL(k_pack, dim3(grid_for(nrec, 256)), dim3(256), 0, as_stream(stream), layout_args(lo),
                       (const uint8_t *)canon, (uint8_t *)packed, nrec);
    return launch_status();
}

int qg_unpack(int fmt, const void *packed, int64_t n, int64_t k, void *canon, void *stream)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!canon || !packed) return QG_EINVAL;
    if (!aligned(packed, W_ALIGN)) return QG_EALIGN;
    const Layout lo = make_layout(fmt, n, k);
    const int64_t nrec = nrecords(lo);
    hipLaunchKernelGGL(k_unpack, dim3(grid_for(nrec, 256)), dim3(256), 0, as_stream(stream), layout_args(lo),
                       (const uint8_t *)packed, (uint8_t *)canon, nrec);
    return launch_status();
}

int qg_dequant_f32(int fmt, const void *w_packed, int64_t n, int64_t k, float *w, void *stream)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!w_packed || !w) return QG_EINVAL;
    if (!aligned(w_packed, W_ALIGN) || !aligned(w, 4)) return QG_EALIGN;
    const Layout lo = make_layout(fmt, n, k);
    const int64_t nrec = nrecords(lo);
    hipLaunchKernelGGL(k_dequant, dim3(grid_for(nrec, 256)), dim3(256), 0, as_stream(stream), layout_args(lo),
                       (const uint8_t *)w_packed, w, k, nrec);
    return launch_status();
}

int qg_read_stream(const void *buf, int64_t bytes, uint32_t *sink, void *stream)
{
    if (!buf || !sink || bytes <= 0 || (bytes % 16) != 0) return QG_EINVAL;
    if (!aligned(buf, W_ALIGN) || !aligned(sink, 4)) return QG_EALIGN;
    hipLaunchKernelGGL(k_read_stream, dim3(STREAM_WGS), dim3(TPB), 0, as_stream(stream), (const uint8_t *)buf,
                       bytes / 16, sink);
    return launch_status();
}

int qg_dense_path(int fmt, int64_t n, int64_t k, int xt, int64_t m)
{
    int st = check_shape(fmt, n, k);
    if (st) return -st;
    if (xt != QG_F32 && xt != QG_BF16) return -QG_EINVAL;
    if (m < 1 || m > QG_MAX_M) return -QG_EINVAL;
    Plan p;
    int u = 0;
    return dense_kind(fmt, make_layout(fmt, n, k), xt, m, p, u);
}

int qgemv_q8_0(const void *w, int64_t n, int64_t k, const void *x, int xt, int64_t m, float *y, void *stream)
{
    return dense(QG_Q8_0, w, n, k, x, xt, m, y, stream);
}

int qgemv_q4_0(const void *w, int64_t n, int64_t k, const void *x, int xt, int64_t m, float *y, void *stream)
{
    return dense(QG_Q4_0, w, n, k, x, xt, m, y, stream);
}

int qgemv_mxfp4(const void *w, int64_t n, int64_t k, const void *x, int xt, int64_t m, float *y, void *stream)
{
    return dense(QG_MXFP4, w, n, k, x, xt, m, y, stream);
}

int qgemv_nvfp4(const void *w, int64_t n, int64_t k, const void *x, int xt, int64_t m, float *y, void *stream)
{
    return dense(QG_NVFP4, w, n, k, x, xt, m, y, stream);
}

int qgemv_q4_k(const void *w, int64_t n, int64_t k, const void *x, int xt, int64_t m, float *y, void *stream)
{
    return dense(QG_Q4_K, w, n, k, x, xt, m, y, stream);
}

int qgemv_q6_k(const void *w, int64_t n, int64_t k, const void *x, int xt, int64_t m, float *y, void *stream)
{
    return dense(QG_Q6_K, w, n, k, x, xt, m, y, stream);
}

int qg_requant_q8_0_nvfp4(const void *canon_q8_0, int64_t n, int64_t k, void *nvfp4_packed, void *stream)
{
    int st = check_shape(QG_NVFP4, n, k);
    if (st) return st;
    if (!canon_q8_0 || !nvfp4_packed) return QG_EINVAL;
    if (!aligned(nvfp4_packed, W_ALIGN)) return QG_EALIGN;
    const Layout lo = make_layout(QG_NVFP4, n, k);
    return launch_requant_nvfp4(lo, (const uint8_t *)canon_q8_0, (uint8_t *)nvfp4_packed, as_stream(stream)) ==
                   hipSuccess
               ? QG_OK
               : QG_EHIP;
}

// Token groups on the matrix cores: bf16 activations, layouts of at most
// GEMM_MAX_L lanes per row, 32-bit per-lane tile offsets.
static bool gemm_fits(const Layout &lo, int xt)
{
    if (xt != QG_BF16 || lo.L > GEMM_MAX_L) return false;
    const int64_t tpw = lo.L >= 8 ? lo.L / 4 : 1;
    return lo.ctb * tpw < ((int64_t)1 << 31) && lo.stb * tpw < ((int64_t)1 << 31);
}

int qg_gemm_path(int fmt, int64_t n, int64_t k, int xt, int64_t m)
{
    int st = check_shape(fmt, n, k);
    if (st) return -st;
    if (xt != QG_F32 && xt != QG_BF16) return -QG_EINVAL;
    if (m < 1 || m > QG_MAX_GEMM_M) return -QG_EINVAL;
    if (is_kq(fmt)) return -QG_EUNSUPPORTED;
    return gemm_fits(make_layout(fmt, n, k), xt) ? QG_PATH_MFMA : QG_PATH_VALU;
}

int qgemm(int fmt, const void *w, int64_t n, int64_t k, const void *x, int xt, int64_t m, float *y, void *stream)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!w || !x || !y) return QG_EINVAL;
    if (xt != QG_F32 && xt != QG_BF16) return QG_EINVAL;
    if (m < 1 || m > QG_MAX_GEMM_M) return QG_EINVAL;
    if (is_kq(fmt)) return QG_EUNSUPPORTED;
    if (!aligned(w, W_ALIGN) || !aligned(x, 16) || !aligned(y, 4)) return QG_EALIGN;
    const Layout lo = make_layout(fmt, n, k);
    if (gemm_fits(lo, xt)) {
        // one launch: grid.y = passes of TG token groups of 16, LDS planned for one pass
        const int TG = gemm_groups(lo.L, m);
        const int per_pass = 16 * TG;
        const int passes = (int)((m + per_pass - 1) / per_pass);
        MPlan p = make_mplan(lo, (int)(m < per_pass ? m : per_pass), passes, TG);
        p.g.m = (int32_t)m;
        p.g.w = (const uint8_t *)w;
        mfma_fn f = fmt == QG_Q8_0 ? mfma_kernel_q8_0(lo.L, TG)
                    : fmt == QG_Q4_0 ? mfma_kernel_q4_0(lo.L, TG) : mfma_kernel_mxfp4(lo.L, TG);
        void *args[] = {(void *)&p.g, (void *)&x, (void *)&y};
        if (allow_lds((const void *)f, p.lds) != hipSuccess) return QG_EHIP;
        hipError_t e = hipLaunchKernel((const void *)f, dim3(p.grid, (unsigned)passes), dim3(TPB), args, p.lds,
                                       as_stream(stream));
        return e == hipSuccess ? launch_status() : QG_EHIP;
    }
    // otherwise the dense product, QG_MAX_M tokens per launch
    const size_t xsz = xt == QG_BF16 ? 2 : 4;
    for (int64_t t0 = 0; t0 < m; t0 += QG_MAX_M) {
        const int64_t mt = m - t0 < QG_MAX_M ? m - t0 : QG_MAX_M;
        st = dense(fmt, w, n, k, (const uint8_t *)x + t0 * k * xsz, xt, mt, y + t0 * n, stream);
        if (st) return st;
    }
    return QG_OK;
}

static bool overlaps(const void *a, size_t abytes, const void *b, size_t bbytes)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

int qgemv_fused(int fmt, const void *w, int64_t n, int64_t k, const void *x, int xt, int64_t m,
                const float *norm_weight, float norm_eps, int act, const float *residual,
                void *y, int yt, void *stream)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!w || !x || !y) return QG_EINVAL;
    if (xt != QG_F32 && xt != QG_BF16) return QG_EINVAL;
    if (yt != QG_F32 && yt != QG_BF16) return QG_EINVAL;
    if (act != QG_ACT_NONE && act != QG_ACT_SWIGLU) return QG_EINVAL;
    if (m < 1 || m > QG_MAX_M) return QG_EINVAL;
    if (norm_weight && !(norm_eps >= 0.0f && norm_eps <= 3.4e38f)) return QG_EINVAL;    // rejects NaN too
    if (act == QG_ACT_SWIGLU && (n % 2) != 0) return QG_EINVAL;
    if (is_kq(fmt)) return QG_EUNSUPPORTED;
    if (!aligned(w, W_ALIGN) || !aligned(x, 16) || !aligned(y, yt == QG_F32 ? 4 : 2)) return QG_EALIGN;
    if ((norm_weight && !aligned(norm_weight, 16)) || (residual && !aligned(residual, 4))) return QG_EALIGN;
    const int64_t n_out = act == QG_ACT_SWIGLU ? n / 2 : n;
    if (residual && !(yt == QG_F32 && (const void *)residual == y) &&
        overlaps(residual, (size_t)(m * n_out * 4), y, (size_t)(m * n_out * (yt == QG_F32 ? 4 : 2))))
        return QG_EINVAL;
    const Layout lo = make_layout(fmt, n, k);
    if (act == QG_ACT_SWIGLU && (n_out % lo.R) != 0) return QG_EUNSUPPORTED;
    const bool norm = norm_weight != nullptr;
    const bool dot = !norm && uses_dot(fmt, xt);
    Plan p = make_plan(lo, (int)m, dot, (int)m);
    p.g.w = (const uint8_t *)w;
    EpiArgs e{};
    e.gamma = norm_weight;
    e.eps = norm_eps;
    e.residual = residual;
    e.y = y;
    e.n_out = (int32_t)n_out;
    e.half_tiles = act == QG_ACT_SWIGLU ? (int32_t)(n_out / lo.R) : 0;
    e.y_bf16 = yt == QG_BF16;
    // the gate: 0 none; 1 gate and up halves in one wave (the plain grid: the
    // work units are as many as the tiles); 2 for one-row tiles (64 lanes per
    // row), GLU_WAVES-wave workgroups whose halves hold gate and up tiles
    const int glu = e.half_tiles == 0 ? 0 : lo.L <= 32 ? 1 : 2;
    int block = TPB;
    if (glu == 2) {
        p.g.tpi = GLU_WAVES / p.g.KS;
        const int pp = p.g.tpi / 2;
        p.g.ngroups = (e.half_tiles + pp - 1) / pp;
        p.grid = p.g.ngroups > 65535 ? 65535 : p.g.ngroups;
        p.lds += (size_t)(GLU_WAVES - WAVES) * m * 64 * 4;     // split-K partials of the extra waves
        block = 64 * GLU_WAVES;
    }
    // without normalisation or gate, the plain product's one-batch form where it applies
    const int u = !norm && glu == 0 ? one_batch(fmt, xt, p, m) : 0;
    dense_ep_fn f = u ? (fmt == QG_Q8_0 ? dense_one_ep_kernel_q8_0(xt, (int)m, u)
                         : fmt == QG_Q4_0 ? dense_one_ep_kernel_q4_0(xt, (int)m, u)
                         : fmt == QG_MXFP4 ? dense_one_ep_kernel_mxfp4(xt, (int)m, u)
                                           : dense_one_ep_kernel_nvfp4(xt, (int)m, u))
                      : fmt == QG_Q8_0 ? dense_ep_kernel_q8_0(xt, (int)m, norm, glu)
                      : fmt == QG_Q4_0 ? dense_ep_kernel_q4_0(xt, (int)m, norm, glu)
                      : fmt == QG_MXFP4 ? dense_ep_kernel_mxfp4(xt, (int)m, norm, glu)
                                        : dense_ep_kernel_nvfp4(xt, (int)m, norm, glu);
    void *args[] = {(void *)&p.g, (void *)&e, (void *)&x};
    if (allow_lds((const void *)f, p.lds) != hipSuccess) return QG_EHIP;
    hipError_t err = hipLaunchKernel((const void *)f, dim3(p.grid), dim3(block), args, p.lds, as_stream(stream));
    return err == hipSuccess ? launch_status() : QG_EHIP;
}

// The expert product, plain or fused (norm, gate, residual or a bf16 output
// requested): fused calls run only on the streaming kernel.
static int moe_impl(int fmt, const void *w_experts, int64_t n_experts, int64_t n, int64_t k,
                    const int32_t *topk_ids, const float *topk_w, int64_t m, int64_t top_k, const void *x, int xt,
                    int mode, const float *norm_weight, float norm_eps, int act, const float *residual, void *y, int yt,
                    void *stream)
{
    int st = check_shape(fmt, n, k);
    if (st) return st;
    if (!w_experts || !topk_ids || !x || !y) return QG_EINVAL;
    if (fmt == QG_NVFP4) return QG_EUNSUPPORTED;   // per-expert tensor scales: not served by the expert kernels
    if (is_kq(fmt)) return QG_EUNSUPPORTED;        // super-block formats: the dense product only
    if (xt != QG_F32 && xt != QG_BF16) return QG_EINVAL;
    if (yt != QG_F32 && yt != QG_BF16) return QG_EINVAL;
    if (mode != QG_MOE_GATE_UP && mode != QG_MOE_DOWN_COMBINE) return QG_EINVAL;
    if (mode == QG_MOE_DOWN_COMBINE && !topk_w) return QG_EINVAL;
    if (act != QG_ACT_NONE && act != QG_ACT_SWIGLU) return QG_EINVAL;
    if (mode == QG_MOE_GATE_UP && residual) return QG_EINVAL;
    if (mode == QG_MOE_DOWN_COMBINE && (norm_weight || act != QG_ACT_NONE)) return QG_EINVAL;
    if (norm_weight && !(norm_eps >= 0.0f && norm_eps <= 3.4e38f)) return QG_EINVAL;
    if (act == QG_ACT_SWIGLU && (n % 2) != 0) return QG_EINVAL;
    if (m < 1 || m > QG_MAX_M || n_experts < 1 || top_k < 1 || top_k > n_experts) return QG_EINVAL;
    if (m * top_k > 64 || n_experts > 65536) return QG_EUNSUPPORTED;
    if (!aligned(w_experts, W_ALIGN) || !aligned(x, 16) || !aligned(y, yt == QG_F32 ? 4 : 2) || !aligned(topk_ids, 4) ||
        (topk_w && !aligned(topk_w, 4)) || (norm_weight && !aligned(norm_weight, 16)) ||
        (residual && !aligned(residual, 4)))
        return QG_EALIGN;
    const int64_t n_out = act == QG_ACT_SWIGLU ? n / 2 : n;
    const int64_t ny = mode == QG_MOE_GATE_UP ? m * top_k * n_out : m * n_out;
    if (residual && !(yt == QG_F32 && (const void *)residual == y) &&
        overlaps(residual, (size_t)(ny * 4), y, (size_t)(ny * (yt == QG_F32 ? 4 : 2))))
        return QG_EINVAL;
    const bool fused = norm_weight || act != QG_ACT_NONE || residual || yt != QG_F32;
    const Layout lo = make_layout(fmt, n, k);
    if (act == QG_ACT_SWIGLU && (n_out % lo.R) != 0) return QG_EUNSUPPORTED;
    const bool norm = norm_weight != nullptr, glu = act == QG_ACT_SWIGLU;
    const bool dot = uses_dot(fmt, xt);
    MoeArgs a;
    a.experts = (const uint8_t *)w_experts;
    a.expert_bytes = lo.total;
    a.ids = topk_ids;
    a.gw = topk_w;
    a.n_experts = (int32_t)n_experts;
    a.m = (int32_t)m;
    a.top_k = (int32_t)top_k;
    a.isplit = 1;
    EpiArgs e{};
    e.gamma = norm_weight;
    e.eps = norm_eps;
    e.residual = residual;
    e.y = y;
    e.n_out = (int32_t)n_out;
    e.half_tiles = glu ? (int32_t)(n_out / lo.R) : 0;
    e.y_bf16 = yt == QG_BF16;
    hipStream_t s = as_stream(stream);
    {
        // streaming kernel: every activation row of the call staged at once
        // (normalised rows in fp32)
        const int nrows = (int)(mode == QG_MOE_GATE_UP ? m : m * top_k);
        // down-combine of several tokens over few tiles: workgroups of
        // WIDE_WAVES waves, all splitting one tile's items (twice the waves of
        // the four-wave form, two per SIMD where the tiles fill the CUs once)
        const bool wide = mode == QG_MOE_DOWN_COMBINE && m > 1 && lo.tiles <= QG_CUS &&
                          moe_stream_lds(fmt, dot, nrows, (int)(lo.S * lo.L), mode, 0, 0, WIDE_WAVES) <= MOE_STREAM_LDS;
        const int nw = wide ? WIDE_WAVES : WAVES;
        const size_t lds = moe_stream_lds(fmt, dot && !norm, nrows, (int)(lo.S * lo.L), mode,
                                          glu ? (int)(m * top_k) : 0, lo.R, nw);
        Geom g{};
        g.n = (int32_t)lo.n;
        g.k = (int32_t)lo.k;
        g.nb = (int32_t)lo.nb;
        g.L = lo.L;
        g.lsh = lo.lsh;
        g.R = lo.R;
        g.S = (int32_t)lo.S;
        g.tiles = (int32_t)lo.tiles;
        g.ctb = lo.ctb;
        g.stb = lo.stb;
        g.soff = lo.soff;
        // waves per tile, splitting its items, when tiles are few: down-combine
        // up to four, gate_up two (MI355X, the MXFP4 expert shapes at one and
        // four tokens: gate_up 11.4 / 32.6 us with one wave per tile, 9.5 /
        // 24.6 with two, 12.2 / 28.4 with four)
        int IS = 1;
        if (lo.tiles < 4096) IS = 2;
        if (mode == QG_MOE_DOWN_COMBINE && lo.tiles < 2048) IS = 4;
        // the plain gate_up of several tokens over short items (<= 4 steps per
        // lane) splits them over four waves in batches of 4 steps: twice the
        // waves, half the weight registers each (MI355X, 3584x2048 MXFP4 at four
        // tokens: 23.3 -> 18.7 us; at one token 9.3 -> 9.7, so not there;
        // down-combine, already four waves per tile, in batches of 4 steps:
        // 18.2 -> 18.6, not taken)
        const bool short_items = mode == QG_MOE_GATE_UP && !norm && !glu && m > 1 && lo.S <= 4;
        if (short_items && lo.tiles < 2048) IS = 4;
        if (wide) IS = WIDE_WAVES;
        a.isplit = IS;
        g.KS = 1;
        g.ksh = 0;
        g.tpi = nw / IS;
        // with the gate a workgroup holds tpi / 2 gate/up tile pairs
        g.ngroups = glu ? (int32_t)((e.half_tiles + g.tpi / 2 - 1) / (g.tpi / 2))
                        : (int32_t)((lo.tiles + g.tpi - 1) / g.tpi);
        g.SW = (int32_t)lo.S;
        g.nwin = 1;
        g.wblk = (int32_t)(lo.S * lo.L);
        if (lds <= (glu ? MOE_STREAM_LDS_GLU : MOE_STREAM_LDS) && g.ngroups <= 65535) {
            g.w = (const uint8_t *)w_experts;
            const int ms = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8;
            moe_stream_fn f = fmt == QG_Q8_0 ? moe_stream_kernel_q8_0(xt, mode, ms, norm, glu, short_items, wide)
                              : fmt == QG_Q4_0 ? moe_stream_kernel_q4_0(xt, mode, ms, norm, glu, short_items, wide)
                                               : moe_stream_kernel_mxfp4(xt, mode, ms, norm, glu, short_items, wide);
            void *args[] = {(void *)&g, (void *)&a, (void *)&e, (void *)&x};
            if (allow_lds((const void *)f, lds) != hipSuccess) return QG_EHIP;
            hipError_t err = hipLaunchKernel((const void *)f, dim3(g.ngroups), dim3(64 * nw), args, lds, s);
            return err == hipSuccess ? launch_status() : QG_EHIP;
        }
    }
    if (fused) return QG_EUNSUPPORTED;     // the per-expert kernels have no fused epilogue
    // general kernels: activations staged per expert in windows
    float *yf = (float *)y;
    Plan p = make_plan(lo, QG_MAX_M, dot, QG_MAX_M);
    const int maxdistinct = (int)((m * top_k < n_experts) ? m * top_k : n_experts);
    size_t lds = p.lds;
    if (mode == QG_MOE_DOWN_COMBINE) {
        const size_t rows_pg = (size_t)p.g.tpi * p.g.R;
        lds += (size_t)(m * top_k + QG_MAX_M) * rows_pg * 4;
    }
    hipError_t err = fmt == QG_Q8_0 ? launch_moe_q8_0(xt, mode, p, a, maxdistinct, lds, x, yf, s)
                     : fmt == QG_Q4_0 ? launch_moe_q4_0(xt, mode, p, a, maxdistinct, lds, x, yf, s)
                                      : launch_moe_mxfp4(xt, mode, p, a, maxdistinct, lds, x, yf, s);
    if (err != hipSuccess) return QG_EHIP;
    return launch_status();
}

int moe_qgemv_topk(int fmt, const void *w_experts, int64_t n_experts, int64_t n, int64_t k,
                   const int32_t *topk_ids, const float *topk_w, int64_t m, int64_t top_k,
                   const void *x, int xt, int mode, float *y, void *stream)
{
    return moe_impl(fmt, w_experts, n_experts, n, k, topk_ids, topk_w, m, top_k, x, xt, mode, nullptr, 0.0f,
                    QG_ACT_NONE, nullptr, y, QG_F32, stream);
}

int moe_qgemv_topk_fused(int fmt, const void *w_experts, int64_t n_experts, int64_t n, int64_t k,
                         const int32_t *topk_ids, const float *topk_w, int64_t m, int64_t top_k,
                         const void *x, int xt, int mode, const float *norm_weight, float norm_eps, int act,
                         const float *residual, void *y, int yt, void *stream)
{
    return moe_impl(fmt, w_experts, n_experts, n, k, topk_ids, topk_w, m, top_k, x, xt, mode, norm_weight, norm_eps,
                    act, residual, y, yt, stream);
}

int moe_router_topk(const float *logits, int64_t m, int64_t n_experts, int64_t top_k, int32_t *ids, float *weights,
                    void *stream)
{
    if (!logits || !ids || !weights) return QG_EINVAL;
    if (m < 1 || n_experts < 1 || top_k < 1 || top_k > n_experts) return QG_EINVAL;
    if (n_experts > ROUTER_MAX_EXPERTS || top_k > ROUTER_MAX_K || m > 0x7FFFFFFF) return QG_EUNSUPPORTED;
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(weights, 4)) return QG_EALIGN;
    const int nv = (int)((n_experts + 63) / 64);
    void (*f)(const float *, int, int, int32_t *, float *) = nv <= 1 ? k_router<1> : nv <= 2 ? k_router<2>
                                                             : nv <= 4 ? k_router<4> : nv <= 8 ? k_router<8>
                                                                                    : k_router<16>;
    hipLaunchKernelGGL(f, dim3((unsigned)m), dim3(64), 0, as_stream(stream), logits, (int)n_experts, (int)top_k, ids,
                       weights);
    return launch_status();
}

int64_t qg_chain_plan_bytes(int64_t count)
{
    if (count < 1 || count > (1 << 20)) return -1;
    return (int64_t)(sizeof(ChainHdr) + 16 + (size_t)count * sizeof(ChainLink));
}

int qg_chain_plan(int fmt, int xt, int64_t m, const qg_chain_link_t *links, int64_t count, void *plan)
{
    if (!valid_fmt(fmt) || (xt != QG_F32 && xt != QG_BF16) || m < 1 || m > QG_MAX_M) return QG_EINVAL;
    if (!links || !plan || count < 1) return QG_EINVAL;
    if (fmt == QG_NVFP4 || is_kq(fmt)) return QG_EUNSUPPORTED;
    if (count > (1 << 20)) return QG_EUNSUPPORTED;
    int dev = 0, cus = 0, occ = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QG_EHIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return QG_EHIP;
    ChainHdr *h = (ChainHdr *)plan;
    ChainLink *L = (ChainLink *)((uint8_t *)plan + sizeof(ChainHdr) + 16);
    int P = cus < CHAIN_MAX_WG ? cus : CHAIN_MAX_WG;
    size_t xs = 0, part = 0, outb = 0;
    for (int64_t i = 0; i < count; ++i) {
        size_t a = 0, b = 0, c = 0;
        int st = chain_link_plan(fmt, xt, (int)m, P, links[i], &L[i], &a, &b, &c);
        if (st) return st;
        xs = a > xs ? a : xs;
        part = b > part ? b : part;
        outb = c > outb ? c : outb;
    }
    // LDS: staged x of the widest link, then partial sums, then finished rows
    const size_t lds = xs + part + outb;
    if (lds > CHAIN_LDS_MAX) return QG_EUNSUPPORTED;
    const void *fn = chain_kernel(fmt, xt, (int)m);
    if (allow_lds(fn, lds) != hipSuccess) return QG_EHIP;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, CTPB, lds) != hipSuccess) return QG_EHIP;
    if (occ < 1) return QG_EUNSUPPORTED;
    // The grid barriers need every workgroup resident at once.  A kernel that
    // spills registers to scratch may have its waves held back until scratch
    // memory is free (the runtime sizes scratch for fewer waves than a full
    // device), which would leave the barrier waiting for workgroups that
    // cannot start; such a variant is refused.
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, fn) != hipSuccess) return QG_EHIP;
    if (fa.localSizeBytes > 0) return QG_EUNSUPPORTED;
    memset(h, 0, sizeof(*h));
    h->magic = CHAIN_MAGIC;
    h->fmt = fmt;
    h->xt = xt;
    h->m = (int32_t)m;
    h->count = (int32_t)count;
    h->grid = P;
    h->lds = (int64_t)lds;
    h->part_off = (int64_t)xs;
    h->out_off = (int64_t)(xs + part);
    return QG_OK;
}

int qgemv_chain(const void *plan_host, const void *plan_device, void *stream)
{
    if (!plan_host || !plan_device) return QG_EINVAL;
    const ChainHdr *h = (const ChainHdr *)plan_host;
    if (h->magic != CHAIN_MAGIC || h->count < 1 || h->grid < 1) return QG_EINVAL;
    if (!aligned(plan_device, 16)) return QG_EALIGN;
    return chain_launch(h, plan_device, as_stream(stream));
}

int qgemv_chain_noalloc(const void *plan_host, void *stream)
{
    if (!plan_host) return QG_EINVAL;
    const ChainHdr *h = (const ChainHdr *)plan_host;
    if (h->magic != CHAIN_MAGIC || h->count < 1 || h->grid < 1) return QG_EINVAL;
    const int64_t bytes = qg_chain_plan_bytes(h->count);
    if (bytes < 0) return QG_EINVAL;
    if (bytes > QG_CHAIN_STATIC_BYTES) return QG_EUNSUPPORTED;
    void *p = nullptr;
    const int st = scratch_on_device(&p);
    if (st) return st;
    // the whole plan is rewritten, so nothing of an earlier call's plan is read
    if (hipMemcpyAsync(p, plan_host, (size_t)bytes, hipMemcpyHostToDevice, as_stream(stream)) != hipSuccess)
        return QG_EHIP;
    return chain_launch(h, p, as_stream(stream));
}

int qg_chain_error(void)
{
    if (hipDeviceSynchronize() != hipSuccess) return -1;
    int a = chain_error_q8_0(true), b = chain_error_q4_0(true), c = chain_error_mxfp4(true);
    if (a < 0 || b < 0 || c < 0) return -1;
    return (a | b | c) ? 1 : 0;
}

} // extern "C"
