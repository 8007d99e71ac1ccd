// qg_nvfp4.hip -- NVFP4 instantiations of the dense GEMV kernels and the
// load-time Q8_0 -> NVFP4 re-quantizer (a "decode cache").
//
// imp converts GGUF Q8_0 weights to FP4 when a model loads and streams the
// FP4 copy during decode, roughly halving the bytes per token (imp README,
// "Why this exists"; its sm_120a kernels dequantize NVFP4 with packed E2M1 /
// E4M3 conversions: "Features" table).  Its release notes record the cost: the
// cache changes the numerics, and v0.4.1 moved Q8_0 decode back to a path
// that reads the Q8_0 bytes.  Here the cache is an explicit, separate call;
// the Q8_0 product is untouched.
//
// NVFP4 (public definition): blocks of 16 E2M1 values with one FP8 E4M3 scale
// each and one fp32 scale per tensor.  The re-quantizer follows the usual
// recipe, in fp32 and in this order:
//   A   = max |w| over the tensor            (w = d * q of the Q8_0 blocks, exact)
//   s_t = A / 2688 (= 6 * 448, the largest E2M1 times the largest E4M3), or 1
//   per block of 16:  a = max |w|;  s = E4M3 rounding of (a / 6) / s_t
//                     S = E4M3(s) * s_t;  code = E2M1 rounding of w / S (0 if S = 0)
// Roundings are to nearest with ties to the even code, saturating at the
// largest finite value (448 and 6).  Inputs must be finite.
#include "qg_fused.h"

namespace qg {

dense_fn dense_kernel_nvfp4(int xt, int m)
{
    return xt == QG_BF16 ? pick_dense<QG_NVFP4, true, true>(m) : pick_dense<QG_NVFP4, false, false>(m);
}

dense_fn dense_one_kernel_nvfp4(int xt, int m, int u)
{
    return xt == QG_BF16 ? pick_dense_one<QG_NVFP4, true, true>(m, u) : pick_dense_one<QG_NVFP4, false, false>(m, u);
}

dense_ep_fn dense_one_ep_kernel_nvfp4(int xt, int m, int u) { return pick_dense_one_ep<QG_NVFP4>(xt, m, u); }

dense_ep_fn dense_ep_kernel_nvfp4(int xt, int m, bool norm, int glu)
{
    return pick_dense_ep_fmt<QG_NVFP4>(xt, m, norm, glu);
}

namespace {

// Nearest E2M1 code of r (ties to the even code, saturating at +-6; zero
// magnitudes get the +0 code; NaN gives 0): compare |r| with the midpoints of
// the value list {0, 0.5, 1, 1.5, 2, 3, 4, 6}, the tie side of each midpoint
// going to the even code.
__device__ __forceinline__ uint32_t e2m1_rne(float r)
{
    const float a = fabsf(r);
    uint32_t m;
    if (!(a == a) || a <= 0.25f) m = 0;
    else if (a < 0.75f) m = 1;
    else if (a <= 1.25f) m = 2;
    else if (a < 1.75f) m = 3;
    else if (a <= 2.5f) m = 4;
    else if (a < 3.5f) m = 5;
    else if (a <= 5.0f) m = 6;
    else m = 7;
    return (m != 0 && r < 0.0f) ? (m | 8u) : m;
}

// Nearest non-negative E4M3 code of v >= 0 (ties to the even code,
// saturating at 448 = 0x7E; NaN gives 0), from the fp32 bits: below 2^-6 the
// subnormal grid m * 2^-9 (rounded by rint, which rounds ties to even), above
// it the 23-bit mantissa rounded to 3 bits.
__device__ __forceinline__ uint32_t e4m3_rne(float v)
{
    if (!(v == v)) return 0;
    if (!(v < 448.0f)) return 0x7E;
    if (v < 0x1p-6f) return (uint32_t)__builtin_rintf(v * 512.0f);     // 0..8; 8 is the code of 2^-6
    const uint32_t b = __builtin_bit_cast(uint32_t, v);
    int e = (int)((b >> 23) & 255) - 127;                                // -6 .. 8
    uint32_t keep = (b >> 20) & 7, rem = b & 0xFFFFF;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1))) ++keep;
    if (keep == 8) {
        keep = 0;
        ++e;
    }
    const uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
    return code > 0x7E ? 0x7E : code;
}

// Writes the tensor's largest |w| slot (the trailer word after the tensor
// scale) as zero before the maximum is taken.
__global__ void k_requant_init(uint8_t *__restrict__ packed, int64_t tsoff)
{
    if (threadIdx.x == 0) *(uint32_t *)(packed + tsoff + 4) = 0;
}

// max |w| of the Q8_0 tensor: one canonical block per thread, the wave's
// maximum folded into the slot by an atomic maximum on the (non-negative)
// float bits, an exact and order-free reduction.
__global__ void k_requant_amax(const uint8_t *__restrict__ canon, int64_t nblocks, uint8_t *__restrict__ packed,
                               int64_t tsoff)
{
    float a = 0.0f;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nblocks; i += (int64_t)gridDim.x * blockDim.x) {
        const uint8_t *b = canon + i * 34;
        const float d = fabsf(f16_bits_to_f32((uint32_t)b[0] | ((uint32_t)b[1] << 8)));
        int qm = 0;
        for (int j = 0; j < 32; ++j) qm = max(qm, abs((int)(int8_t)b[2 + j]));
        a = fmaxf(a, d * (float)qm);     // exact: |d * q| is largest for the largest |q|
    }
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    if ((threadIdx.x & 63) == 0 && a > 0.0f)
        atomicMax((unsigned int *)(packed + tsoff + 4), __builtin_bit_cast(unsigned int, a));
}

// One thread per packed record: the record's 32 weights (two NVFP4 blocks)
// quantized and written in the packed layout; padding records get zeros.
// Thread 0 also writes the tensor scale.
__global__ void k_requant(LayoutArgs a, const uint8_t *__restrict__ canon, uint8_t *__restrict__ packed, int64_t nrec)
{
    const float A = __builtin_bit_cast(float, *(const uint32_t *)(packed + a.tsoff + 4));
    const float st = A > 0.0f ? A / 2688.0f : 1.0f;
    const int64_t tid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x, nthr = (int64_t)gridDim.x * blockDim.x;
    if (tid == 0) *(float *)(packed + a.tsoff) = st;
    // the rest of the trailer and the tail padding: zero (the max slot stays)
    for (int64_t o = a.end + tid; o < a.total; o += nthr)
        if (o < a.tsoff || o >= a.tsoff + 8) packed[o] = 0;
    for (int64_t rec = tid; rec < nrec; rec += nthr) {
        int64_t row, blk, co, so;
        record_geom(a, rec, &row, &blk, &co, &so);
        uint32_t packed_codes[4] = {0, 0, 0, 0};
        uint32_t scales = 0;
        if (row < a.n && blk < a.nb) {
            const uint8_t *b = canon + (row * a.nb + blk) * 34;
            const float d = f16_bits_to_f32((uint32_t)b[0] | ((uint32_t)b[1] << 8));
            float w[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) w[j] = d * (float)(int8_t)b[2 + j];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float amax = 0.0f;
#pragma unroll
                for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(w[16 * h + j]));
                const float u = amax / 6.0f;
                const float v = u / st;
                const uint32_t s8 = e4m3_rne(v);
                const float S = e4m3_to_f32(s8) * st;
                scales |= s8 << (8 * h);
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int e = 16 * h + j;       // packed byte e / 2, low nibble for even e
                    const uint32_t c = S == 0.0f ? 0u : e2m1_rne(w[e] / S);
                    packed_codes[e >> 3] |= c << (4 * (e & 7));
                }
            }
        }
        *(uint4 *)(packed + co) = make_uint4(packed_codes[0], packed_codes[1], packed_codes[2], packed_codes[3]);
        packed[so] = (uint8_t)(scales & 0xFF);
        packed[so + 1] = (uint8_t)(scales >> 8);
    }
}

} // namespace

// Enqueues the three re-quantization kernels (the argument checks are the caller's).
hipError_t launch_requant_nvfp4(const Layout &lo, const uint8_t *canon_q8_0, uint8_t *packed, hipStream_t s)
{
    const LayoutArgs a = layout_args(lo);
    const int64_t nblocks = lo.n * lo.nb, nrec = lo.tiles * lo.S * 64;
    hipLaunchKernelGGL(k_requant_init, dim3(1), dim3(64), 0, s, packed, lo.tsoff);
    int64_t g1 = (nblocks + 255) / 256;
    if (g1 > 65535 * 8) g1 = 65535 * 8;
    hipLaunchKernelGGL(k_requant_amax, dim3((unsigned)g1), dim3(256), 0, s, canon_q8_0, nblocks, packed, lo.tsoff);
    int64_t g2 = (nrec + 255) / 256;
    if (g2 > 65535 * 8) g2 = 65535 * 8;
    hipLaunchKernelGGL(k_requant, dim3((unsigned)g2), dim3(256), 0, s, a, canon_q8_0, packed, nrec);
    return hipGetLastError();
}

} // namespace qg
