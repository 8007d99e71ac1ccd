#pragma once
// qg_common.h -- shared device code of the block-quantized weight GEMV library
// for MI355X (gfx950, CDNA4).
//
// The decode step of an LLM streams each weight matrix once per token through
// a matrix-vector product, so the product is bound by HBM bandwidth (imp
// README, "Known limitations": a card with less bandwidth decodes
// proportionally slower).  Everything here is shaped for that:
//
//  * Packed layout (built once at load time).  A tile holds R = 64/L rows.
//    Lane l of a wavefront owns row l/L of the tile and, at step j, block
//    j*L + l%L of that row.  The codes of one step are stored lane-major, so
//    each wavefront load instruction (64 lanes x 16 B) reads 1 KiB that is
//    contiguous in memory.  Scales are a separate stream in the same
//    (tile, step, lane) order.  Nibbles are permuted inside a block so that
//    the unpack below needs one or two ALU operations per pair of weights.
//  * Activations are staged once per workgroup into LDS in the type the
//    inner product uses (fp32 for int8 codes, bf16 pairs for 4-bit codes),
//    in a quad-major order that makes every ds_read_b128 conflict-free.
//  * Inner products: int8 codes go through one sign-extending byte convert
//    and one fp32 FMA per weight; Q4_0 codes are stored as the 4-bit two's
//    complement of q-8 and each becomes the exact fp32 (q-8)/16 through one
//    v_cvt_off_f32_i4 (byte-selected by SDWA), then bf16 pairs for
//    v_dot2c_f32_bf16 (or fp32 FMAs with fp32 activations); E2M1 nibbles are
//    converted two at a time by the gfx950 scaled FP4->bf16 convert and also
//    fed to the bf16 dot.  Every weight enters the dot product as its exact
//    value (times a power of two), so the rounding error of a row is bounded
//    by its sum of |w * x|.  Accumulation is fp32; the block scale is applied
//    once per block.
//  * Split-K inside a workgroup (KS waves per tile) is reduced through LDS in
//    a fixed order, then across the L lanes of a row by a xor butterfly.  No
//    atomics: results are bitwise reproducible.
//
// Prior art on the pages: imp's NVFP4 block-scaled GEMV with packed E2M1
// dequant in registers (imp README, "Features" table, sm_120a kernels row),
// its dp4a Q8_0 decode route (imp release notes, v0.4.1), and Imparo's
// private GateUp weight layout kept beside the canonical GGUF one (Imparo
// README, opening release notes).  Those were built for NVIDIA GPUs; the
// design here is for 64-wide wavefronts, LDS and HBM3E.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <type_traits>

#include "../../include/qgemv.h"

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

namespace qg {


constexpr int QK = 32;          // weights per block
constexpr int WAVES = 4;        // wavefronts per workgroup
constexpr int TPB = 64 * WAVES; // threads per workgroup
constexpr int XBUDGET = 64 * 1024;  // LDS bytes for one window of staged activations

// ------------------------------------------------------------------ layout
struct Layout {
    int fmt, L, lsh, R, P, sb;
    int64_t n, k, nb, S, tiles;
    int64_t ctb, stb, soff, tsoff, total;   // tsoff: NVFP4 tensor scale (fp32), 0 otherwise
    int64_t htb, hoff;           // Q6_K: high code bits, 8 B per record (S * 512 per tile), else 0
    int64_t nsb, sboff;          // K-quants: super-blocks per row, per-row super-block words (4 B), else 0
    int64_t used;                // end of the streams; [used, total) is padding (and the NVFP4 trailer)
};

// The K-quant super-block formats: 256 weights, eight 32-weight sub-blocks.
__host__ __device__ constexpr bool is_kq(int fmt) { return fmt == QG_Q4_K || fmt == QG_Q6_K; }
__host__ __device__ constexpr int kq_bytes(int fmt) { return fmt == QG_Q4_K ? 144 : 210; }

// Staged form of one block of 32 activations in LDS: x_quads() 16-byte quads
// (fp32, or bf16 pairs for the bf16 dot).
__host__ __device__ constexpr int x_quads(int fmt, bool dot) { return dot ? 4 : 8; }

// Canonical bytes per 32 weights (NVFP4: two 16-weight blocks of 9 bytes).
inline int block_bytes(int fmt) { return fmt == QG_Q8_0 ? 34 : fmt == QG_MXFP4 ? 17 : 18; }

inline bool valid_fmt(int fmt)
{
    return fmt == QG_Q8_0 || fmt == QG_Q4_0 || fmt == QG_MXFP4 || fmt == QG_NVFP4 || is_kq(fmt);
}

// Bytes of a canonical n x k tensor (NVFP4: blocks, then its fp32 tensor
// scale; K-quants: super-blocks of 256 weights).
inline int64_t canon_bytes(int fmt, int64_t n, int64_t k)
{
    if (is_kq(fmt)) return n * (k / 256) * kq_bytes(fmt);
    return n * (k / 32) * block_bytes(fmt) + (fmt == QG_NVFP4 ? 4 : 0);
}

inline int ilog2(int v) { int s = 0; while ((1 << s) < v) ++s; return s; }

// Lanes per row.  Padding (blocks beyond k/32 and rows beyond n) is avoided
// first; among the low-padding choices the fewest lanes per row that still give
// >= 512 tiles is taken (long per-lane streams, short reductions), else the
// choice with the most tiles.
inline Layout make_layout(int fmt, int64_t n, int64_t k)
{
    Layout lo{};
    lo.fmt = fmt;
    lo.n = n;
    lo.k = k;
    lo.nb = k / QK;
    lo.P = fmt == QG_Q8_0 ? 2 : 1;
    lo.sb = fmt == QG_MXFP4 ? 1 : 2;
    const int cand[7] = {1, 2, 4, 8, 16, 32, 64};
    double waste[7];
    double best_w = 1e30;
    for (int i = 0; i < 7; ++i) {
        int L = cand[i], R = 64 / L;
        int64_t S = (lo.nb + L - 1) / L, tiles = (n + R - 1) / R;
        double padded = (double)tiles * R * S * L;
        waste[i] = padded / ((double)n * (double)lo.nb) - 1.0;
        if (waste[i] < best_w) best_w = waste[i];
    }
    int pick = -1;
    int64_t target = n < 512 ? n : 512;
    for (int i = 0; i < 7; ++i) {
        if (waste[i] > best_w + 0.005) continue;
        int64_t tiles = (n + 64 / cand[i] - 1) / (64 / cand[i]);
        if (tiles >= target) { pick = i; break; }
    }
    if (pick < 0) {
        for (int i = 6; i >= 0; --i)
            if (waste[i] <= best_w + 0.005) { pick = i; break; }
    }
    lo.L = cand[pick];
    lo.lsh = ilog2(lo.L);
    lo.R = 64 / lo.L;
    lo.S = (lo.nb + lo.L - 1) / lo.L;
    lo.tiles = (n + lo.R - 1) / lo.R;
    lo.ctb = lo.S * lo.P * 1024;
    lo.stb = lo.S * 64 * lo.sb;
    lo.soff = lo.tiles * lo.ctb;
    int64_t end = lo.soff + lo.tiles * lo.stb;
    if (is_kq(fmt)) {
        // Q6_K high code bits; then d (and dmin) per row and super-block,
        // rows of the last tile's padding included
        if (fmt == QG_Q6_K) {
            lo.htb = lo.S * 512;
            lo.hoff = end;
            end += lo.tiles * lo.htb;
        }
        lo.nsb = k / 256;
        lo.sboff = end;
        end += lo.tiles * lo.R * lo.nsb * 4;
    }
    lo.used = end;
    lo.total = (end + 255) / 256 * 256;   // experts stay 256-byte aligned
    lo.tsoff = 0;
    if (fmt == QG_NVFP4) {
        // the fp32 tensor scale in a 256-byte trailer of its own
        lo.tsoff = lo.total;
        lo.total += 256;
    }
    return lo;
}

// ------------------------------------------------- per-block code permutation
// Canonical block -> packed codes (P*16 bytes) and scale; and back.
//  Q8_0 : part 0 = codes 0..15, part 1 = codes 16..31 (no permutation).
//  Q4_0 : packed byte B = t[2B] | t[2B+1] << 4 with t = q ^ 8, the 4-bit two's
//         complement of the signed weight q - 8 (one byte = one adjacent pair).
//  MXFP4: packed byte B = q[2B] | q[2B+1] << 4 (one byte = one adjacent pair).
//  NVFP4: the same for the 32 codes of the two 16-weight blocks (elements
//         0..15 use the first block's scale, 16..31 the second's); the two
//         E4M3 scale bytes form the 16-bit scale entry (first block low).
__host__ __device__ inline void nibbles_from_canon(const uint8_t *body, uint8_t q[32])
{
    for (int j = 0; j < 16; ++j) {
        q[j] = body[j] & 15;
        q[j + 16] = body[j] >> 4;
    }
}

__host__ __device__ inline void nibbles_to_canon(const uint8_t q[32], uint8_t *body)
{
    for (int j = 0; j < 16; ++j)
        body[j] = (uint8_t)(q[j] | (q[j + 16] << 4));
}

__host__ __device__ inline void canon_to_packed(int fmt, const uint8_t *blk, uint8_t *codes, uint16_t *scale)
{
    if (fmt == QG_Q8_0) {
        *scale = (uint16_t)(blk[0] | (blk[1] << 8));
        for (int i = 0; i < 32; ++i) codes[i] = blk[2 + i];
        return;
    }
    uint8_t q[32];
    if (fmt == QG_Q4_0) {
        *scale = (uint16_t)(blk[0] | (blk[1] << 8));
        nibbles_from_canon(blk + 2, q);
        for (int b = 0; b < 16; ++b) codes[b] = (uint8_t)((q[2 * b] ^ 8) | ((q[2 * b + 1] ^ 8) << 4));
        return;
    }
    if (fmt == QG_NVFP4) {
        // blk: [s0][8 bytes of block 0][s1][8 bytes of block 1]; byte j of a
        // block holds its element j (low nibble) and j + 8 (high nibble)
        *scale = (uint16_t)(blk[0] | (blk[9] << 8));
        for (int h = 0; h < 2; ++h)
            for (int j = 0; j < 8; ++j) {
                q[16 * h + j] = blk[9 * h + 1 + j] & 15;
                q[16 * h + j + 8] = blk[9 * h + 1 + j] >> 4;
            }
        for (int b = 0; b < 16; ++b) codes[b] = (uint8_t)(q[2 * b] | (q[2 * b + 1] << 4));
        return;
    }
    *scale = blk[0];
    nibbles_from_canon(blk + 1, q);
    for (int b = 0; b < 16; ++b) codes[b] = (uint8_t)(q[2 * b] | (q[2 * b + 1] << 4));
}

__host__ __device__ inline void packed_to_canon(int fmt, const uint8_t *codes, uint16_t scale, uint8_t *blk)
{
    if (fmt == QG_Q8_0) {
        blk[0] = (uint8_t)(scale & 0xFF);
        blk[1] = (uint8_t)(scale >> 8);
        for (int i = 0; i < 32; ++i) blk[2 + i] = codes[i];
        return;
    }
    uint8_t q[32];
    if (fmt == QG_Q4_0) {
        blk[0] = (uint8_t)(scale & 0xFF);
        blk[1] = (uint8_t)(scale >> 8);
        for (int b = 0; b < 16; ++b) {
            q[2 * b] = (codes[b] & 15) ^ 8;
            q[2 * b + 1] = (codes[b] >> 4) ^ 8;
        }
        nibbles_to_canon(q, blk + 2);
        return;
    }
    for (int b = 0; b < 16; ++b) {
        q[2 * b] = codes[b] & 15;
        q[2 * b + 1] = codes[b] >> 4;
    }
    if (fmt == QG_NVFP4) {
        blk[0] = (uint8_t)(scale & 0xFF);
        blk[9] = (uint8_t)(scale >> 8);
        for (int h = 0; h < 2; ++h)
            for (int j = 0; j < 8; ++j) blk[9 * h + 1 + j] = (uint8_t)(q[16 * h + j] | (q[16 * h + j + 8] << 4));
        return;
    }
    blk[0] = (uint8_t)scale;
    nibbles_to_canon(q, blk + 1);
}

// Geometry passed to the layout kernels.
struct LayoutArgs {
    int fmt, L, lsh, R, P, sb, bb;
    int64_t n, nb, S, tiles, ctb, stb, soff, end, total;   // [end, total) is tail padding
    int64_t tsoff, cts;          // NVFP4: tensor scale offsets, packed and canonical (else 0)
    int64_t htb, hoff, nsb, sboff;   // K-quants (Layout)
};

inline LayoutArgs layout_args(const Layout &lo)
{
    LayoutArgs a;
    a.fmt = lo.fmt; a.L = lo.L; a.lsh = lo.lsh; a.R = lo.R; a.P = lo.P; a.sb = lo.sb;
    a.bb = block_bytes(lo.fmt);
    a.n = lo.n; a.nb = lo.nb; a.S = lo.S; a.tiles = lo.tiles;
    a.ctb = lo.ctb; a.stb = lo.stb; a.soff = lo.soff;
    a.end = lo.used;
    a.htb = lo.htb; a.hoff = lo.hoff; a.nsb = lo.nsb; a.sboff = lo.sboff;
    a.total = lo.total;
    a.tsoff = lo.tsoff;
    a.cts = lo.fmt == QG_NVFP4 ? lo.n * lo.nb * 18 : 0;
    return a;
}

// Tail padding byte o of the packed form (o in [end, total)): zero, except the
// NVFP4 tensor scale, which is copied from the canonical tensor.
__host__ __device__ inline uint8_t tail_byte(const LayoutArgs &a, const uint8_t *canon, int64_t o)
{
    if (a.fmt == QG_NVFP4 && o >= a.tsoff && o < a.tsoff + 4) return canon[a.cts + (o - a.tsoff)];
    return 0;
}

// One record = (tile, step, lane): its row/block and its byte offsets.
__host__ __device__ inline void record_geom(const LayoutArgs &a, int64_t rec, int64_t *row, int64_t *blk,
                                            int64_t *code_off, int64_t *scale_off)
{
    int64_t lane = rec & 63, rest = rec >> 6;
    int64_t j = rest % a.S, tile = rest / a.S;
    *row = tile * a.R + (lane >> a.lsh);
    *blk = j * a.L + (lane & (a.L - 1));
    *code_off = tile * a.ctb + j * a.P * 1024 + lane * 16;
    *scale_off = a.soff + tile * a.stb + j * 64 * a.sb + lane * a.sb;
}

// ------------------------------------------------------- K-quant records
// A K-quant record is one 32-weight sub-block (sub-block j = blk % 8 of
// super-block blk / 8 of its row), in element order (weights 32j..32j+31 of
// the super-block):
//  Q4_K: codes as Q4_0 (packed byte B = t[2B] | t[2B+1] << 4, t = q ^ 8); the
//        16-bit scale entry is sc | m << 8.
//  Q6_K: with t = q ^ 32 (the 6-bit two's complement of q - 32): code dword a
//        byte b = (t[8a+b] & 15) | (t[8a+4+b] & 15) << 4; high-bits dword h
//        byte b holds t >> 4 of elements 16h+b, 16h+4+b, 16h+8+b, 16h+12+b in
//        its bit pairs 0-1, 2-3, 4-5, 6-7; the scale entry is the two int8
//        scales (elements 0..15 low byte, 16..31 high byte).
//  The row's super-block word (d | dmin << 16 for Q4_K, d for Q6_K) sits in
//  the super-block stream at sboff + (row * nsb + blk / 8) * 4.

// Sub-block j's 6-bit scale and min of a Q4_K super-block's 12 scale bytes.
__host__ __device__ inline void q4k_scale_min(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

// Byte offset of the Q6_K high bits of record rec.
__host__ __device__ inline int64_t kq_high_off(const LayoutArgs &a, int64_t rec)
{
    const int64_t lane = rec & 63, rest = rec >> 6;
    return a.hoff + (rest / a.S) * a.htb + (rest % a.S) * 512 + lane * 8;
}

__host__ __device__ inline void pack_record_kq(const LayoutArgs &a, const uint8_t *canon, uint8_t *packed, int64_t rec)
{
    int64_t row, blk, co, so;
    record_geom(a, rec, &row, &blk, &co, &so);
    uint8_t codes[16], hi[8];
    for (int i = 0; i < 16; ++i) codes[i] = 0;
    for (int i = 0; i < 8; ++i) hi[i] = 0;
    uint32_t scale = 0, sbw = 0;
    if (row < a.n && blk < a.nb) {
        const int j = (int)(blk & 7);
        const uint8_t *sb = canon + (row * a.nsb + (blk >> 3)) * kq_bytes(a.fmt);
        uint8_t t[32];
        if (a.fmt == QG_Q4_K) {
            for (int l = 0; l < 32; ++l) {
                const uint8_t byte = sb[16 + 32 * (j >> 1) + l];
                t[l] = (uint8_t)(((j & 1) ? byte >> 4 : byte & 15) ^ 8);
            }
            for (int b = 0; b < 16; ++b) codes[b] = (uint8_t)(t[2 * b] | (t[2 * b + 1] << 4));
            int sc, m;
            q4k_scale_min(sb + 4, j, &sc, &m);
            scale = (uint32_t)sc | ((uint32_t)m << 8);
            sbw = (uint32_t)sb[0] | ((uint32_t)sb[1] << 8) | ((uint32_t)sb[2] << 16) | ((uint32_t)sb[3] << 24);
        } else {
            const int h = j >> 2, r = j & 3;
            for (int l = 0; l < 32; ++l) {
                const uint8_t lb = sb[64 * h + l + 32 * (r & 1)];
                const int lo = r < 2 ? (lb & 15) : (lb >> 4);
                const int hb = (sb[128 + 32 * h + l] >> (2 * r)) & 3;
                t[l] = (uint8_t)((lo | (hb << 4)) ^ 32);
            }
            for (int q = 0; q < 4; ++q)
                for (int b = 0; b < 4; ++b) codes[4 * q + b] = (uint8_t)((t[8 * q + b] & 15) | ((t[8 * q + 4 + b] & 15) << 4));
            for (int q = 0; q < 2; ++q)
                for (int b = 0; b < 4; ++b)
                    hi[4 * q + b] = (uint8_t)((t[16 * q + b] >> 4) | ((t[16 * q + 4 + b] >> 4) << 2) |
                                              ((t[16 * q + 8 + b] >> 4) << 4) | ((t[16 * q + 12 + b] >> 4) << 6));
            scale = (uint32_t)sb[192 + 8 * h + 2 * r] | ((uint32_t)sb[192 + 8 * h + 2 * r + 1] << 8);
            sbw = (uint32_t)sb[208] | ((uint32_t)sb[209] << 8);
        }
    }
    for (int i = 0; i < 16; ++i) packed[co + i] = codes[i];
    packed[so] = (uint8_t)(scale & 0xFF);
    packed[so + 1] = (uint8_t)(scale >> 8);
    if (a.fmt == QG_Q6_K) {
        const int64_t ho = kq_high_off(a, rec);
        for (int i = 0; i < 8; ++i) packed[ho + i] = hi[i];
    }
    if ((blk & 7) == 0 && blk < a.nb) {       // the row's super-block word (zero on padding rows)
        const int64_t wo = a.sboff + (row * a.nsb + (blk >> 3)) * 4;
        for (int i = 0; i < 4; ++i) packed[wo + i] = (uint8_t)(sbw >> (8 * i));
    }
}

// Rebuilds canonical super-block s of row `row` from its eight records.
__host__ __device__ inline void unpack_superblock_kq(const LayoutArgs &a, const uint8_t *packed, uint8_t *canon,
                                                     int64_t row, int64_t s)
{
    uint8_t out[210];
    const int nbytes = kq_bytes(a.fmt);
    for (int i = 0; i < nbytes; ++i) out[i] = 0;
    const int64_t wo = a.sboff + (row * a.nsb + s) * 4;
    if (a.fmt == QG_Q4_K) {
        for (int i = 0; i < 4; ++i) out[i] = packed[wo + i];
    } else {
        out[208] = packed[wo];
        out[209] = packed[wo + 1];
    }
    const int64_t tile = row / a.R, rr = row % a.R;
    for (int j = 0; j < 8; ++j) {
        const int64_t blk = 8 * s + j;
        const int64_t rec = ((tile * a.S) + (blk >> a.lsh)) * 64 + ((rr << a.lsh) | (blk & (a.L - 1)));
        int64_t r2, b2, co, so;
        record_geom(a, rec, &r2, &b2, &co, &so);
        const uint32_t scale = (uint32_t)packed[so] | ((uint32_t)packed[so + 1] << 8);
        uint8_t t[32];
        if (a.fmt == QG_Q4_K) {
            for (int b = 0; b < 16; ++b) {
                t[2 * b] = (uint8_t)((packed[co + b] & 15) ^ 8);
                t[2 * b + 1] = (uint8_t)((packed[co + b] >> 4) ^ 8);
            }
            for (int l = 0; l < 32; ++l) out[16 + 32 * (j >> 1) + l] |= (uint8_t)((j & 1) ? t[l] << 4 : t[l]);
            const int sc = scale & 63, m = (scale >> 8) & 63;
            uint8_t *sx = out + 4;
            if (j < 4) {
                sx[j] |= (uint8_t)sc;
                sx[j + 4] |= (uint8_t)m;
            } else {
                sx[j + 4] |= (uint8_t)((sc & 15) | ((m & 15) << 4));
                sx[j - 4] |= (uint8_t)((sc >> 4) << 6);
                sx[j] |= (uint8_t)((m >> 4) << 6);
            }
        } else {
            const int64_t ho = kq_high_off(a, rec);
            for (int q = 0; q < 4; ++q)
                for (int b = 0; b < 4; ++b) {
                    t[8 * q + b] = packed[co + 4 * q + b] & 15;
                    t[8 * q + 4 + b] = packed[co + 4 * q + b] >> 4;
                }
            for (int q = 0; q < 2; ++q)
                for (int b = 0; b < 4; ++b) {
                    const uint8_t hb = packed[ho + 4 * q + b];
                    for (int f = 0; f < 4; ++f) t[16 * q + 4 * f + b] |= (uint8_t)(((hb >> (2 * f)) & 3) << 4);
                }
            const int h = j >> 2, r = j & 3;
            for (int l = 0; l < 32; ++l) {
                const int qv = t[l] ^ 32;
                out[64 * h + l + 32 * (r & 1)] |= (uint8_t)(r < 2 ? (qv & 15) : (qv & 15) << 4);
                out[128 + 32 * h + l] |= (uint8_t)((qv >> 4) << (2 * r));
            }
            out[192 + 8 * h + 2 * r] = (uint8_t)(scale & 0xFF);
            out[192 + 8 * h + 2 * r + 1] = (uint8_t)(scale >> 8);
        }
    }
    uint8_t *dst = canon + (row * a.nsb + s) * nbytes;
    for (int i = 0; i < nbytes; ++i) dst[i] = out[i];
}

__host__ __device__ inline void pack_record(const LayoutArgs &a, const uint8_t *canon, uint8_t *packed, int64_t rec)
{
    if (is_kq(a.fmt)) {
        pack_record_kq(a, canon, packed, rec);
        return;
    }
    int64_t row, blk, co, so;
    record_geom(a, rec, &row, &blk, &co, &so);
    uint8_t codes[32];
    uint16_t scale = 0;
    for (int i = 0; i < 32; ++i) codes[i] = 0;
    if (row < a.n && blk < a.nb) {
        uint8_t b[34];
        const uint8_t *src = canon + (row * a.nb + blk) * a.bb;
        for (int i = 0; i < a.bb; ++i) b[i] = src[i];
        canon_to_packed(a.fmt, b, codes, &scale);
    }
    for (int h = 0; h < a.P; ++h)
        for (int i = 0; i < 16; ++i) packed[co + h * 1024 + i] = codes[16 * h + i];
    packed[so] = (uint8_t)(scale & 0xFF);
    if (a.sb == 2) packed[so + 1] = (uint8_t)(scale >> 8);
}

__host__ __device__ inline void unpack_record(const LayoutArgs &a, const uint8_t *packed, uint8_t *canon, int64_t rec)
{
    int64_t row, blk, co, so;
    record_geom(a, rec, &row, &blk, &co, &so);
    if (row >= a.n || blk >= a.nb) return;
    uint8_t codes[32];
    for (int h = 0; h < a.P; ++h)
        for (int i = 0; i < 16; ++i) codes[16 * h + i] = packed[co + h * 1024 + i];
    uint16_t scale = packed[so];
    if (a.sb == 2) scale = (uint16_t)(scale | (packed[so + 1] << 8));
    uint8_t b[34];
    packed_to_canon(a.fmt, codes, scale, b);
    uint8_t *dst = canon + (row * a.nb + blk) * a.bb;
    for (int i = 0; i < a.bb; ++i) dst[i] = b[i];
}

// ------------------------------------------------------------ unpack math
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// OCP FP8 E4M3 -> fp32 (exact): 1 sign, 4 exponent bits (bias 7), 3
// mantissa bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN.
__host__ __device__ __forceinline__ float e4m3_to_f32(uint32_t b)
{
    const uint32_t e = (b >> 3) & 15, m = b & 7;
    float v = e == 0 ? (float)m * 0x1p-9f : __builtin_bit_cast(float, ((e + 120) << 23) | (m << 20));
    if (e == 15 && m == 7) v = __builtin_nanf("");
    return (b & 0x80) ? -v : v;
}

// UE8M0 -> fp32 2^(E-127): E = 0 is the subnormal 2^-127, E = 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t e)
{
    uint32_t b = e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : (e << 23));
    return __builtin_bit_cast(float, b);
}

__device__ __forceinline__ float i8_at(uint32_t w, int p)
{
    return (float)(int8_t)(w >> (8 * p));   // v_cvt_f32_i32 with a sign-extended byte select
}

// The eight Q4_0 weights of a packed dword, in element order, as the exact
// fp32 values (q - 8) / 16.  Byte b holds t = q ^ 8 of elements 2b (low
// nibble) and 2b + 1 (high nibble); v_cvt_off_f32_i4 reads bits [3:0] of its
// operand as a signed 4-bit integer s and returns s / 16 exactly (the CDNA3
// ISA's table for it runs from -0.5 for 1000b to 0.4375 for 0111b).  SDWA
// selects the byte, so the dword costs one shift and eight converts.  The
// block scale is applied as 16 * d.
__device__ __forceinline__ void q4_unpack8(uint32_t w, float (&v)[8])
{
    uint32_t h;
    asm("v_lshrrev_b32 %8, 4, %9\n\t"
        "v_cvt_off_f32_i4_e32 %0, %9\n\t"
        "v_cvt_off_f32_i4_e32 %1, %8\n\t"
        "v_cvt_off_f32_i4_sdwa %2, %9 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1\n\t"
        "v_cvt_off_f32_i4_sdwa %3, %8 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1\n\t"
        "v_cvt_off_f32_i4_sdwa %4, %9 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_off_f32_i4_sdwa %5, %8 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2\n\t"
        "v_cvt_off_f32_i4_sdwa %6, %9 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3\n\t"
        "v_cvt_off_f32_i4_sdwa %7, %8 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
          "=&v"(h)
        : "v"(w));
}

// Two exact fp32 values (at most 8 significant bits) as a bf16 pair.
__device__ __forceinline__ bf16x2_t pk_bf16(float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    return __builtin_convertvector(v, bf16x2_t);
}

// Q4_0 block scale as applied to the (q - 8) / 16 values.
__device__ __forceinline__ float q4_scale(uint32_t bits) { return 16.0f * f16_bits_to_f32(bits); }

// Global-memory accessors.  Pointers that reach a kernel through memory (not
// as kernel arguments) are generic; casting them to the global address space
// keeps the accesses global_* (flat accesses would also count against the LDS
// wait counter and serialise LDS waits behind weight loads in flight).
#define QG_GLOBAL __attribute__((address_space(1)))
typedef unsigned int qg_u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load of weights: read once, so marked nontemporal.
__device__ __forceinline__ uint4 ld_stream16(const uint8_t *p)
{
    const qg_u32x4 v = __builtin_nontemporal_load((const QG_GLOBAL qg_u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Narrow results: a caller that keeps them narrow until their use keeps the
// widening (and so the wait for the load) at the use.
__device__ __forceinline__ uint16_t ld_stream_u16(const uint16_t *p)
{
    return __builtin_nontemporal_load((const QG_GLOBAL uint16_t *)p);
}

__device__ __forceinline__ uint8_t ld_stream_u8(const uint8_t *p)
{
    return __builtin_nontemporal_load((const QG_GLOBAL uint8_t *)p);
}

__device__ __forceinline__ uint4 ld_global16(const void *p)
{
    const qg_u32x4 v = *(const QG_GLOBAL qg_u32x4 *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void st_global_f32(float *p, float v)
{
    *(QG_GLOBAL float *)p = v;
}

__device__ __forceinline__ bf16x2_t u32_as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

__device__ __forceinline__ float dot2(bf16x2_t a, bf16x2_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// Byte p of a packed MXFP4 dword as a bf16 pair (element 2p of the dword's
// eight, element 2p+1), scale 1.0 (the block scale is applied in fp32 later).
template <int PSEL>
__device__ __forceinline__ bf16x2_t fp4_pair_bf16(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, PSEL);
}

template <int PSEL>
__device__ __forceinline__ f32x2_t fp4_pair_f32(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, PSEL);
}

// Staged form of one block of 32 activations (raw: 4 quads of bf16 or 8
// quads of fp32, in element order): q[0 .. x_quads).
template <bool XBF16, bool DOT>
__device__ __forceinline__ void stage_block(const uint4 *raw, uint4 (&q)[8])
{
    if (XBF16) {
        if (DOT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = raw[i];
        } else {
            const uint32_t *rw = (const uint32_t *)raw;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t a0 = rw[2 * i], a1 = rw[2 * i + 1];
                q[i] = make_uint4(a0 << 16, a0 & 0xFFFF0000u, a1 << 16, a1 & 0xFFFF0000u);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = raw[i];
    }
}

// ------------------------------------------------------------- GEMV engine
// A "pass" of one workgroup: WAVES/KS tiles, each covered by KS waves that
// split the tile's steps (step j goes to wave j % KS).  Activations for up to
// M token slots are staged in LDS per window of SW steps.
struct Geom {
    const uint8_t *w;            // packed matrix base
    int32_t n, k, nb;
    int32_t L, lsh, R, S, tiles;
    int64_t ctb, stb, soff;
    int64_t tsoff;               // NVFP4: byte offset of the fp32 tensor scale
    int64_t hoff, htb, sboff;    // K-quants: high-bits stream (Q6_K), super-block words
    int32_t nsb;                 // K-quants: super-blocks per row
    int32_t KS, ksh, tpi, ngroups;
    int32_t SW, nwin, wblk;      // steps per window, windows, blocks per window
};

// Where the activations of token slot t come from and where its outputs go.
// Both arrays live in LDS so that the offsets cost no registers.
struct Slots {
    const int32_t *xrow;         // activation row of slot t: x + xrow[t] * k
    const int32_t *yrow;         // output row of slot t:     y + yrow[t] * n + row
};

template <bool XBF16, bool DOT>
struct XStage {
    // Stages window w of M slots: xs[(t*QPB + q)*wblk + bl] (16 B quads).
    template <int M, int FMT>
    static __device__ __forceinline__ void run(const Geom &g, const void *x, const Slots &sl, int w, uint4 *xs)
    {
        constexpr int QPB = x_quads(FMT, DOT);
        const int b0 = w * g.SW * g.L;
        const int total = M * g.wblk;
        for (int idx = threadIdx.x; idx < total; idx += (int)blockDim.x) {
            const int t = idx / g.wblk, bl = idx - t * g.wblk, b = b0 + bl;
            const int64_t xo = (int64_t)sl.xrow[t] * g.k;
            uint4 raw[8], q[8];
            if (b < g.nb) {
                if (XBF16) {
                    const uint4 *src = (const uint4 *)((const uint16_t *)x + xo + (int64_t)b * QK);
#pragma unroll
                    for (int i = 0; i < 4; ++i) raw[i] = ld_global16(src + i);
                } else {
                    const uint4 *src = (const uint4 *)((const float *)x + xo + (int64_t)b * QK);
#pragma unroll
                    for (int i = 0; i < 8; ++i) raw[i] = ld_global16(src + i);
                }
                stage_block<XBF16, DOT>(raw, q);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < QPB; ++i) xs[(t * QPB + i) * g.wblk + bl] = q[i];
        }
    }
};

// The NVFP4 tensor scale (one fp32 in the packed trailer), 1 for the other
// formats; applied to the row totals.
template <int FMT>
__device__ __forceinline__ float tensor_scale(const Geom &g)
{
    if (FMT == QG_NVFP4) return *(const QG_GLOBAL float *)(g.w + g.tsoff);
    return 1.0f;
}

// Slot -> staged activation row map of the dense product: slot t reads row t.
struct IdMap {
    __device__ __forceinline__ int operator()(int t) const { return t; }
    __device__ __forceinline__ int count() const { return QG_MAX_M; }
};

// Steps per batch (loads in flight per lane before the first use).
template <int FMT, bool DOT> struct Batch { static constexpr int U = (FMT == QG_Q8_0 || is_kq(FMT) || !DOT) ? 4 : 8; };

// Per-lane extras of a K-quant batch: the row's super-block word of each
// step, and for Q6_K the record's high code bits.
template <int FMT, int U> struct KqRegs {};
template <int U> struct KqRegs<QG_Q4_K, U> { uint32_t sw[U]; };
template <int U> struct KqRegs<QG_Q6_K, U> { uint32_t sw[U]; uint2 hh[U]; };

// Where a K-quant lane finds them: its tile's high-bits stream and its row's
// super-block words.
struct KqPtr {
    const uint8_t *ht = nullptr;
    const uint8_t *sbrow = nullptr;
};

__device__ __forceinline__ KqPtr kq_ptr(const Geom &g, int tl, int rl)
{
    KqPtr p;
    p.ht = g.w + g.hoff + (int64_t)tl * g.htb;
    p.sbrow = g.w + g.sboff + ((int64_t)tl * g.R + (rl >> g.lsh)) * g.nsb * 4;
    return p;
}

__device__ __forceinline__ uint2 ld_stream8(const uint8_t *p)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load((const QG_GLOBAL u32x2 *)p);
    return make_uint2(v.x, v.y);
}

template <int FMT, bool XBF16, bool DOT, int M, int UB = Batch<FMT, DOT>::U>
struct Engine {
    static constexpr int P = FMT == QG_Q8_0 ? 2 : 1;
    static constexpr int U = UB;
    static constexpr int QPB = x_quads(FMT, DOT);

    // Scales stay in their stored width until step() widens them: widened at
    // the load, the compiler placed the widening (and so a wait for the whole
    // batch) ahead of the next batch's loads.
    using ScaleT = std::conditional_t<FMT == QG_MXFP4, uint8_t, uint16_t>;
    static constexpr bool KQ = is_kq(FMT);
    struct Regs : KqRegs<FMT, U> {
        uint4 c[U][P];
        ScaleT s[U];
    };

    // Issues the loads of `cnt` (>= 1) steps jfirst, jfirst+KS, ...  Every call
    // issues exactly U*(P+1) loads: steps past cnt repeat the last one (a cache
    // hit, never used).  The fixed count keeps the compiler's vmcnt waits exact,
    // so a batch in flight overlaps the compute of the previous one.
    static __device__ __forceinline__ void load(const Geom &g, const uint8_t *ct, const uint8_t *st, int lane,
                                                int jfirst, int cnt, int KS, Regs &r, const KqPtr &kp = KqPtr{})
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = jfirst + min(u, cnt - 1) * KS;
            const uint8_t *cp = ct + (int64_t)j * (P * 1024) + lane * 16;
#pragma unroll
            for (int h = 0; h < P; ++h) r.c[u][h] = ld_stream16(cp + h * 1024);
            if (FMT == QG_MXFP4)
                r.s[u] = ld_stream_u8(st + (int64_t)j * 64 + lane);
            else
                r.s[u] = ld_stream_u16((const uint16_t *)st + (int64_t)j * 64 + lane);
            if constexpr (KQ) {
                // the word of the record's super-block (padding steps repeat the row's last)
                const int sbi = min((j * g.L + (lane & (g.L - 1))) >> 3, g.nsb - 1);
                r.sw[u] = *(const QG_GLOBAL uint32_t *)(kp.sbrow + sbi * 4);
                if constexpr (FMT == QG_Q6_K) r.hh[u] = ld_stream8(kp.ht + (int64_t)j * 512 + lane * 8);
            }
        }
    }

    // K-quant record: its 32 weights formed exactly, then their products.
    // Q4_K: w = d sc q - dmin m, rounded once (fma of exact fp32 factors).
    // Q6_K: the integer q - 32 (exact), summed against x per 16 elements,
    // each sum scaled by d sc (exact in fp32).
    template <typename XMap = IdMap>
    static __device__ __forceinline__ void step_kq(const Geom &g, const Regs &r, int u, const uint4 *xs, int bl,
                                                   float acc[M], const XMap &xm = XMap())
    {
        const uint4 c = r.c[u][0];
        const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
        const uint32_t sbits = r.s[u], swd = r.sw[u];
        if constexpr (FMT == QG_Q4_K) {
            const float D = f16_bits_to_f32(swd & 0xFFFF) * (float)(sbits & 63);
            const float Mn = -(f16_bits_to_f32(swd >> 16) * (float)((sbits >> 8) & 63));
            float wv[32];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float v[8];
                q4_unpack8(cw[a], v);           // (q - 8) / 16, exact
#pragma unroll
                for (int e = 0; e < 8; ++e) wv[8 * a + e] = __builtin_fmaf(D, __builtin_fmaf(16.0f, v[e], 8.0f), Mn);
            }
#pragma unroll
            for (int t = 0; t < M; ++t) {
                if (t >= xm.count()) break;
                float s = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 xq = __builtin_bit_cast(float4, xs[(xm(t) * 8 + i) * g.wblk + bl]);
                    s = __builtin_fmaf(wv[4 * i], xq.x, s);
                    s = __builtin_fmaf(wv[4 * i + 1], xq.y, s);
                    s = __builtin_fmaf(wv[4 * i + 2], xq.z, s);
                    s = __builtin_fmaf(wv[4 * i + 3], xq.w, s);
                }
                acc[t] += s;
            }
        } else {
            const float d = f16_bits_to_f32(swd & 0xFFFF);
            const float Da = d * (float)(int8_t)(sbits & 0xFF), Db = d * (float)(int8_t)(sbits >> 8);
            const uint32_t hw[2] = {r.hh[u].x, r.hh[u].y};
            float dv[32];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int f = 2 * (a & 1) + e;
                    const uint32_t H = hw[a >> 1];
                    const uint32_t hp = f == 0 ? H << 4 : f == 1 ? H << 2 : f == 2 ? H : H >> 2;
                    uint32_t Q = ((cw[a] >> (4 * e)) & 0x0F0F0F0Fu) | (hp & 0x30303030u);
                    const uint32_t sg = Q & 0x20202020u;      // bytes: 6-bit two's complement -> int8
                    Q |= (sg << 1) | (sg << 2);
#pragma unroll
                    for (int b = 0; b < 4; ++b) dv[8 * a + 4 * e + b] = i8_at(Q, b);
                }
            }
            if constexpr (DOT) {
                // bf16 activations: q - 32 is exact in bf16, two weights per dot2
                bf16x2_t pr[16];
#pragma unroll
                for (int p = 0; p < 16; ++p) pr[p] = pk_bf16(dv[2 * p], dv[2 * p + 1]);
#pragma unroll
                for (int t = 0; t < M; ++t) {
                    if (t >= xm.count()) break;
                    float sh[2] = {0.0f, 0.0f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 xq = xs[(xm(t) * 4 + i) * g.wblk + bl];
                        float &s = sh[i >> 1];
                        s = dot2(pr[4 * i], u32_as_bf16x2(xq.x), s);
                        s = dot2(pr[4 * i + 1], u32_as_bf16x2(xq.y), s);
                        s = dot2(pr[4 * i + 2], u32_as_bf16x2(xq.z), s);
                        s = dot2(pr[4 * i + 3], u32_as_bf16x2(xq.w), s);
                    }
                    acc[t] = __builtin_fmaf(Db, sh[1], __builtin_fmaf(Da, sh[0], acc[t]));
                }
            } else {
#pragma unroll
                for (int t = 0; t < M; ++t) {
                    if (t >= xm.count()) break;
                    float sh[2] = {0.0f, 0.0f};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float4 xq = __builtin_bit_cast(float4, xs[(xm(t) * 8 + i) * g.wblk + bl]);
                        float &s = sh[i >> 2];
                        s = __builtin_fmaf(dv[4 * i], xq.x, s);
                        s = __builtin_fmaf(dv[4 * i + 1], xq.y, s);
                        s = __builtin_fmaf(dv[4 * i + 2], xq.z, s);
                        s = __builtin_fmaf(dv[4 * i + 3], xq.w, s);
                    }
                    acc[t] = __builtin_fmaf(Db, sh[1], __builtin_fmaf(Da, sh[0], acc[t]));
                }
            }
        }
    }

    // Adds the contributions of one step (block b of this lane's row) to acc.
    // Slot t reads staged activation row xm(t) (the identity for the dense
    // product); slots t >= xm.count() are skipped.
    template <typename XMap = IdMap>
    static __device__ __forceinline__ void step(const Geom &g, const uint4 *c, uint32_t sbits, const uint4 *xs, int bl,
                                                float acc[M], const XMap &xm = XMap())
    {
        if (FMT == QG_Q8_0) {
            const float d = f16_bits_to_f32(sbits);
            const uint32_t cw[8] = {c[0].x, c[0].y, c[0].z, c[0].w, c[1].x, c[1].y, c[1].z, c[1].w};
#pragma unroll
            for (int t = 0; t < M; ++t) {
                if (t >= xm.count()) break;
                float s = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float4 xq = __builtin_bit_cast(float4, xs[(xm(t) * 8 + i) * g.wblk + bl]);
                    s = __builtin_fmaf(i8_at(cw[i], 0), xq.x, s);
                    s = __builtin_fmaf(i8_at(cw[i], 1), xq.y, s);
                    s = __builtin_fmaf(i8_at(cw[i], 2), xq.z, s);
                    s = __builtin_fmaf(i8_at(cw[i], 3), xq.w, s);
                }
                acc[t] = __builtin_fmaf(d, s, acc[t]);
            }
        } else if (FMT == QG_Q4_0) {
            const float d = q4_scale(sbits);
            const uint32_t cw[4] = {c[0].x, c[0].y, c[0].z, c[0].w};
            float v[4][8];          // v[i][e]: element 8i + e, (q - 8) / 16
#pragma unroll
            for (int i = 0; i < 4; ++i) q4_unpack8(cw[i], v[i]);
            if (DOT) {
                bf16x2_t pr[16];
#pragma unroll
                for (int p = 0; p < 16; ++p) pr[p] = pk_bf16(v[p >> 2][2 * (p & 3)], v[p >> 2][2 * (p & 3) + 1]);
#pragma unroll
                for (int t = 0; t < M; ++t) {
                    if (t >= xm.count()) break;
                    float s = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 xq = xs[(xm(t) * 4 + i) * g.wblk + bl];
                        s = dot2(pr[4 * i + 0], u32_as_bf16x2(xq.x), s);
                        s = dot2(pr[4 * i + 1], u32_as_bf16x2(xq.y), s);
                        s = dot2(pr[4 * i + 2], u32_as_bf16x2(xq.z), s);
                        s = dot2(pr[4 * i + 3], u32_as_bf16x2(xq.w), s);
                    }
                    acc[t] = __builtin_fmaf(d, s, acc[t]);
                }
            } else {
#pragma unroll
                for (int t = 0; t < M; ++t) {
                    if (t >= xm.count()) break;
                    float s = 0.0f;
#pragma unroll
                    for (int qd = 0; qd < 8; ++qd) {
                        const float4 xq = __builtin_bit_cast(float4, xs[(xm(t) * 8 + qd) * g.wblk + bl]);
                        s = __builtin_fmaf(v[qd >> 1][4 * (qd & 1) + 0], xq.x, s);
                        s = __builtin_fmaf(v[qd >> 1][4 * (qd & 1) + 1], xq.y, s);
                        s = __builtin_fmaf(v[qd >> 1][4 * (qd & 1) + 2], xq.z, s);
                        s = __builtin_fmaf(v[qd >> 1][4 * (qd & 1) + 3], xq.w, s);
                    }
                    acc[t] = __builtin_fmaf(d, s, acc[t]);
                }
            }
        } else if (FMT == QG_NVFP4) {
            // two 16-weight blocks: dwords 0-1 with the first E4M3 scale, 2-3
            // with the second (the tensor scale is applied to the row totals)
            const float s0 = e4m3_to_f32(sbits & 0xFF), s1 = e4m3_to_f32(sbits >> 8);
            const uint32_t cw[4] = {c[0].x, c[0].y, c[0].z, c[0].w};
            if (DOT) {
                bf16x2_t pr[4][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i][0] = fp4_pair_bf16<0>(cw[i]);
                    pr[i][1] = fp4_pair_bf16<1>(cw[i]);
                    pr[i][2] = fp4_pair_bf16<2>(cw[i]);
                    pr[i][3] = fp4_pair_bf16<3>(cw[i]);
                }
#pragma unroll
                for (int t = 0; t < M; ++t) {
                    if (t >= xm.count()) break;
                    float sh[2] = {0.0f, 0.0f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 xq = xs[(xm(t) * 4 + i) * g.wblk + bl];
                        float &s = sh[i >> 1];
                        s = dot2(pr[i][0], u32_as_bf16x2(xq.x), s);
                        s = dot2(pr[i][1], u32_as_bf16x2(xq.y), s);
                        s = dot2(pr[i][2], u32_as_bf16x2(xq.z), s);
                        s = dot2(pr[i][3], u32_as_bf16x2(xq.w), s);
                    }
                    acc[t] = __builtin_fmaf(s1, sh[1], __builtin_fmaf(s0, sh[0], acc[t]));
                }
            } else {
                f32x2_t pr[4][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i][0] = fp4_pair_f32<0>(cw[i]);
                    pr[i][1] = fp4_pair_f32<1>(cw[i]);
                    pr[i][2] = fp4_pair_f32<2>(cw[i]);
                    pr[i][3] = fp4_pair_f32<3>(cw[i]);
                }
#pragma unroll
                for (int t = 0; t < M; ++t) {
                    if (t >= xm.count()) break;
                    float sh[2] = {0.0f, 0.0f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float4 xa = __builtin_bit_cast(float4, xs[(xm(t) * 8 + 2 * i) * g.wblk + bl]);
                        const float4 xb = __builtin_bit_cast(float4, xs[(xm(t) * 8 + 2 * i + 1) * g.wblk + bl]);
                        float &s = sh[i >> 1];
                        s = __builtin_fmaf(pr[i][0].x, xa.x, s);
                        s = __builtin_fmaf(pr[i][0].y, xa.y, s);
                        s = __builtin_fmaf(pr[i][1].x, xa.z, s);
                        s = __builtin_fmaf(pr[i][1].y, xa.w, s);
                        s = __builtin_fmaf(pr[i][2].x, xb.x, s);
                        s = __builtin_fmaf(pr[i][2].y, xb.y, s);
                        s = __builtin_fmaf(pr[i][3].x, xb.z, s);
                        s = __builtin_fmaf(pr[i][3].y, xb.w, s);
                    }
                    acc[t] = __builtin_fmaf(s1, sh[1], __builtin_fmaf(s0, sh[0], acc[t]));
                }
            }
        } else {
            const float sc = e8m0_to_f32(sbits);
            const uint32_t cw[4] = {c[0].x, c[0].y, c[0].z, c[0].w};
            if (DOT) {
                bf16x2_t pr[4][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i][0] = fp4_pair_bf16<0>(cw[i]);
                    pr[i][1] = fp4_pair_bf16<1>(cw[i]);
                    pr[i][2] = fp4_pair_bf16<2>(cw[i]);
                    pr[i][3] = fp4_pair_bf16<3>(cw[i]);
                }
#pragma unroll
                for (int t = 0; t < M; ++t) {
                    if (t >= xm.count()) break;
                    float s = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 xq = xs[(xm(t) * 4 + i) * g.wblk + bl];
                        s = dot2(pr[i][0], u32_as_bf16x2(xq.x), s);
                        s = dot2(pr[i][1], u32_as_bf16x2(xq.y), s);
                        s = dot2(pr[i][2], u32_as_bf16x2(xq.z), s);
                        s = dot2(pr[i][3], u32_as_bf16x2(xq.w), s);
                    }
                    acc[t] = __builtin_fmaf(sc, s, acc[t]);
                }
            } else {
                f32x2_t pr[4][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pr[i][0] = fp4_pair_f32<0>(cw[i]);
                    pr[i][1] = fp4_pair_f32<1>(cw[i]);
                    pr[i][2] = fp4_pair_f32<2>(cw[i]);
                    pr[i][3] = fp4_pair_f32<3>(cw[i]);
                }
#pragma unroll
                for (int t = 0; t < M; ++t) {
                    if (t >= xm.count()) break;
                    float s = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float4 xa = __builtin_bit_cast(float4, xs[(xm(t) * 8 + 2 * i) * g.wblk + bl]);
                        const float4 xb = __builtin_bit_cast(float4, xs[(xm(t) * 8 + 2 * i + 1) * g.wblk + bl]);
                        s = __builtin_fmaf(pr[i][0].x, xa.x, s);
                        s = __builtin_fmaf(pr[i][0].y, xa.y, s);
                        s = __builtin_fmaf(pr[i][1].x, xa.z, s);
                        s = __builtin_fmaf(pr[i][1].y, xa.w, s);
                        s = __builtin_fmaf(pr[i][2].x, xb.x, s);
                        s = __builtin_fmaf(pr[i][2].y, xb.y, s);
                        s = __builtin_fmaf(pr[i][3].x, xb.z, s);
                        s = __builtin_fmaf(pr[i][3].y, xb.w, s);
                    }
                    acc[t] = __builtin_fmaf(sc, s, acc[t]);
                }
            }
        }
    }

    template <typename XMap = IdMap>
    static __device__ __forceinline__ void compute(const Geom &g, const Regs &r, int cnt, int jfirst, int KS,
                                                   int slot, int b0, const uint4 *xs, float acc[M],
                                                   const XMap &xm = XMap())
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (u < cnt) {
                const int j = jfirst + u * KS;
                const int bl = j * g.L + slot - b0;
                if constexpr (KQ)
                    step_kq(g, r, u, xs, bl, acc, xm);
                else
                    step(g, r.c[u], r.s[u], xs, bl, acc, xm);
            }
        }
        consume(r);
    }

    // Marks every register of a batch as read, those of steps past cnt too.
    // Otherwise the compiler, reusing such a register later, cannot tell
    // which load it waits for and waits for all of them, the next batch's
    // included, which serialises the batches.  The loads past cnt repeat a
    // step already read, so waiting for them here costs nothing.
    static __device__ __forceinline__ void consume(const Regs &r)
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            asm volatile("" ::"v"((uint32_t)r.s[u]));
#pragma unroll
            for (int h = 0; h < P; ++h) asm volatile("" ::"v"(r.c[u][h].x), "v"(r.c[u][h].y), "v"(r.c[u][h].z), "v"(r.c[u][h].w));
            if constexpr (KQ) asm volatile("" ::"v"(r.sw[u]));
            if constexpr (FMT == QG_Q6_K) asm volatile("" ::"v"(r.hh[u].x), "v"(r.hh[u].y));
        }
    }

    // One pass over tile `tile` (or none if tile >= tiles) for this wave; the
    // whole workgroup calls it together (it contains barriers when staging).
    // Returns the per-lane partial sums (before the KS and L reductions).
    static __device__ __forceinline__ void pass(const Geom &g, const void *x, const Slots &sl, int tile, bool &staged,
                                                uint4 *xs, float acc[M])
    {
        XStage<XBF16, DOT> st;
        pass_st(g, x, sl, tile, staged, xs, acc, st);
    }

    // The same with a given stager: an object whose run<M, FMT>(g, x, sl, w,
    // xs) fills window w's staged activations in this engine's form; the
    // whole workgroup calls it between two barriers.
    template <class ST>
    static __device__ __forceinline__ void pass_st(const Geom &g, const void *x, const Slots &sl, int tile, bool &staged,
                                                   uint4 *xs, float acc[M], ST &stg)
    {
        const bool active = tile < g.tiles;
        // inactive waves load (and ignore) tile 0, step 0, so that loads stay unconditional
        const int tl = active ? tile : 0;
        KqPtr kp;
        if constexpr (KQ) kp = kq_ptr(g, tl, threadIdx.x & 63);
        pass_core(g, x, sl, g.w + (int64_t)tl * g.ctb, g.w + g.soff + (int64_t)tl * g.stb, threadIdx.x & 63, active,
                  staged, xs, acc, stg, kp);
    }

    // The pass with the lane's own tile bases (ct, st) and record lane rl:
    // the lane reads 16-byte record rl of each step of that tile (its row
    // rl / L, block rl % L).  With rl = the lane, a whole tile per wave.
    // Requires rl % L == lane % L (the staged activations are indexed by it).
    template <class ST>
    static __device__ __forceinline__ void pass_core(const Geom &g, const void *x, const Slots &sl, const uint8_t *ct,
                                                     const uint8_t *st, int rl, bool active, bool &staged, uint4 *xs,
                                                     float acc[M], ST &stg, const KqPtr &kp = KqPtr{})
    {
        const int lane = rl, wave = threadIdx.x >> 6;
        const int KS = g.KS, kpart = wave & (KS - 1);
        const int slot = rl & (g.L - 1);
#pragma unroll
        for (int t = 0; t < M; ++t) acc[t] = 0.0f;
        for (int w = 0; w < g.nwin; ++w) {
            const int j0 = w * g.SW;
            const int j1 = min(g.S, j0 + g.SW);
            const int jf = j0 + kpart;      // SW is a multiple of KS
            const int nsteps = (active && jf < j1) ? (j1 - jf + KS - 1) / KS : 0;
            const int jlast = nsteps > 0 ? jf + (nsteps - 1) * KS : 0;
            Regs ra, rb;
            load(g, ct, st, lane, nsteps > 0 ? jf : 0, max(1, min(nsteps, U)), KS, ra, kp);
            if (g.nwin > 1 || !staged) {
                __syncthreads();
                stg.template run<M, FMT>(g, x, sl, w, xs);
                __syncthreads();
                staged = true;
            }
            const int b0 = j0 * g.L;
            int done = 0;
            while (done < nsteps) {
                const int cA = min(nsteps - done, U);
                const int rB = nsteps - done - cA;
                load(g, ct, st, lane, rB > 0 ? jf + (done + cA) * KS : jlast, rB > 0 ? min(rB, U) : 1, KS, rb, kp);
                compute(g, ra, cA, jf + done * KS, KS, slot, b0, xs, acc);
                done += cA;
                if (done >= nsteps) break;
                const int cB = min(nsteps - done, U);
                const int rA = nsteps - done - cB;
                load(g, ct, st, lane, rA > 0 ? jf + (done + cB) * KS : jlast, rA > 0 ? min(rA, U) : 1, KS, ra, kp);
                compute(g, rb, cB, jf + done * KS, KS, slot, b0, xs, acc);
                done += cB;
            }
        }
    }
};

// Sums the KS per-wave partials (fixed order) and the L lanes of each row.
// Must be called by the whole workgroup.  Afterwards every lane of a row in a
// wave with kpart == 0 holds that row's totals.
template <int M>
__device__ __forceinline__ void reduce_partials(const Geom &g, float *red, float acc[M])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kpart = wave & (g.KS - 1);
    if (g.KS > 1) {
#pragma unroll
        for (int t = 0; t < M; ++t) red[(wave * M + t) * 64 + lane] = acc[t];
        __syncthreads();
        if (kpart == 0) {
            for (int q = 1; q < g.KS; ++q)
#pragma unroll
                for (int t = 0; t < M; ++t) acc[t] += red[((wave + q) * M + t) * 64 + lane];
        }
        __syncthreads();
    }
    for (int off = 1; off < g.L; off <<= 1) {
#pragma unroll
        for (int t = 0; t < M; ++t) acc[t] += __shfl_xor(acc[t], off, 64);
    }
}

inline __host__ __device__ size_t lds_bytes(int M, bool dot, int fmt, int wblk)
{
    size_t b = (size_t)M * x_quads(fmt, dot) * wblk * 16;
    b += (size_t)WAVES * M * 64 * 4;
    return b;
}

template <int FMT, bool XBF16, bool DOT, int M>
__global__ __launch_bounds__(TPB) void k_dense(Geom g, const void *__restrict__ x, float *__restrict__ y)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int QPB = x_quads(FMT, DOT);
    uint4 *xs = (uint4 *)smem;
    float *red = (float *)(smem + (size_t)M * QPB * g.wblk * 16);
    __shared__ int32_t s_rows[QG_MAX_M];
    if (threadIdx.x < QG_MAX_M) s_rows[threadIdx.x] = threadIdx.x;   // read only after the staging barrier
    Slots sl{s_rows, s_rows};
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tsub = wave >> g.ksh, kpart = wave & (g.KS - 1);
    const int rsub = lane >> g.lsh, slot = lane & (g.L - 1);
    bool staged = false;
    for (int grp = blockIdx.x; grp < g.ngroups; grp += gridDim.x) {
        const int tile = grp * g.tpi + tsub;
        float acc[M];
        Engine<FMT, XBF16, DOT, M>::pass(g, x, sl, tile, staged, xs, acc);
        reduce_partials<M>(g, red, acc);
        const int64_t row = (int64_t)tile * g.R + rsub;
        if (kpart == 0 && tile < g.tiles && row < g.n) {
            const float ts = tensor_scale<FMT>(g);
#pragma unroll
            for (int t = 0; t < M; ++t)
                if ((t & (g.L - 1)) == slot) y[(int64_t)sl.yrow[t] * g.n + row] = FMT == QG_NVFP4 ? acc[t] * ts : acc[t];
        }
    }
}

// ------------------------------------------------- one-batch dense product
// For matrices whose per-wave share of a tile is short (at most U steps, one
// activation window, every activation block of the call held by the
// workgroup's threads at ONE_XR blocks each), each wave issues all of its
// weight loads at once, directly after the loads of its threads' activation
// blocks.  HBM then has the whole matrix requested from the start of the
// launch (the batched pass above requests one batch ahead of the arithmetic,
// and its second batch only after the staging barrier), the staging of x
// overlaps the weight stream, and the arithmetic of each step follows the
// arrival of its data.  A wave's loads complete in issue order, so the
// activations, needed first, are issued first.  Same arithmetic, reduction
// and output as k_dense.
constexpr int ONE_XR = 3;
constexpr int ONE_MAX_U = 20;
constexpr int QG_CUS = 256;             // compute units of the MI355X / MI350X

// Waves per SIMD each variant is compiled to allow (its register budget):
// a workgroup has one wave per SIMD, so a compute unit holds this many.
__host__ __device__ constexpr int one_waves(int fmt, bool xbf16, int u)
{
    return (!xbf16 || is_kq(fmt)) ? 2 : fmt == QG_Q8_0 ? (u <= 8 ? 3 : 2) : u <= 8 ? 4 : u <= 12 ? 3 : 2;
}

// The workgroup's one-batch pass over its tile group (grid = ngroups): on
// return acc holds what reduce_partials leaves (row totals in the lanes of
// waves with kpart == 0).
template <int FMT, bool XBF16, bool DOT, int M, int U>
__device__ __forceinline__ void dense_one_pass(const Geom &g, const void *__restrict__ x, float acc[M])
{
    extern __shared__ __align__(16) uint8_t smem[];
    using E = Engine<FMT, XBF16, DOT, M, U>;
    constexpr int QPB = x_quads(FMT, DOT);
    constexpr int XQ = XBF16 ? 4 : 8;       // 16-byte loads per activation block
    uint4 *xs = (uint4 *)smem;
    float *red = (float *)(smem + (size_t)M * QPB * g.wblk * 16);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tsub = wave >> g.ksh, kpart = wave & (g.KS - 1);
    const int slot = lane & (g.L - 1);
    const int tile = blockIdx.x * g.tpi + tsub;
    const int total = M * g.wblk;

    // activation blocks idx = thread + r * blockDim: token idx / wblk, block idx % wblk
    // (blocks past the row or past the call load block 0 of token 0 and stage zeros)
    uint4 raw[ONE_XR][8];
#pragma unroll
    for (int r = 0; r < ONE_XR; ++r) {
        const int idx = threadIdx.x + r * (int)blockDim.x;
        const int t = idx / g.wblk, bl = idx - t * g.wblk;
        const bool ok = idx < total && bl < g.nb;
        const int64_t off = ok ? (int64_t)t * g.k + (int64_t)bl * QK : 0;
        const uint4 *src = XBF16 ? (const uint4 *)((const uint16_t *)x + off) : (const uint4 *)((const float *)x + off);
#pragma unroll
        for (int i = 0; i < XQ; ++i) raw[r][i] = ld_global16(src + i);
#pragma unroll
        for (int i = XQ; i < 8; ++i) raw[r][i] = make_uint4(0, 0, 0, 0);
    }

    // every weight step of this wave: steps kpart, kpart + KS, ... of its tile
    const bool active = tile < g.tiles;
    const int tl = active ? tile : 0;
    const uint8_t *ct = g.w + (int64_t)tl * g.ctb;
    const uint8_t *st = g.w + g.soff + (int64_t)tl * g.stb;
    const int nsteps = (active && kpart < g.S) ? (g.S - kpart + g.KS - 1) / g.KS : 0;
    KqPtr kp;
    if constexpr (is_kq(FMT)) kp = kq_ptr(g, tl, lane);
    typename E::Regs rw;
    E::load(g, ct, st, lane, nsteps > 0 ? kpart : 0, max(1, nsteps), g.KS, rw, kp);

#pragma unroll
    for (int r = 0; r < ONE_XR; ++r) {
        const int idx = threadIdx.x + r * (int)blockDim.x;
        if (idx < total) {
            const int t = idx / g.wblk, bl = idx - t * g.wblk;
            uint4 q[8];
            if (bl < g.nb) {
                stage_block<XBF16, DOT>(raw[r], q);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < QPB; ++i) xs[(t * QPB + i) * g.wblk + bl] = q[i];
        }
    }
    __syncthreads();

#pragma unroll
    for (int t = 0; t < M; ++t) acc[t] = 0.0f;
    E::compute(g, rw, nsteps, kpart, g.KS, slot, 0, xs, acc);
    reduce_partials<M>(g, red, acc);
}

template <int FMT, bool XBF16, bool DOT, int M, int U>
__global__ __launch_bounds__(TPB, one_waves(FMT, XBF16, U)) void k_dense_one(Geom g, const void *__restrict__ x,
                                                                              float *__restrict__ y)
{
    float acc[M];
    dense_one_pass<FMT, XBF16, DOT, M, U>(g, x, acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tile = blockIdx.x * g.tpi + (wave >> g.ksh);
    const int64_t row = (int64_t)tile * g.R + (lane >> g.lsh);
    if ((wave & (g.KS - 1)) == 0 && tile < g.tiles && row < g.n) {
        const float ts = tensor_scale<FMT>(g);
#pragma unroll
        for (int t = 0; t < M; ++t)
            if ((t & (g.L - 1)) == (lane & (g.L - 1))) y[(int64_t)t * g.n + row] = FMT == QG_NVFP4 ? acc[t] * ts : acc[t];
    }
}

// ------------------------------------------------------------------- MoE
// Distinct selected experts, ascending, computed by every workgroup from the
// device-resident ids (no host round trip).  s_ids receives the ids,
// list[i] for i < *count the distinct valid ones.  nslots <= 64.
__device__ inline void distinct_experts(const int32_t *__restrict__ ids, int nslots, int n_experts, int *s_ids,
                                        int *list, int *count)
{
    __shared__ int s_first[64];
    const int t = threadIdx.x;
    if (t < nslots) s_ids[t] = ids[t];
    __syncthreads();
    if (t < nslots) {
        const int e = s_ids[t];
        bool first = e >= 0 && e < n_experts;
        for (int q = 0; q < t && first; ++q) first = s_ids[q] != e;
        s_first[t] = first ? 1 : 0;
    }
    __syncthreads();
    if (t < nslots && s_first[t]) {
        const int e = s_ids[t];
        int rank = 0;
        for (int q = 0; q < nslots; ++q) rank += (s_first[q] && s_ids[q] < e) ? 1 : 0;
        list[rank] = e;
    }
    if (t < 64) {
        const uint64_t mask = __ballot(t < nslots && s_first[t]);
        if (t == 0) *count = __popcll(mask);
    }
    __syncthreads();
}

// Slots (t * top_k + j) that chose expert e, in increasing order, by one
// wave with a ballot over the ids in LDS; the caller synchronises.
__device__ __forceinline__ void expert_slots(int e, int nslots, const int *s_ids, int *s_slots, int *s_nsl)
{
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const bool match = lane < nslots && s_ids[lane] == e;
        const uint64_t mask = __ballot(match);
        if (match) s_slots[__popcll(mask & ((1ull << lane) - 1))] = lane;
        if (lane == 0) *s_nsl = __popcll(mask);
    }
}

struct MoeArgs {
    const uint8_t *experts;
    int64_t expert_bytes;
    const int32_t *ids;
    const float *gw;
    int32_t n_experts, m, top_k;
    int32_t isplit;              // streaming kernel: waves that share a tile, splitting its items
};

// Runs the dense passes of this workgroup over expert `e` for `cnt` slots
// (1 <= cnt <= 8), dispatched to the engine instantiated for that count.
template <int FMT, bool XBF16, bool DOT, int M>
__device__ __forceinline__ void moe_tiles(Geom g, const void *x, const Slots sl, uint4 *xs, float *red, int grp,
                          float *part_out /* [M][tpi*R] or null */, float *y)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tsub = wave >> g.ksh, kpart = wave & (g.KS - 1);
    const int rsub = lane >> g.lsh, slot = lane & (g.L - 1);
    bool staged = false;
    const int tile = grp * g.tpi + tsub;
    float acc[M];
    Engine<FMT, XBF16, DOT, M>::pass(g, x, sl, tile, staged, xs, acc);
    reduce_partials<M>(g, red, acc);
    const int64_t row = (int64_t)tile * g.R + rsub;
    if (kpart == 0 && tile < g.tiles && row < g.n) {
        const int rl = tsub * g.R + rsub;
#pragma unroll
        for (int t = 0; t < M; ++t) {
            if ((t & (g.L - 1)) == slot) {
                if (part_out)
                    part_out[t * (g.tpi * g.R) + rl] = acc[t];
                else
                    y[(int64_t)sl.yrow[t] * g.n + row] = acc[t];
            }
        }
    }
}

template <int FMT, bool XBF16, bool DOT>
__device__ __forceinline__ void moe_dispatch(int cnt, Geom g, const void *x, const Slots sl, uint4 *xs, float *red,
                             int grp, float *part_out, float *y)
{
    switch (cnt) {
    case 1: moe_tiles<FMT, XBF16, DOT, 1>(g, x, sl, xs, red, grp, part_out, y); break;
    case 2: moe_tiles<FMT, XBF16, DOT, 2>(g, x, sl, xs, red, grp, part_out, y); break;
    case 3: moe_tiles<FMT, XBF16, DOT, 3>(g, x, sl, xs, red, grp, part_out, y); break;
    case 4: moe_tiles<FMT, XBF16, DOT, 4>(g, x, sl, xs, red, grp, part_out, y); break;
    case 5: moe_tiles<FMT, XBF16, DOT, 5>(g, x, sl, xs, red, grp, part_out, y); break;
    case 6: moe_tiles<FMT, XBF16, DOT, 6>(g, x, sl, xs, red, grp, part_out, y); break;
    case 7: moe_tiles<FMT, XBF16, DOT, 7>(g, x, sl, xs, red, grp, part_out, y); break;
    default: moe_tiles<FMT, XBF16, DOT, 8>(g, x, sl, xs, red, grp, part_out, y); break;
    }
}

// gate_up mode: grid = (row-tile groups, distinct-expert index).
template <int FMT, bool XBF16, bool DOT>
__global__ __launch_bounds__(TPB) void k_moe_gate_up(Geom g, MoeArgs a, const void *__restrict__ x, float *__restrict__ y)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_ids[64];
    __shared__ int s_list[64];
    __shared__ int s_count;
    __shared__ int s_slots[64];
    __shared__ int s_nsl;
    __shared__ int32_t s_xrow[QG_MAX_M], s_yrow[QG_MAX_M];
    const int nslots = a.m * a.top_k;
    distinct_experts(a.ids, nslots, a.n_experts, s_ids, s_list, &s_count);
    if ((int)blockIdx.y >= s_count) return;      // uniform over the workgroup
    const int e = s_list[blockIdx.y];
    expert_slots(e, nslots, s_ids, s_slots, &s_nsl);
    __syncthreads();
    const int nsl = s_nsl;
    constexpr int QPB = x_quads(FMT, DOT);
    uint4 *xs = (uint4 *)smem;
    float *red = (float *)(smem + (size_t)QG_MAX_M * QPB * g.wblk * 16);
    Geom ge = g;
    ge.w = a.experts + (int64_t)e * a.expert_bytes;
    for (int c0 = 0; c0 < nsl; c0 += QG_MAX_M) {
        const int cnt = min(QG_MAX_M, nsl - c0);
        __syncthreads();     // earlier passes are done with the slot map
        if (threadIdx.x < QG_MAX_M) {
            const int s = s_slots[c0 + min((int)threadIdx.x, cnt - 1)];
            s_xrow[threadIdx.x] = s / a.top_k;
            s_yrow[threadIdx.x] = s;
        }
        Slots sl{s_xrow, s_yrow};
        for (int grp = blockIdx.x; grp < g.ngroups; grp += gridDim.x) {
            __syncthreads();
            moe_dispatch<FMT, XBF16, DOT>(cnt, ge, x, sl, xs, red, grp, nullptr, y);
        }
    }
}

// down-combine mode: grid = row-tile groups; each workgroup walks the
// distinct experts in ascending order, keeps the per-slot partial products
// of its rows in LDS and combines them with the router weights in slot order.
template <int FMT, bool XBF16, bool DOT>
__global__ __launch_bounds__(TPB) void k_moe_down(Geom g, MoeArgs a, const void *__restrict__ x, float *__restrict__ y)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int s_ids[64];
    __shared__ int s_list[64];
    __shared__ int s_count;
    __shared__ int s_slots[64];
    __shared__ int s_nsl;
    __shared__ int32_t s_xrow[QG_MAX_M], s_yrow[QG_MAX_M];
    const int nslots = a.m * a.top_k;
    distinct_experts(a.ids, nslots, a.n_experts, s_ids, s_list, &s_count);
    constexpr int QPB = x_quads(FMT, DOT);
    uint4 *xs = (uint4 *)smem;
    float *red = (float *)(smem + (size_t)QG_MAX_M * QPB * g.wblk * 16);
    float *part = red + WAVES * QG_MAX_M * 64;           // [nslots][tpi*R]
    const int rows_pg = g.tpi * g.R;
    for (int grp = blockIdx.x; grp < g.ngroups; grp += gridDim.x) {
        for (int i = threadIdx.x; i < nslots * rows_pg; i += TPB) part[i] = 0.0f;
        for (int ei = 0; ei < s_count; ++ei) {
            const int e = s_list[ei];
            __syncthreads();
            expert_slots(e, nslots, s_ids, s_slots, &s_nsl);
            __syncthreads();
            const int nsl = s_nsl;
            Geom ge = g;
            ge.w = a.experts + (int64_t)e * a.expert_bytes;
            for (int c0 = 0; c0 < nsl; c0 += QG_MAX_M) {
                const int cnt = min(QG_MAX_M, nsl - c0);
                __syncthreads();     // earlier passes are done with the slot map
                if (threadIdx.x < QG_MAX_M) {
                    // x is [m][top_k][k]: slot s reads row s
                    s_xrow[threadIdx.x] = s_slots[c0 + min((int)threadIdx.x, cnt - 1)];
                    s_yrow[threadIdx.x] = 0;
                }
                Slots sl{s_xrow, s_yrow};
                __syncthreads();
                // partial results land in a staging area, then move to part[slot]
                float *tmp = part + nslots * rows_pg;    // [8][rows_pg]
                moe_dispatch<FMT, XBF16, DOT>(cnt, ge, x, sl, xs, red, grp, tmp, nullptr);
                __syncthreads();
                for (int i = threadIdx.x; i < cnt * rows_pg; i += TPB) {
                    const int t = i / rows_pg, rl = i - t * rows_pg;
                    part[s_slots[c0 + t] * rows_pg + rl] = tmp[t * rows_pg + rl];
                }
            }
        }
        __syncthreads();
        // combine: y[t][row] = sum_j w[t][j] * part[t*top_k+j][row], j ascending
        for (int i = threadIdx.x; i < a.m * rows_pg; i += TPB) {
            const int t = i / rows_pg, rl = i - t * rows_pg;
            const int64_t row = (int64_t)grp * rows_pg + rl;
            if (row < g.n) {
                float s = 0.0f;
                for (int j = 0; j < a.top_k; ++j) {
                    const int sidx = t * a.top_k + j;
                    const int e = s_ids[sidx];
                    if (e >= 0 && e < a.n_experts) s = __builtin_fmaf(a.gw[sidx], part[sidx * rows_pg + rl], s);
                }
                y[(int64_t)t * g.n + row] = s;
            }
        }
        __syncthreads();
    }
}


// ------------------------------------------------------------ host plumbing
struct Plan {
    Geom g;
    size_t lds;
    int grid;
    int threads;                 // workgroup size: 64 * (tiles per workgroup) * KS
};

typedef void (*dense_fn)(Geom, const void *, float *);

// Per-format kernel tables (one translation unit each, compiled in parallel).
dense_fn dense_kernel_q8_0(int xt, int m);
dense_fn dense_kernel_q4_0(int xt, int m);
dense_fn dense_kernel_mxfp4(int xt, int m);
dense_fn dense_kernel_nvfp4(int xt, int m);
dense_fn dense_one_kernel_q8_0(int xt, int m, int u);
dense_fn dense_one_kernel_q4_0(int xt, int m, int u);
dense_fn dense_one_kernel_mxfp4(int xt, int m, int u);
dense_fn dense_one_kernel_nvfp4(int xt, int m, int u);
dense_fn dense_kernel_kq(int fmt, int xt, int m);
dense_fn dense_one_kernel_kq(int fmt, int xt, int m, int u);
hipError_t launch_requant_nvfp4(const Layout &lo, const uint8_t *canon_q8_0, uint8_t *packed, hipStream_t s);
hipError_t launch_moe_q8_0(int xt, int mode, const Plan &p, const MoeArgs &a, int maxdistinct, size_t lds,
                           const void *x, float *y, hipStream_t s);
hipError_t launch_moe_q4_0(int xt, int mode, const Plan &p, const MoeArgs &a, int maxdistinct, size_t lds,
                           const void *x, float *y, hipStream_t s);
hipError_t launch_moe_mxfp4(int xt, int mode, const Plan &p, const MoeArgs &a, int maxdistinct, size_t lds,
                            const void *x, float *y, hipStream_t s);

template <int FMT, bool XBF16, bool DOT>
dense_fn pick_dense(int m)
{
    switch (m) {
    case 1: return k_dense<FMT, XBF16, DOT, 1>;
    case 2: return k_dense<FMT, XBF16, DOT, 2>;
    case 3: return k_dense<FMT, XBF16, DOT, 3>;
    case 4: return k_dense<FMT, XBF16, DOT, 4>;
    case 5: return k_dense<FMT, XBF16, DOT, 5>;
    case 6: return k_dense<FMT, XBF16, DOT, 6>;
    case 7: return k_dense<FMT, XBF16, DOT, 7>;
    default: return k_dense<FMT, XBF16, DOT, 8>;
    }
}

// Steps in flight of the one-batch kernel for one token whose waves each
// stream `need` steps, or 0 where the batched pass is faster.  Measured on
// MI355X (graph replay, 36 distinct copies, µs per launch, batched -> one
// batch): Q4_0 6144x2560 7.04 -> 5.91, 2560x4096 5.95 -> 5.03, 19456x2560
// (4 waves per tile) 11.54 -> 10.58, 2560x9728 (19 steps) 9.44 -> 8.69;
// MXFP4 alike.  Q8_0 (twice the bytes and the arithmetic per step) gains
// only on short streams: 2560x4096 (8 steps) 6.27 -> 5.89, while 6144x2560
// (10 steps) 7.04 -> 7.21 and 2560x9728 (19 steps) 10.00 -> 10.65 lose.
// The 4-bit formats use it for co-batches of up to ONE_MAX_M tokens too (the
// vector co-batch range of bf16 activations).
constexpr int ONE_MAX_M = 3;

// Steps in flight of the one-batch kernel for m tokens and `need` steps per
// wave, 0 where it does not apply.  Q8_0 (two 16-byte parts per step) takes
// up to 10 at two waves per SIMD: the 10-step streams of the 2560-column
// decode matrices in one batch (MI355X, 6144x2560: 6.83 -> 6.65 us); 12 spill.
inline int one_batch_u(int fmt, int m, int need)
{
    if (fmt == QG_Q8_0) return m != 1 ? 0 : need <= 8 ? 8 : need <= 10 ? 10 : 0;
    if (is_kq(fmt)) return m == 1 && need <= 8 ? 8 : 0;
    if (m > ONE_MAX_M) return 0;
    return need <= 8 ? 8 : need <= 12 ? 12 : need <= ONE_MAX_U ? ONE_MAX_U : 0;
}

template <int FMT, bool XBF16, bool DOT, int M>
dense_fn pick_dense_one_u(int u)
{
    return u == 8 ? k_dense_one<FMT, XBF16, DOT, M, 8>
                  : u == 12 ? k_dense_one<FMT, XBF16, DOT, M, 12> : k_dense_one<FMT, XBF16, DOT, M, ONE_MAX_U>;
}

// m tokens (1..ONE_MAX_M; Q8_0 one), u steps in flight (one_batch_u).
template <int FMT, bool XBF16, bool DOT>
dense_fn pick_dense_one(int m, int u)
{
    if constexpr (FMT == QG_Q8_0) {
        return u == 10 ? k_dense_one<FMT, XBF16, DOT, 1, 10> : k_dense_one<FMT, XBF16, DOT, 1, 8>;
    } else if constexpr (is_kq(FMT)) {
        return k_dense_one<FMT, XBF16, DOT, 1, 8>;
    } else {
        return m == 1 ? pick_dense_one_u<FMT, XBF16, DOT, 1>(u)
                      : m == 2 ? pick_dense_one_u<FMT, XBF16, DOT, 2>(u) : pick_dense_one_u<FMT, XBF16, DOT, 3>(u);
    }
}

// Workgroups may use more than 64 KiB of LDS on gfx950 (160 KiB per CU);
// larger dynamic allocations are declared to the runtime first.
inline hipError_t allow_lds(const void *fn, size_t bytes)
{
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int FMT, bool XBF16, bool DOT>
hipError_t launch_moe_t(int mode, const Plan &p, const MoeArgs &a, int maxdistinct, size_t lds, const void *x,
                        float *y, hipStream_t s)
{
    const void *fn = mode == QG_MOE_GATE_UP ? (const void *)k_moe_gate_up<FMT, XBF16, DOT>
                                            : (const void *)k_moe_down<FMT, XBF16, DOT>;
    hipError_t e = allow_lds(fn, lds);
    if (e != hipSuccess) return e;
    if (mode == QG_MOE_GATE_UP)
        hipLaunchKernelGGL((k_moe_gate_up<FMT, XBF16, DOT>), dim3(p.grid, maxdistinct), dim3(TPB), lds, s, p.g, a, x, y);
    else
        hipLaunchKernelGGL((k_moe_down<FMT, XBF16, DOT>), dim3(p.grid), dim3(TPB), lds, s, p.g, a, x, y);
    return hipGetLastError();
}

} // namespace qg
