/*
 * qgemv.h -- C ABI of libqgemv.so: block-quantized weight matrix-vector
 * products for MI355X (gfx950).
 *
 * What is computed.  The decode step of an LLM streams every weight matrix
 * once per generated token through a matrix-vector product; decode is bound by
 * memory bandwidth (imp README, "Known limitations": a card with a quarter
 * less bandwidth decodes about a quarter slower).
 * The weights are stored in the block formats the engines serve: Q8_0 and
 * Q4_0 (Imparo README, opening release notes and the M3 Pro benchmark table;
 * imp README, "Features" table, Quantization row) and MXFP4, 4-bit E2M1
 * values with UE8M0 block scales at 4.25 bits per weight (imp release notes,
 * v0.6).
 * The top-k expert variant covers mixture-of-experts layers such as
 * gpt-oss-20b, 32 experts of which 4 serve each token, in MXFP4 (imp README,
 * "Supported models" table), with expert routing read on the device, not copied to the
 * host (imp release notes, v0.7.0 "Known issues": host-side MoE routing is
 * incompatible with graph capture).
 *
 * Canonical block formats (32 weights along K per block, little-endian):
 *   Q8_0  34 B: fp16 scale d, then 32 int8 codes q;              w = d * q
 *   Q4_0  18 B: fp16 scale d, then 16 bytes; byte j holds code j in its low
 *               nibble and code j+16 in its high nibble;          w = d * (q - 8)
 *   MXFP4 17 B: UE8M0 exponent byte E, then 16 bytes with the same nibble
 *               split; each nibble is an E2M1 code c (sign in bit 3);
 *                                                                 w = E2M1(c) * 2^(E-127)
 *   NVFP4  9 B per 16 weights: FP8 E4M3 scale s, then 8 bytes; byte j holds
 *               code j in its low nibble and code j+8 in its high nibble; the
 *               tensor's N * (K/16) blocks are followed by its fp32 scale s_t
 *               (4 bytes);                                        w = E2M1(c) * E4M3(s) * s_t
 *               (the FP4 format of imp's load-time decode cache and sm_120a
 *               GEMV: imp README, "Why this exists" and "Features"; the
 *               definition is the public one, the byte order a reading)
 *   K-quant super-blocks of 256 weights (the GGUF Q4_K / Q6_K formats of the
 *   imp engine's models: imp README, "Features" table, Quantization row; imp
 *   release notes v0.7.0, Q4_K_M; named on the pages, defined publicly):
 *   Q4_K 144 B: fp16 d, fp16 dmin, 12 bytes s of 6-bit scales and mins, 128
 *               code bytes qs.  Sub-block j (weights 32j..32j+31): for j < 4
 *               sc = s[j] & 63, m = s[j+4] & 63; for j >= 4
 *               sc = (s[j+4] & 15) | (s[j-4] >> 6) << 4,
 *               m = (s[j+4] >> 4) | (s[j] >> 6) << 4.  Weight 64c+l (l < 32)
 *               is the low nibble of qs[32c+l], weight 64c+32+l its high nibble;
 *                                                                 w = d * sc * q - dmin * m
 *   Q6_K 210 B: ql[128], qh[64], 16 int8 scales sc, fp16 d.  Weight
 *               128h+32r+l (h < 2, r < 4, l < 32): low 4 bits from
 *               ql[64h+l+32(r&1)] (low nibble if r < 2, else high), high 2
 *               bits (qh[32h+l] >> 2r) & 3, scale sc[8h+2r+l/16];
 *                                                                 w = d * sc * (q - 32)
 * A matrix is N rows (outputs) by K columns (inputs), stored as N * (K/32)
 * canonical blocks (N * (K/16) for NVFP4, N * (K/256) for the K-quants, whose
 * K must be a multiple of 256), row-major.  E = 255 decodes to NaN; E2M1 has
 * no NaN; E4M3 S.1111.111 is NaN.  K-quant scales (d, dmin) must be finite.
 *
 * Packed layout.  The GEMV entry points read weights in a packed layout made
 * once at load time by qg_pack (device) or qg_pack_host (CPU): per tile of
 * R = 64/L rows, each wavefront load instruction reads 1 KiB of codes that is
 * contiguous in memory; scales are a separate stream.  The layout depends only
 * on (fmt, n, k); qg_layout reports it, qg_packed_bytes its size.  Packing is
 * bit-exact: qg_unpack(qg_pack(B)) == B byte for byte.  Keeping a private
 * kernel layout beside the canonical file format follows Imparo, which
 * converts its GateUp weights into a layout of its own at load time (Imparo
 * README, opening release notes); the canonical blocks stay the interchange
 * form, as GGUF is for both engines (imp README, "What is imp").
 * Packed weight pointers (w_packed, w_experts, qg_pack's output, qg_unpack's
 * input) must be 256-byte aligned: every 1 KiB load then covers whole cache
 * lines.
 *
 * Conventions for every entry point below:
 *  - Pointers named as device memory are device memory owned by the caller
 *    (for example torch tensors).  Pointers named as host memory are host
 *    memory.  No entry point frees caller memory.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Device work is enqueued on it and the call returns without waiting.
 *  - Arguments are validated on the host before any HIP call; on error a
 *    status is returned and nothing is enqueued.  A HIP launch failure returns
 *    QG_EHIP.  Faults inside kernels surface at the caller's next
 *    synchronisation, as in HIP.
 *  - Results are deterministic: the same inputs give the same bits (every
 *    reduction has a fixed order).
 *  - Device-resident values are not inspected on the host: expert ids must be
 *    in [0, n_experts); an id outside that range is skipped (its slot
 *    contributes nothing and, in gate_up mode, its output rows are left
 *    unwritten).
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    QG_OK = 0,
    QG_EINVAL = 1,        /* null pointer, non-positive size, k % 32 != 0 (K-quants: k % 256 != 0),
                             m outside [1, 8], bad enum */
    QG_EUNSUPPORTED = 2,  /* valid but outside what the kernels serve (see the limits per call) */
    QG_EALIGN = 3,        /* device pointer misaligned */
    QG_EHIP = 4           /* a HIP runtime call failed */
};

/* Weight formats. */
enum { QG_Q8_0 = 0, QG_Q4_0 = 1, QG_MXFP4 = 2, QG_NVFP4 = 3, QG_Q4_K = 4, QG_Q6_K = 5 };

/* Activation element types: fp32, or bf16 bit patterns (uint16). */
enum { QG_F32 = 0, QG_BF16 = 1 };

/* Expert modes of moe_qgemv_topk. */
enum { QG_MOE_GATE_UP = 0, QG_MOE_DOWN_COMBINE = 1 };

/* Largest co-batch (tokens per call) of the GEMV entry points. */
#define QG_MAX_M 8

/* Largest token count of qgemm. */
#define QG_MAX_GEMM_M 128

/* Kernel families of the dense product (qg_dense_path): the vector code
 * with a few steps in flight per wave, the matrix cores, and the vector code
 * with each wave's whole stream requested at once (one token, short rows). */
enum { QG_PATH_VALU = 0, QG_PATH_MFMA = 1, QG_PATH_VALU_ONE = 2 };

/* Activation of the fused product's epilogue (qgemv_fused). */
enum { QG_ACT_NONE = 0, QG_ACT_SWIGLU = 1 };

/* Description of the packed layout of one n x k matrix. */
typedef struct {
    int32_t fmt;
    int32_t lanes_per_row;      /* L: lanes of a wavefront that share one row */
    int32_t rows_per_tile;      /* R = 64 / L */
    int32_t parts_per_step;     /* 16-byte code loads per lane per step: 2 (Q8_0) or 1 */
    int32_t scale_bytes;        /* 2 (fp16) or 1 (UE8M0) */
    int32_t reserved;
    int64_t n, k;
    int64_t steps;              /* S: blocks per lane per tile = ceil((k/32) / L) */
    int64_t tiles;              /* ceil(n / R) */
    int64_t code_tile_bytes;    /* S * parts * 1024 */
    int64_t scale_tile_bytes;   /* S * 64 * scale_bytes */
    int64_t scale_offset;       /* byte offset of the scale stream = tiles * code_tile_bytes */
    int64_t packed_bytes;       /* total size, rounded up to a multiple of 256 */
    int64_t tensor_scale_offset;  /* NVFP4: byte offset of the fp32 tensor scale (a 256-byte trailer); else 0 */
    int64_t high_offset;          /* Q6_K: byte offset of the stream of high code bits (8 B per record); else 0 */
    int64_t superblock_offset;    /* K-quants: byte offset of the per-row super-block words
                                     (d | dmin << 16, fp16 bits; 4 B each); else 0 */
} qg_layout_t;

/* Human-readable name of a status code (static string). */
const char *qg_status_str(int status);

/* Size in bytes of the packed form of an n x k matrix (a multiple of 256), or
 * -1 if (fmt, n, k) is invalid.  Part of the load-time layout described above
 * (Imparo README, opening release notes: a private weight layout made at load). */
int64_t qg_packed_bytes(int fmt, int64_t n, int64_t k);

/* Fills *out with the packed layout of an n x k matrix.  out: host memory.
 * Returns QG_EINVAL (null out, bad shape) or QG_EUNSUPPORTED (n or k above
 * 2^31 - 1); nothing is written then. */
int qg_layout(int fmt, int64_t n, int64_t k, qg_layout_t *out);

/*
 * Canonical -> packed (and back) on the host: the load-time conversion into
 * the kernels' private layout (Imparo README, opening release notes).
 * canon: host memory, n * (k/32) canonical blocks.  packed: host memory,
 * qg_packed_bytes bytes; every padding byte of the packed form is written as
 * zero.  Unpacking restores the canonical bytes exactly.  Synchronous; status
 * QG_EINVAL for null pointers or a bad shape.
 */
int qg_pack_host(int fmt, const void *canon, int64_t n, int64_t k, void *packed);
int qg_unpack_host(int fmt, const void *packed, int64_t n, int64_t k, void *canon);

/*
 * The same transforms on the device, enqueued on `stream`.  canon, packed:
 * device memory owned by the caller; packed must be 256-byte aligned
 * (QG_EALIGN otherwise).  Bit-identical to the host versions.
 */
int qg_pack(int fmt, const void *canon, int64_t n, int64_t k, void *packed, void *stream);
int qg_unpack(int fmt, const void *packed, int64_t n, int64_t k, void *canon, void *stream);

/*
 * Test aid: decodes a packed matrix to fp32 w[n][k] (device memory, row-major,
 * 4-byte aligned) through the same unpack steps the GEMV kernels use, so the
 * block definitions above (the Q8_0 / Q4_0 rows of the imp README "Features"
 * table and the MXFP4 format of the imp release notes v0.6) can be checked
 * weight by weight.  Every Q8_0, Q4_0 and MXFP4 weight is exact in fp32
 * when it is finite, so the result is comparable bit for bit; an NVFP4
 * weight is E2M1 * E4M3 (exact) times the fp32 tensor scale, rounded once
 * to nearest.  w_packed: 256-byte aligned.
 */
int qg_dequant_f32(int fmt, const void *w_packed, int64_t n, int64_t k, float *w, void *stream);

/*
 * Dense product for a co-batch of m tokens (1 <= m <= 8):
 *     y[t][i] = sum_c W[i][c] * x[t][c]        t < m, i < n
 * w_packed: device, packed layout of (fmt, n, k), 256-byte aligned.
 * x: device, [m][k] row-major, fp32 or bf16 (xt), 16-byte aligned.
 * y: device, fp32 [m][n] row-major, 4-byte aligned, overwritten.
 * Accumulation is fp32; x is used exactly (bf16 -> fp32 is exact).
 * Two kernel families compute it (qg_dense_path says which one a call uses):
 * lane-per-block vector code, and for bf16 co-batches of 2 or more tokens
 * on layouts of at most 8 lanes per row, the matrix cores (one bf16 MFMA per
 * 16 rows x 32-weight block, scales applied in fp32).  Results of the two
 * agree within the rounding of fp32 sums.  For one token (4-bit formats: up
 * to 3) over short rows the vector code requests each wave's whole weight
 * stream at once (same arithmetic, same bits); where it does, it also takes
 * those co-batches.
 * Limits: n, k <= 2^31 - 1 and k % 32 == 0.
 */
int qgemv_q8_0(const void *w_packed, int64_t n, int64_t k, const void *x, int xt, int64_t m,
               float *y, void *stream);
int qgemv_q4_0(const void *w_packed, int64_t n, int64_t k, const void *x, int xt, int64_t m,
               float *y, void *stream);
int qgemv_mxfp4(const void *w_packed, int64_t n, int64_t k, const void *x, int xt, int64_t m,
                float *y, void *stream);

/*
 * The same product for NVFP4 weights (packed by qg_pack from a canonical
 * NVFP4 tensor, or made by qg_requant_q8_0_nvfp4).  Runs the vector kernel
 * family for every m (each 32-weight record carries two block scales); the
 * tensor scale is applied to the row totals.  Limits as qgemv_*.
 */
int qgemv_nvfp4(const void *w_packed, int64_t n, int64_t k, const void *x, int xt, int64_t m,
                float *y, void *stream);

/*
 * The same product for K-quant weights (Q4_K, Q6_K; packed by qg_pack from
 * canonical super-blocks).  The packed form keeps a 32-weight sub-block per
 * 16-byte record with its scale (and min) in the scale stream, the Q6_K
 * high code bits in a stream of their own and d (and dmin) once per row and
 * super-block.  Each weight is formed exactly before its product (Q4_K:
 * d * sc * q - dmin * m rounded once to fp32; Q6_K: the integer q - 32,
 * whose sum is scaled by d * sc per 16 weights), so rounding stays relative
 * to the sum of |w * x| and zero weights contribute exactly zero.
 * Q4_K stages activations in fp32 for both x types; Q6_K with bf16
 * activations pairs the exact bf16 q - 32 with them through dot2.  Runs the vector kernel
 * family for every m.  Limits as qgemv_*, with k % 256 == 0.
 * The other entry points (expert, fused, many-token and chain products)
 * return QG_EUNSUPPORTED for these formats.
 */
int qgemv_q4_k(const void *w_packed, int64_t n, int64_t k, const void *x, int xt, int64_t m,
               float *y, void *stream);
int qgemv_q6_k(const void *w_packed, int64_t n, int64_t k, const void *x, int xt, int64_t m,
               float *y, void *stream);

/*
 * Load-time decode cache: re-quantizes a Q8_0 matrix into packed NVFP4 for
 * qgemv_nvfp4, as imp converts GGUF Q8_0 weights to FP4 when a model loads
 * (imp README, "Why this exists").  The result approximates the Q8_0 weights
 * (4-bit values: imp release notes v0.4.1 record the accuracy cost); the
 * Q8_0 product is unaffected.  Recipe, fp32 arithmetic in this order:
 *   A = max |w| (w = d * q),  s_t = A / 2688 (or 1 if A = 0);  per 16 weights:
 *   a = max |w|,  s = E4M3 rounding of (a / 6) / s_t,  S = E4M3(s) * s_t,
 *   code = E2M1 rounding of w / S (0 if S = 0); roundings to nearest, ties to
 *   the even code, saturating at 448 and 6.  The trailer after the tensor
 *   scale keeps A (fp32 bits) at tensor_scale_offset + 4.
 * canon_q8_0: device, n * (k/32) canonical Q8_0 blocks with finite scales.
 * nvfp4_packed: device, qg_packed_bytes(QG_NVFP4, n, k) bytes, 256-byte
 * aligned, overwritten.  Three kernels on `stream`; deterministic.
 */
int qg_requant_q8_0_nvfp4(const void *canon_q8_0, int64_t n, int64_t k, void *nvfp4_packed, void *stream);

/*
 * Measurement aid: reads every byte of buf once (16-byte nontemporal loads,
 * 1 KiB per wavefront load instruction, the GEMV kernels' access shape) and
 * XOR-folds it into sink, one word per wavefront.  Timing it over a buffer
 * far larger than the device caches gives the achievable HBM read rate that
 * the products' bandwidth is compared with (decode is bound by memory
 * bandwidth: imp README, "Known limitations").  buf: device, 256-byte
 * aligned, bytes a positive multiple of 16.  sink: device uint32
 * [QG_STREAM_SINK], overwritten.
 */
#define QG_STREAM_SINK 16384
int qg_read_stream(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/*
 * Which kernel family a dense call with these arguments runs: QG_PATH_VALU,
 * QG_PATH_MFMA or QG_PATH_VALU_ONE, or a negative status (-QG_EINVAL, -QG_EUNSUPPORTED) for
 * arguments the dense calls would reject.  Host only; no device work.
 */
int qg_dense_path(int fmt, int64_t n, int64_t k, int xt, int64_t m);

/*
 * Dense product for 1 <= m <= QG_MAX_GEMM_M tokens (the prefill side of the
 * co-batch route: Imparo README, "Bonsai CUDA Validation", whose tensor-core
 * projections serve M 9..128 while small M keeps its own routes):
 *     y[t][i] = sum_c W[i][c] * x[t][c]        t < m, i < n
 * Arguments, layouts and limits as qgemv_* except m.  bf16 activations on
 * layouts of at most 16 lanes per row run on the matrix cores in one launch:
 * each group of 16 tokens is one MFMA operand, groups are a grid dimension
 * (they share each weight tile through the device caches).  Other calls
 * (fp32 activations, shorter matrices with more lanes per row) run the
 * dense product QG_MAX_M tokens per launch.  qg_gemm_path says which.
 */
int qgemm(int fmt, const void *w_packed, int64_t n, int64_t k, const void *x, int xt, int64_t m, float *y,
          void *stream);
int qg_gemm_path(int fmt, int64_t n, int64_t k, int xt, int64_t m);

/*
 * Dense product with its decode-step neighbours fused in (the pages report
 * such hand-made fusions: imp release notes v0.4, a fused RMSNorm-gated +
 * SiLU kernel; Imparo README, "Bonsai CUDA Validation", an RMS/Add tail
 * fusion; the operations themselves are the published ones):
 *     x'  = norm_weight ? x * r * norm_weight : x,
 *           r = 1 / sqrt(mean over c of x[t][c]^2 + norm_eps)    (RMSNorm)
 *     z   = W x'                                                   (n rows)
 *     o   = act == QG_ACT_SWIGLU ? SiLU(z[0 .. F)) * z[F .. 2F) : z,
 *           F = n / 2, SiLU(v) = v / (1 + exp(-v))   (gate rows first)
 *     y   = o + residual (if residual) ;  y [m][n_out], n_out = F or n
 * fmt: weight format of the packed w (as qgemv_*); x, xt, m as qgemv_*.
 * norm_weight: device fp32 [k], 16-byte aligned, or NULL (no normalisation);
 * norm_eps: finite, >= 0.  residual: device fp32 [m][n_out], 4-byte aligned,
 * or NULL; with an fp32 output it may be y itself (in-place add), otherwise
 * it must not overlap y.  y: device [m][n_out], fp32 (yt = QG_F32, 4-byte
 * aligned) or bf16 round-to-nearest-even (yt = QG_BF16, 2-byte aligned),
 * overwritten.  Runs the vector kernel family for every m: normalised
 * activations are kept in fp32 (a bf16 copy for the matrix cores would
 * round each by up to 2^-9).  r is computed in fp32 per workgroup, in a
 * fixed order, so the same inputs give the same bits.
 * Limits: those of qgemv_*; with SwiGLU n is even and F a multiple of the
 * layout's rows per tile (QG_EUNSUPPORTED otherwise).
 */
int qgemv_fused(int fmt, const void *w_packed, int64_t n, int64_t k, const void *x, int xt, int64_t m,
                const float *norm_weight, float norm_eps, int act, const float *residual,
                void *y, int yt, void *stream);

/*
 * Top-k expert product.  w_experts: device, n_experts packed matrices of
 * identical shape (fmt, n, k) back to back, expert e at byte offset
 * e * qg_packed_bytes(fmt, n, k) (a multiple of 256); 256-byte aligned.
 * topk_ids: device int32 [m][top_k]; topk_w: device fp32 [m][top_k].
 * Ids should be distinct within a token (repeated ids still follow the
 * formulas below); an id outside [0, n_experts) contributes nothing.
 *   QG_MOE_GATE_UP:      x [m][k];         y [m][top_k][n],
 *                        y[t][j][i] = W_{ids[t][j]}[i] . x[t]   (topk_w unused, may be NULL)
 *   QG_MOE_DOWN_COMBINE: x [m][top_k][k];  y [m][n],
 *                        y[t][i] = sum over j of topk_w[t][j] * (W_{ids[t][j]}[i] . x[t][j])
 * fp32 accumulation in a fixed order (ascending expert id, then slot), so
 * the same inputs give the same bits.  Only the selected experts' weights
 * are read; each distinct selected expert is streamed once per call for all
 * tokens that chose it.  NVFP4 experts: QG_EUNSUPPORTED.
 * Limits: 1 <= m <= 8, 1 <= top_k <= n_experts, m * top_k <= 64,
 * n_experts <= 65536.  y is overwritten, except gate_up rows of invalid ids.
 */
int moe_qgemv_topk(int fmt, const void *w_experts, int64_t n_experts, int64_t n, int64_t k,
                   const int32_t *topk_ids, const float *topk_w, int64_t m, int64_t top_k,
                   const void *x, int xt, int mode, float *y, void *stream);

/*
 * Top-k expert product with its decode-step neighbours fused in (the
 * definitions of qgemv_fused, per slot; the pages' MoE layers are gated
 * FFNs whose gate_up matrices have twice the down matrix's K rows):
 *   QG_MOE_GATE_UP:      y[t][j] = act(W_{ids[t][j]} x'_t), x'_t = RMSNorm(x_t) when
 *                        norm_weight is given; act = SwiGLU (gate rows first,
 *                        n_out = n / 2) or none.  y [m][top_k][n_out]; residual
 *                        must be NULL.  Rows of slots with invalid ids are not written.
 *   QG_MOE_DOWN_COMBINE: y[t] = sum over j of topk_w[t][j] * W_{ids[t][j]} x[t][j]
 *                        (+ residual[t]); y [m][n]; norm_weight must be NULL and
 *                        act QG_ACT_NONE.  residual: fp32 [m][n] or NULL; with an
 *                        fp32 y it may be y itself.
 * Other arguments as moe_qgemv_topk; norm_weight, norm_eps, yt as qgemv_fused.
 * Only the streaming kernel serves these calls: QG_EUNSUPPORTED when the
 * call's activation rows (fp32 when normalised) exceed its 96 KiB of LDS,
 * or with SwiGLU when F is not a multiple of the layout's rows per tile.
 */
int moe_qgemv_topk_fused(int fmt, const void *w_experts, int64_t n_experts, int64_t n, int64_t k,
                         const int32_t *topk_ids, const float *topk_w, int64_t m, int64_t top_k,
                         const void *x, int xt, int mode, const float *norm_weight, float norm_eps, int act,
                         const float *residual, void *y, int yt, void *stream);

/*
 * Top-k routing on the device, producing moe_qgemv_topk's ids and weights
 * without a host round trip (imp keeps MoE routing on the device so the
 * decode graph stays capturable: imp release notes v0.7.0, known issues).
 * logits: device fp32 [m][n_experts].  ids: device int32 [m][top_k], the
 * top_k experts of each token by descending logit, a lower expert id first
 * among equal logits.  weights: device fp32 [m][top_k], the softmax of the
 * selected logits (exp(l - l_max) / sum, fp32).  NaN logits rank as -inf; a
 * token whose selected logits are all -inf gets NaN weights.
 * Limits: 1 <= top_k <= min(n_experts, 64), n_experts <= 1024.  4-byte
 * aligned pointers; ids and weights are overwritten.
 */
int moe_router_topk(const float *logits, int64_t m, int64_t n_experts, int64_t top_k, int32_t *ids, float *weights,
                    void *stream);

/*
 * A chain of dense products executed in order by one persistent kernel:
 * product i+1 starts only after product i has completed on the whole device
 * (its outputs are visible device-wide), as consecutive projections of one
 * decode step require.  This removes the per-launch cost between products and
 * keeps the next product's weights streaming while a product drains, the way
 * Imparo's decode puts a layer's work into a single persistent launch whose
 * grid barriers stand where dispatch boundaries were (Imparo README,
 * "Megakernel Decode").
 *
 * Use: fill `count` links on the host, size a plan with qg_chain_plan_bytes,
 * build it with qg_chain_plan (host memory; queries the current device), copy
 * the plan bytes to device memory once, then call qgemv_chain with both
 * copies as often as needed (the links' pointers are baked into the plan).
 * All links share fmt, xt and m (1..8).  Each link's x must fit in LDS
 * (m * k * 4 bytes for Q8_0 or fp32 activations, m * k * 2 otherwise, up to
 * about 128 KiB), else QG_EUNSUPPORTED.  The kernel uses one workgroup per
 * compute unit and is launched cooperatively.  Barrier state lives in static
 * device memory: chains launched concurrently on one device (different
 * streams) race and must not overlap.  A barrier that waits too long ends its
 * wait and records a timeout, so the kernel always finishes; the rows a
 * workgroup computes after such a wait are written as NaN (their activations
 * may be stale), and qg_chain_error reports it.  qg_chain_plan refuses
 * (QG_EUNSUPPORTED) a kernel variant that would need scratch memory: the
 * runtime may hold back waves that need scratch, so not every workgroup could
 * be resident for the barriers.
 */
typedef struct {
    const void *w_packed;   /* device, packed (fmt, n, k) */
    const void *x;          /* device, [m][k] */
    float *y;               /* device, [m][n], overwritten */
    int64_t n, k;
} qg_chain_link_t;

/* Bytes of a plan for `count` links, or -1. */
int64_t qg_chain_plan_bytes(int64_t count);
/* Builds the plan in host memory (`plan`, qg_chain_plan_bytes bytes). */
int qg_chain_plan(int fmt, int xt, int64_t m, const qg_chain_link_t *links, int64_t count, void *plan);
/* Launches the chain.  plan_host: the built plan; plan_device: a 16-byte
 * aligned device copy of the same bytes. */
int qgemv_chain(const void *plan_host, const void *plan_device, void *stream);
/*
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): qgemv_chain without
 * the caller's device copy of the plan.  The plan bytes are copied from
 * plan_host (hipMemcpyAsync on `stream`) into a static device buffer of
 * QG_CHAIN_STATIC_BYTES bytes that the library holds on each device until
 * the process ends, and the chain kernel reads them there.  Allocates
 * nothing.  plan_host must stay unchanged until the stream has run the call.
 * A plan of more than QG_CHAIN_STATIC_BYTES bytes (qg_chain_plan_bytes of
 * more than 430 links) is refused with QG_EUNSUPPORTED before any device
 * work.  Every call on a device shares that device's buffer, and each call
 * rewrites the whole plan it reads: calls that overlap on one device (other
 * streams, other threads) race, as overlapping chain launches do anyway.
 * Results are those of qgemv_chain with the same plan, bit for bit.
 */
#define QG_CHAIN_STATIC_BYTES 65536
int qgemv_chain_noalloc(const void *plan_host, void *stream);
/* Diagnostic: synchronises the device; returns 1 if any chain barrier timed
 * out since the previous call (and clears the record), 0 if none, -1 on a
 * HIP error. */
int qg_chain_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
