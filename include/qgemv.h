/*
 * qgemv.h -- C interface of libqgemv: block-quantized weight x Q8-quantized
 * activation products for decode on AMD Instinct MI355X (gfx950).
 *
 * The operations follow the statement of the problem on these pages:
 *
 *  [PR623] "ROCm: restore DeepSeek V4 Flash decode performance and Q4 SSD
 *          streaming", antirez/ds4 pull request 623 -- Summary (the attention
 *          output projections -- single, two-matrix, HC-expand and grouped
 *          low-rank -- consuming an activation quantized to Q8 once; a compact
 *          table of the experts in use, built
 *          before the expert launch, which takes the expert matrices by
 *          pointer), Correctness (a call without that table fails instead of
 *          falling back) and the review comments (per-stage
 *          timing of the Q8_0 entry points; a decode log in which an expert id
 *          of -1, out of the range 0..256, fails the decode).
 *  [PR621] "Support AProjQ4 GGUFs: Q4_K dense attention projections ...",
 *          antirez/ds4 pull request 621 -- Q4_K dense attention projections
 *          and the dequantize + GEMM prefill path.
 *  [SOOT]  "DeepSeek V4 Flash on Strix Halo: tuning ROCm, matching Vulkan"
 *          (soothill.io) -- "Why I did not keep a ROCm kernel patch": the
 *          decode mat-vec plus the Q8 activation quantizer with a block sum.
 *  [ATOM]  ROCm/ATOM "DeepSeek-V4 Usage Guide" -- sigmoid routing of 6
 *          experts out of 256 or 384.
 *  [ATOMQ] ROCm/ATOM "DeepSeek-V4 Usage Guide", section "FP8 on MI308 /
 *          gfx942" -- the routed-expert quantization configs: FP8 e4m3 with
 *          128 x 128 weight blocks and FP4 e2m1 with 1 x 32 microscaling, both
 *          with ue8m0 scales (and the V4-Pro MoE backend note on FP4 e2m1).
 *  [LCPP]  llama.cpp pull request 24162 (DeepSeek V4 support) -- the grouped
 *          attention-output tensor, 8 groups of 1024 x 4096 rather than one
 *          4096 x 8192 matrix.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller, 16-byte
 *    aligned, row-major and densely packed.  The library never allocates,
 *    frees or retains them.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on it and returns; nothing synchronizes.
 *  - Outputs are overwritten, never accumulated into.
 *  - Return value: QG_OK (0) when the work was enqueued; a negative QG_ERR_*
 *    code when the host-side checks fail, in which case NOTHING was launched
 *    and no output was touched.  QG_ERR_LAUNCH reports a failed launch of
 *    the call's own kernels (an error that an earlier, unrelated HIP call
 *    left for the calling thread is cleared before the first launch).
 *  - Data errors that only the device can see (expert ids) are reported in a
 *    caller-provided device int32 status word (see moe_routed_qgemv).
 *  - The library's only process-wide state is set-up done once per device
 *    (the device's compute-unit count, kernels' dynamic-LDS limits), kept per
 *    device behind one lock, so calls from several host threads, on several
 *    streams or devices, may run concurrently (calls that share an output or
 *    a workspace must be ordered by the caller).  Results are deterministic:
 *    the same inputs give bit-identical outputs, and row t of a batched call
 *    equals the M = 1 call on token t.
 *
 * Weight formats (the pages name Q8_0 and Q4_K but print no byte layout; this
 * library defines its own, "Q4_K-style"):
 *
 *  QG_FMT_Q8_0  blocks of 32 weights, 34 bytes: fp16 scale d (little endian),
 *               then 32 int8 quants q.  weight = d * q.
 *  QG_FMT_Q4K   superblocks of 256 weights, 144 bytes: fp16 d, fp16 dmin,
 *               then 12 bytes holding sixteen 6-bit fields as one
 *               little-endian 96-bit string (field f = bits [6f, 6f+6);
 *               fields 0..7 are sub-block scales sc[j], 8..15 sub-block mins
 *               m[j]), then 128 bytes of 4-bit quants: sub-block 2p (p=0..3)
 *               in the low nibbles of bytes 16+32p .. 16+32p+31, sub-block
 *               2p+1 in the high nibbles of the same bytes.
 *               weight = d * sc[j] * q - dmin * m[j].
 *  A weight matrix with N rows (outputs) and K columns (inputs) is N rows of
 *  K/32 Q8_0 blocks or K/256 Q4_K superblocks; rows are consecutive.  Every
 *  projection here needs K % 256 == 0 (so each row is 16-byte aligned) and
 *  256 <= K <= QG_MAX_K.
 *
 *  Block-scaled expert formats [ATOMQ] (the page gives the element, block and
 *  scale formats, not the bytes; one matrix is one buffer of
 *  qg_matrix_bytes(fmt, N, K) bytes: the codes, then from the first multiple
 *  of 256 bytes after them, the scale bytes, then padding up to a multiple of
 *  16 bytes, so that matrices stored back to back stay 16-byte aligned):
 *  QG_FMT_FP8_E4M3_B128  codes uint8 [N, K], OCP FP8 E4M3 (sign, 4-bit
 *               exponent with bias 7, 3-bit mantissa, no infinities,
 *               S.1111.111 = NaN, largest value 448); scales uint8
 *               [ceil(N/128), K/128], UE8M0.
 *               weight (n, k) = e4m3(code) * 2^(S[n/128][k/128] - 127).
 *  QG_FMT_FP4_E2M1_MX    codes uint8 [N, K/2], two OCP FP4 E2M1 values per
 *               byte (element 2i in the low nibble of byte i, 2i+1 in the
 *               high nibble; values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
 *               negatives); scales uint8 [N, K/32], UE8M0.
 *               weight (n, k) = e2m1(code) * 2^(S[n][k/32] - 127).
 *  UE8M0: an unsigned exponent, 2^(s - 127); s = 255 (NaN in the OCP
 *  definition) is outside the contract.  Codes that are NaN give NaN.
 *
 * Q8 activation (what quantize_act_q8 produces and every projection consumes):
 *  qx int8 [M, K]; dx fp32 [M, K/32], the scale of each 32-block;
 *  sx int32 [M, K/32], the sum of each block's quants (used by Q4_K's min term).
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define QG_OK 0
#define QG_ERR_NULL (-1)      /* a required pointer is NULL */
#define QG_ERR_SHAPE (-2)     /* a size is out of range (see each call) */
#define QG_ERR_ALIGN (-3)     /* a pointer is not 16-byte aligned */
#define QG_ERR_FORMAT (-4)    /* unknown weight format */
#define QG_ERR_WORKSPACE (-5) /* workspace smaller than moe_routed_workspace_bytes() */
#define QG_ERR_LAUNCH (-6)    /* the kernel launch failed (hipGetLastError) */

/* device status word values (moe_routed_qgemv) */
#define QG_DEV_OK 0
#define QG_DEV_BAD_EXPERT 1  /* an expert id outside [0, E) */
#define QG_DEV_NULL_EXPERT 2 /* a selected expert has a NULL or misaligned weight pointer */

/* weight formats */
#define QG_FMT_Q8_0 0
#define QG_FMT_Q4K 1
#define QG_FMT_FP8_E4M3_B128 2
#define QG_FMT_FP4_E2M1_MX 3

/* limits */
#define QG_MAX_K 16384        /* largest K (inputs) of a projection */
#define QG_MAX_M 32           /* largest token batch of qgemv_* */
#define QG_MAX_PREFILL_M 65536 /* largest token count of qgemm_q8_0 */
#define QG_MAX_MOE_PAIRS 8192 /* largest T * topk of moe_routed_qgemv */
#define QG_MAX_EXPERTS 4096   /* largest E of moe_routed_qgemv */

/* ---- activation quantization ------------------------------------------- */
/*
 * quantize_act_q8 -- [PR623] Summary: quantize the decode activation to Q8
 * once, then feed every Q8 projection; [SOOT] the quantizer that keeps a block
 * sum next to the scale.
 *
 * For each row m < M and each block b < K/32 of x (fp32 [M, K]):
 *   amax = max |x|;  d = amax / 127 (IEEE fp32 division, round to nearest);
 *   q_i  = round-half-to-even(x_i / d) clamped to [-127, 127], or 0 when d == 0;
 *   dx[m, b] = d;  sx[m, b] = sum_i q_i;  qx[m, 32b + i] = q_i.
 * Bit-exact: the fp32 quotient is correctly rounded, subnormals are kept.
 * NaN or Inf inputs are outside the contract.
 * Errors: QG_ERR_NULL; QG_ERR_SHAPE unless M >= 1 and K >= 32, K % 32 == 0;
 * QG_ERR_ALIGN.
 */
int quantize_act_q8(const float *x, int M, int K, int8_t *qx, float *dx, int32_t *sx, void *stream);

/* ---- decode mat-vec ---------------------------------------------------- */
/*
 * qgemv_q8_0 -- [PR623] the regular Q8_0 projection on a prequantized
 * activation (matmul_q8_0_tensor in the per-stage table).
 *   y[m, n] = sum_b dw[n, b] * dx[m, b] * sum_{i<32} qw[n, b, i] * qx[m, 32b + i]
 * W: QG_FMT_Q8_0 [N, K]; qx/dx: Q8 activation of M tokens; y fp32 [M, N].
 * Each weight block is read once for all M tokens.  The per-block integer
 * sums are exact; scaling and accumulation are fp32 (error well under
 * 1e-5 * sum |w * x| per output).
 * Errors: QG_ERR_NULL; QG_ERR_SHAPE unless N >= 1, 1 <= M <= QG_MAX_M,
 * K % 256 == 0, 256 <= K <= QG_MAX_K; QG_ERR_ALIGN; QG_ERR_LAUNCH.
 */
int qgemv_q8_0(const void *W, int N, int K, const int8_t *qx, const float *dx, int M, float *y, void *stream);

/*
 * qgemv_q4k -- [PR621] Q4_K dense attention projection on a Q8 activation.
 *   y[m, n] = sum_s sum_j dx[m, sj] * ( d[n,s] * sc[n,s,j] * sum_i q[n,s,j,i] * qx[m, ...]
 *                                      - dmin[n,s] * m[n,s,j] * sx[m, sj] )
 * (s = superblock, j = sub-block; sj = 8s + j is the 32-block index.)
 * W: QG_FMT_Q4K [N, K]; qx/dx/sx as from quantize_act_q8; y fp32 [M, N].
 * Errors: as qgemv_q8_0.
 */
int qgemv_q4k(const void *W, int N, int K, const int8_t *qx, const float *dx, const int32_t *sx, int M, float *y,
              void *stream);

/*
 * qgemv_paired -- [PR623] the paired projection (matmul_q8_0_pair_tensor):
 * one prequantized activation feeds two weight matrices in a single launch,
 * e.g. the low-rank style 4096->1024 and 4096->512 pair.
 *   y1 = W1 . x  ([M, N1]),   y2 = W2 . x  ([M, N2])
 * Both matrices have format `fmt` and K inputs.  Each output equals the
 * single-matrix call bit for bit.  sx may be NULL for QG_FMT_Q8_0.
 * Errors: QG_ERR_FORMAT; otherwise as qgemv_q8_0 (N1, N2 >= 1).
 */
int qgemv_paired(int fmt, const void *W1, int N1, const void *W2, int N2, int K, const int8_t *qx, const float *dx,
                 const int32_t *sx, int M, float *y1, float *y2, void *stream);

/*
 * qgemv_grouped -- [PR623] Summary, the low-rank attention-output projection
 * among the prequantized decode call sites; [LCPP] its tensor is G = 8 groups
 * of N x K (1024 x 4096), each applied to its own K-wide slice of the input.
 *   y[m, g, n] = sum_k w_g[n, k] * x[m, g*K + k]        (g < G, n < N)
 * W: G matrices of format `fmt` [N, K] stored one after another (the [G, N, K]
 * tensor); qx/dx/sx: the Q8 activation of the G*K-wide input [M, G*K] (its
 * 32-blocks never straddle two slices); y fp32 [M, G*N].  Group g equals
 * qgemv_q8_0 / qgemv_q4k of matrix g on slice g, bit for bit.  sx may be NULL
 * for QG_FMT_Q8_0.
 * Errors: QG_ERR_FORMAT; QG_ERR_SHAPE unless 1 <= G <= 65535; otherwise as
 * qgemv_q8_0.
 */
int qgemv_grouped(int fmt, const void *W, int G, int N, int K, const int8_t *qx, const float *dx, const int32_t *sx,
                  int M, float *y, void *stream);

/*
 * qgemv_q8_0_quality -- [PR623] Summary: the fp32-activation ("shared-x")
 * Q8_0 product that prequantized decode replaced, kept as its exact-activation
 * comparator (the quality mode).  No activation quantization:
 *   y[m, n] = sum_b dw[n, b] * sum_{i<32} qw[n, b, i] * x[m, 32b + i]
 * W: QG_FMT_Q8_0 [N, K]; x fp32 [M, K]; y fp32 [M, N].  fp32 arithmetic
 * (error well under 1e-5 * sum |w * x| per output, x as given).
 * Errors: as qgemv_q8_0.
 */
int qgemv_q8_0_quality(const void *W, int N, int K, const float *x, int M, float *y, void *stream);

/*
 * qgemv_q8_0_f32, qgemv_q4k_f32, qgemv_paired_f32 -- the same products taking
 * the fp32 activation x [M, K] instead of its Q8 form.  [PR623] Summary:
 * the decode activation is quantized to Q8 once and fed to every projection;
 * here the first projection that consumes x does the quantization inside its
 * kernel (every workgroup quantizes x while staging it, exactly as
 * quantize_act_q8 does), and writes the Q8 activation to qx [M, K], dx and sx
 * [M, K/32] for the projections that follow; each of qx, dx, sx may be NULL.
 * y (and y1, y2) equal the two-step quantize_act_q8 + qgemv_* result bit for
 * bit, and qx/dx/sx equal quantize_act_q8's output.
 * Errors: QG_ERR_NULL if x (or a weight or output) is NULL; otherwise as the
 * Q8-activation forms.
 */
int qgemv_q8_0_f32(const void *W, int N, int K, const float *x, int M, float *y, int8_t *qx, float *dx, int32_t *sx,
                   void *stream);
int qgemv_q4k_f32(const void *W, int N, int K, const float *x, int M, float *y, int8_t *qx, float *dx, int32_t *sx,
                  void *stream);
int qgemv_paired_f32(int fmt, const void *W1, int N1, const void *W2, int N2, int K, const float *x, int M, float *y1,
                     float *y2, int8_t *qx, float *dx, int32_t *sx, void *stream);

/*
 * qgemm_q8_0 -- the Q8_0 projection over a prefill-sized batch on the matrix
 * cores ([PR623]: the Q8_0 projections on a prequantized activation; [PR621]:
 * prefill takes the batched path): the same product and the same arithmetic
 * as qgemv_q8_0, for M up to QG_MAX_PREFILL_M tokens, so row m equals the
 * one-token qgemv_q8_0 call on token m bit for bit.  Each 32-block's integer
 * sums come from int8 MFMA (v_mfma_i32_32x32x32_i8), 32 rows x 32 tokens at a
 * time.
 * W: QG_FMT_Q8_0 [N, K]; qx/dx: Q8 activation [M, K] (quantize_act_q8);
 * y fp32 [M, N].
 * Errors: QG_ERR_NULL; QG_ERR_SHAPE unless N >= 1, 1 <= M <= QG_MAX_PREFILL_M,
 * K % 256 == 0, 256 <= K <= QG_MAX_K; QG_ERR_ALIGN; QG_ERR_LAUNCH.
 */
int qgemm_q8_0(const void *W, int N, int K, const int8_t *qx, const float *dx, int M, float *y, void *stream);

/* ---- block-scaled expert formats -------------------------------------- */
/*
 * qg_matrix_bytes -- bytes of an N x K weight matrix in format fmt (any of the
 * four; for FP8 / FP4 the codes, the padding to 256 bytes, the scales and
 * the padding to a multiple of 16 bytes).
 * Returns 0 for an unknown format or an out-of-range shape (N >= 1,
 * K % 256 == 0, 256 <= K <= QG_MAX_K).
 */
size_t qg_matrix_bytes(int fmt, int N, int K);

/*
 * qgemv_mx -- [ATOMQ] the expert formats' mat-vec as a dense projection:
 *   y[m, n] = sum_k w[n, k] * (dx[m, k/32] * qx[m, k])
 * W: QG_FMT_FP8_E4M3_B128 or QG_FMT_FP4_E2M1_MX [N, K] as described above;
 * qx/dx: Q8 activation of M tokens; y fp32 [M, N].  The codes are converted
 * to fp16 and dotted with the fp16 form of qx (exact) in fp32, one 16-byte
 * chunk of a row at a time (16 FP8 or 32 FP4 weights), each chunk's sum
 * scaled by dx * 2^(s - 127) and accumulated in fp32: the error is well under
 * 1e-5 * sum_k |w x| per output (FP4 chunk sums are exact).
 * Errors: QG_ERR_FORMAT (formats 2 and 3 only); QG_ERR_NULL; QG_ERR_SHAPE
 * unless N >= 1, 1 <= M <= QG_MAX_M, K % 256 == 0, 256 <= K <= QG_MAX_K;
 * QG_ERR_ALIGN; QG_ERR_LAUNCH.
 */
int qgemv_mx(int fmt, const void *W, int N, int K, const int8_t *qx, const float *dx, int M, float *y, void *stream);

/* ---- routed MoE -------------------------------------------------------- */
/*
 * Workspace of moe_routed_qgemv, in bytes, for the given sizes (0 if a size
 * is out of range).  The caller allocates it on the device; its contents
 * after a call are described by moe_routed_workspace_layout.
 */
size_t moe_routed_workspace_bytes(int T, int topk, int E, int D, int F);

/* regions of the MoE workspace (byte offsets from moe_routed_workspace_layout) */
#define QG_WS_NUNIQ 0    /* int32 [1]      number of distinct valid experts U */
#define QG_WS_UNIQ 1     /* int32 [Ucap]   distinct usable expert ids, ascending */
#define QG_WS_SLOT 2     /* int32 [P]      index in uniq of pair p's expert, -1 if invalid */
#define QG_WS_PAIR_OFF 3 /* int32 [Ucap+1] CSR offsets into pairs */
#define QG_WS_PAIRS 4    /* int32 [P]      pair indices grouped by expert, ascending within */
#define QG_WS_G 5        /* fp32  [P, F]   gate outputs */
#define QG_WS_V 6        /* fp32  [P, F]   up outputs */
#define QG_WS_H 7        /* fp32  [P, F]   silu(g) * v */
#define QG_WS_HQ 8       /* int8  [P, F]   Q8 quants of h */
#define QG_WS_HD 9       /* fp32  [P, F/32] Q8 scales of h */
#define QG_WS_HS 10      /* int32 [P, F/32] Q8 block sums of h */
#define QG_WS_O 11       /* fp32  [P, D]   down outputs per pair */
#define QG_WS_HOT 12     /* int32 [1 + 2 Hcap] experts on the matrix cores: count, then per 32-pair
                            tile (slot in uniq, first pair of the tile within the expert) */
#define QG_WS_COUNT 13
/* P = T * topk, Ucap = min(P, E), Hcap = P / 32 + P / QG_MOE_MM_PAIRS + 1.  Rows of pairs with an
 * invalid id are not written. */
#define QG_MOE_MM_PAIRS 9 /* Q4_K experts with this many pairs or more (T >= it) use the matrix cores */

/*
 * moe_routed_workspace_layout -- byte offsets of the regions above, written
 * to offsets[0 .. QG_WS_COUNT).  Returns QG_OK or QG_ERR_SHAPE / QG_ERR_NULL.
 */
int moe_routed_workspace_layout(int T, int topk, int E, int D, int F, size_t *offsets);

/*
 * moe_routed_qgemv -- [PR623] routed-MoE decode driven by a compact
 * selected-expert table built on the device before the pointer-backed expert
 * launches (Summary; the missing compact table of selected experts was the failure it
 * fixes); [ATOM] top-6 sigmoid-normalized routing.
 *
 * For T tokens with Q8 activations qx/dx/sx ([T, D]) and selected experts
 * ids int32 [T, topk] with routing weights rw fp32 [T, topk]:
 *   1. table: uniq = distinct valid ids ascending, slot, CSR pairs (workspace);
 *   2. for each distinct expert e and each of its pairs p = (t, k):
 *        g = gate_e . x_t,  v = up_e . x_t             (Q4_K, F x D)
 *        h = silu(g) * v  (fp32),  (hq, hd, hs) = Q8-quantize(h)
 *   3.   o_p = down_e . hq                              (Q4_K, D x F)
 *   4. y[t] = sum_k rw[t, k] * o_(t,k)   in k order (fp32).
 * Each selected expert's weights are streamed once for all of its pairs.
 * With one token and at most 64 pairs the table is built inside the first
 * expert launch: every workgroup derives its expert from the ids, and one
 * of them writes the table and the status word; otherwise a table launch
 * comes first.  The workspace holds the same table either way.
 * With T >= QG_MOE_MM_PAIRS, experts with at least that many pairs run gate,
 * up and down on the int8 matrix cores (32 pairs at a time, gathered through
 * the pair list); their results equal the one-token form bit for bit, as for
 * the dense batched calls.
 * gate/up/down are DEVICE arrays of E device pointers (pointer-backed expert
 * table); experts that are not selected are never dereferenced and may be
 * NULL.  The host never waits for the table: the number of distinct experts
 * stays on the device.
 *
 * Data errors: an id outside [0, E) sets *d_status to QG_DEV_BAD_EXPERT, and
 * a selected expert whose gate, up or down pointer is NULL or not 16-byte
 * aligned sets QG_DEV_NULL_EXPERT (a bad id takes precedence); such a pair
 * gets slot -1, contributes 0 to y, and every other pair is still computed.
 * Such an expert is left out of uniq.  *d_status (QG_DEV_OK otherwise) is
 * written by the first launch, on the stream, so the caller reads it after
 * synchronizing.
 *
 * Errors: QG_ERR_NULL (any pointer except unselected experts);
 * QG_ERR_SHAPE unless 1 <= T, 1 <= topk, T*topk <= QG_MAX_MOE_PAIRS,
 * 1 <= E <= QG_MAX_EXPERTS, D and F multiples of 256 in [256, QG_MAX_K];
 * QG_ERR_WORKSPACE if ws_bytes < moe_routed_workspace_bytes(...);
 * QG_ERR_ALIGN; QG_ERR_LAUNCH.
 */
int moe_routed_qgemv(const int8_t *qx, const float *dx, const int32_t *sx, int T, int D, int F, int E, int topk,
                     const int32_t *ids, const float *rw, const void *const *gate, const void *const *up,
                     const void *const *down, float *y, void *ws, size_t ws_bytes, int32_t *d_status, void *stream);

/*
 * moe_routed_qgemv_fmt -- moe_routed_qgemv with the experts in format fmt:
 * QG_FMT_Q4K (exactly moe_routed_qgemv), or the [ATOMQ] expert formats
 * QG_FMT_FP8_E4M3_B128 and QG_FMT_FP4_E2M1_MX (each gate/up/down pointer then
 * points at one qg_matrix_bytes(fmt, ...) buffer).  Steps 1-4 as above; with
 * the block-scaled formats gate/up and down run the qgemv_mx engine, and h is
 * Q8-quantized once per pair before the down projection (for one token with
 * FP4 experts inside the down launch, while it stages h; the workspace holds
 * h and its Q8 form either way).
 * Errors: QG_ERR_FORMAT for any other fmt; otherwise as moe_routed_qgemv.
 */
int moe_routed_qgemv_fmt(int fmt, const int8_t *qx, const float *dx, const int32_t *sx, int T, int D, int F, int E,
                         int topk, const int32_t *ids, const float *rw, const void *const *gate,
                         const void *const *up, const void *const *down, float *y, void *ws, size_t ws_bytes,
                         int32_t *d_status, void *stream);

/*
 * moe_routed_qgemv_noalloc -- moe_routed_qgemv_fmt for callers that cannot
 * allocate device memory (work recorded under HIP graph capture, serving loops
 * that must not allocate, hosts that forbid it): the same call, arguments and
 * results, with no workspace argument.  Its workspace is a fixed array of
 * QG_MOE_SCRATCH_BYTES in device memory that the library holds on every
 * device it runs on, from its first call there until the process ends; the
 * call itself allocates nothing.  Calls whose workspace
 * (moe_routed_workspace_bytes) exceeds QG_MOE_SCRATCH_BYTES are rejected with
 * QG_ERR_WORKSPACE before anything is launched (with 6 experts per token,
 * D = 4096 and F = 2048: up to 32 tokens).  Every call on one device shares
 * that device's array: calls that may overlap on one device (several streams
 * or host threads) race and must be ordered by the caller.  Nothing in the
 * array needs to start at zero; its contents after a call are those of the
 * workspace of moe_routed_qgemv (moe_routed_workspace_layout) until the next
 * call.
 * Errors: as moe_routed_qgemv_fmt (QG_ERR_WORKSPACE as above).
 */
#define QG_MOE_SCRATCH_BYTES (8u << 20)
int moe_routed_qgemv_noalloc(int fmt, const int8_t *qx, const float *dx, const int32_t *sx, int T, int D, int F,
                             int E, int topk, const int32_t *ids, const float *rw, const void *const *gate,
                             const void *const *up, const void *const *down, float *y, int32_t *d_status,
                             void *stream);

/* ---- prefill ----------------------------------------------------------- */
/*
 * qgemm_prefill -- [PR621] the dequantize-then-GEMM path for prefill batches
 * of Q4_K projections (the path whose ~16x regression and recovery the page
 * reports).
 *   Y[m, n] = sum_k w[n, k] * x[m, k],  w from QG_FMT_Q4K W [N, K],
 *   x bf16 [M, K] (raw bits), Y fp32 [M, N], fp32 accumulation on matrix
 *   cores (error well under 1e-5 * sum |w * x| per output).  x is converted
 *   to fp16 as it is: |x| must not exceed 65504, and |x| below 2^-17 loses
 *   low bits (qgemm_prefill_ws has no such limit).  d and dmin may take any
 *   fp16 value.
 * Errors: QG_ERR_FORMAT (only QG_FMT_Q4K); QG_ERR_NULL; QG_ERR_SHAPE unless
 * M >= 1, N >= 1, K % 256 == 0, 256 <= K <= QG_MAX_K; QG_ERR_ALIGN;
 * QG_ERR_LAUNCH.
 */
int qgemm_prefill(int fmt, const void *W, int N, int K, const uint16_t *x_bf16, int M, float *y, void *stream);

/*
 * qgemm_prefill_workspace_bytes -- size of the device workspace that
 * qgemm_prefill_ws needs for M tokens of K inputs: x scaled by a power of two
 * per token as fp16 [M, K], the int32 exponents [M], then the sums of the
 * scaled x over each 32-input block as fp16 high and low parts, [M, K/128]
 * records of 8 halves (the high parts of four blocks, then their low parts),
 * every region 256-byte aligned.  Returns 0 for an invalid shape (the rules
 * of qgemm_prefill).
 */
size_t qgemm_prefill_workspace_bytes(int M, int K);

/*
 * qgemm_prefill_ws -- [PR621] the same product as qgemm_prefill, with the
 * bf16 -> fp16 conversion of x done once by a separate pass into the caller's
 * workspace, and a faster GEMM that reads it.  Each token is scaled by a
 * power of two that puts its largest |x| in [2^15, 2^16), so any finite bf16
 * row can be given (qgemm_prefill needs |x| <= 65504).  The conversion is
 * exact for every element within about 2^32 of the token's largest |x|;
 * smaller elements become fp16 subnormals and keep fewer bits (below about
 * 2^-40 of it they become 0), an error far inside the bound, since they
 * weigh that much less in sum |w * x|.  Results agree with qgemm_prefill to
 * rounding (the same error bound).  ws is device memory owned by the caller (at least
 * qgemm_prefill_workspace_bytes(M, K) bytes, 16-byte aligned); its contents on
 * entry are ignored and on return are unspecified.  Calls that share a
 * workspace must be ordered on one stream.
 * Errors: as qgemm_prefill, plus QG_ERR_NULL for ws, QG_ERR_ALIGN for a
 * misaligned ws and QG_ERR_WORKSPACE if ws_bytes is too small.
 */
int qgemm_prefill_ws(int fmt, const void *W, int N, int K, const uint16_t *x_bf16, int M, float *y, void *ws,
                     size_t ws_bytes, void *stream);

/* ---- diagnostics ------------------------------------------------------- */
/* Human-readable text for a QG_* status or QG_DEV_* value (static storage). */
const char *qg_status_string(int status);

/*
 * qgemv_debug_block_isums -- the exact per-block integer sums that the GEMV
 * kernels form, from the same device code:
 *   isum[m, n, b] = sum_{i<32} q_w[n, b, i] * qx[m, 32b + i]
 * (q_w = int8 quant for Q8_0, 4-bit quant 0..15 of sub-block b for Q4_K).
 * isum int32 [M, N, K/32].  For testing; errors as qgemv_q8_0.
 */
int qgemv_debug_block_isums(int fmt, const void *W, int N, int K, const int8_t *qx, int M, int32_t *isum,
                            void *stream);

/*
 * qg_stream_read, qg_stream_read_bursts -- diagnostic: the HBM read rate that
 * the decode mat-vecs are measured against (the pages report mat-vec time
 * against the memory it streams, [SOOT] "Why I did not keep a ROCm kernel
 * patch"; this call gives the same part's own ceiling for a given byte count).
 * Reads bytes bytes of buf once, the way the mat-vec kernels stream weights:
 * the buffer is cut into bursts of chunk_kib KiB (chunk_kib in {1, 2, 4, 8,
 * 16}; the last one may be short), each read by one wave as one run of
 * 16-byte non-temporal loads, 1 KiB per instruction, waves waves (1..16) per
 * workgroup, and no other work.  Burst b writes the XOR of the 32-bit words it
 * read to burst_xor[b] (uint32, device), so the XOR of all entries is the XOR
 * of the buffer's words; with burst_xor NULL nothing is written (the read
 * alone, for timing).  qg_stream_read_bursts returns the number of bursts
 * (the length burst_xor needs), 0 for invalid arguments.
 * Errors: QG_ERR_NULL (buf); QG_ERR_SHAPE unless bytes is a non-zero multiple
 * of 16, chunk_kib and waves are as above and, when burst_xor is given,
 * burst_xor_len >= the burst count;
 * QG_ERR_ALIGN (buf 16-byte, burst_xor 4-byte aligned); QG_ERR_LAUNCH.
 */
size_t qg_stream_read_bursts(size_t bytes, int chunk_kib);
int qg_stream_read(const void *buf, size_t bytes, int chunk_kib, int waves, uint32_t *burst_xor,
                   size_t burst_xor_len, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
