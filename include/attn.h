/*
 * Exact tiled masked softmax attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn.so.  Every entry point validates its arguments on the host
 * before anything is launched; on an error nothing is launched and no output
 * is touched.  Kernels run asynchronously on the caller's stream; the library
 * allocates no memory, keeps no state between calls and is re-entrant.
 *
 * Conventions for every entry point
 *   - Tensor pointers are device pointers allocated and owned by the caller.
 *     Tensors are dense and row-major with the feature dimension contiguous.
 *     16-bit tensors must be 16-byte aligned.
 *   - Outputs (Y, LSE, dQ, dK, dV, O, dKV, dSink) are overwritten, never
 *     accumulated into.
 *   - `stream` is a hipStream_t (NULL = the default stream).
 *   - A failed kernel launch returns ATTN_ERR_HIP.
 *   - Non-finite input values are not checked on the normal path; they
 *     propagate.
 *   - Debug checks: when the environment variable ATTN_DEBUG holds a nonzero
 *     integer at the time of a call, the call also (a) validates on the device,
 *     before any attention kernel is launched, the values of index and length
 *     arrays the host cannot see (dense `lengths` in [0, n]; sparse
 *     `topk_length` in [0, topk] and every `topk_idx` entry below it in
 *     [0, Tkv)), returning ATTN_ERR_INVALID_ARG with no output written; and (b)
 *     after the kernels, scans every output for NaN or infinity (-inf is
 *     allowed in an LSE, where it marks an empty row) and returns
 *     ATTN_ERR_NONFINITE if it finds one.  The course this library follows
 *     refuses non-finite results; device writes cannot be rolled back, so the
 *     outputs' contents are unspecified after ATTN_ERR_NONFINITE.  Debug
 *     checks synchronise the stream and never trap.
 *   - Size limits (ATTN_ERR_UNSUPPORTED beyond them): every per-(batch, head)
 *     tensor below 2^32 bytes; B * H * n_q and B * H_kv * n_k at most
 *     2^28 - 64 rows; fp32 path: B * H at most 65535.
 *
 * Sources.  The operation is defined on these pages:
 *   [P1] alphabetamath.cc, "Tiled attention and its recomputed reverse pass
 *        are exact" (the summary invariant, the empty state, exactness of the
 *        forward row and of the reverse updates);
 *   [P2] alphabetamath.cc, "Exact tiled attention and memory-aware
 *        differentiation -- Examples" (worked examples, inverted dropout);
 *   [P3] intale.github.io, practical LLM in Rust, ch. 19 "Online tiled
 *        attention" (update rule, reverse formulas, grouped heads);
 *   [P5] icavan.github.io, "DeepSeek Sparse Attention Forward and Backward"
 *        (shared-KV top-k sparse attention with a sink).
 */
#ifndef EXACT_TILED_SOFTMAX_ATTN_H
#define EXACT_TILED_SOFTMAX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* bad shape, pointer, alignment, scale, rate or mask */
  ATTN_ERR_UNSUPPORTED = 2, /* valid request this build has no kernel for */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size() */
  ATTN_ERR_HIP = 4,         /* a HIP launch failed */
  ATTN_ERR_NONFINITE = 5    /* debug checks only: an output holds NaN or infinity */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 } attn_dtype;

/*
 * The allowed-key sets A_i of [P1]: allowed(i, j) is the AND of every
 * enabled part; with no part enabled every key is allowed.
 *   causal      nonzero: j <= i (requires n_q == n_k)
 *   window      > 0: i - j < window (a look-back window; with causal the
 *               window holds `window` keys including key i); 0: off
 *   block_mask  device pointer to uint8 [ceil(n_q/block_q)][ceil(n_k/block_k)],
 *               shared by all batches and heads; key j is allowed for row i
 *               only if block_mask[i/block_q][j/block_k] != 0; NULL: off
 *   dense_mask  device pointer to uint8 [n_q][n_k], shared by all batches and
 *               heads; NULL: off
 *   lengths     device pointer to int32 [B] (requires n_q == n_k): the active
 *               length of each batch's sequence; rows i >= lengths[b] are
 *               inactive (Y = 0, LSE = -inf, zero gradients) and keys
 *               j >= lengths[b] are never allowed.  Values outside [0, n] are
 *               clamped into it (rejected by the debug checks).  NULL: off
 *   starts      device pointer to int32 [B][n_q]: key j is allowed for row i
 *               of batch b only if j >= starts[b][i], the row's lower key
 *               bound; for packed segments (several sequences concatenated
 *               along n) starts[b][i] is the first row of the segment that
 *               holds row i, which with `causal` gives block-diagonal causal
 *               attention.  Any int32 value is valid.  NULL: off
 * lengths and starts are the variable-length layout of [P3] ("Rescale earlier
 * mass before adding a new tile": the per-row lower bound and inactive padded
 * rows; "Change attention evaluation inside the existing model": active
 * lengths and packed-segment boundaries intersected with the causal range).
 * A NULL attn_mask_t* means every key is allowed.  A row whose allowed set is
 * empty gets Y = 0 and LSE = -inf and contributes nothing to any gradient
 * (the convention [P3] uses for query rows without keys).
 */
typedef struct {
  int32_t causal;
  int32_t window;
  const uint8_t* block_mask;
  int32_t block_q, block_k;
  const uint8_t* dense_mask;
  const int32_t* lengths;
  const int32_t* starts;
} attn_mask_t;

/*
 * Inverted dropout ([P2], "A different dropout mask changes the reverse
 * result"): each attention weight p_ij is multiplied by xi_ij / (1 - rate).
 * xi is regenerated, never stored: with Philox4x32-10 (Salmon et al., SC'11),
 * key = (seed mod 2^32, seed div 2^32) and counter = (j div 8, i, b*H + h, 0),
 * u is the 16-bit half (j mod 2) of output word (j mod 8) div 2 (low half for
 * even j) and xi_ij = 0 iff u < floor(rate * 2^16), where rate is widened to
 * double: one draw decides eight keys.  The forward and reverse passes draw
 * identical xi.  The normaliser l_i and the LSE use the undropped weights.
 * NULL or rate == 0: no dropout.  rate must lie in [0, 1).
 */
typedef struct {
  float rate;
  uint64_t seed;
} attn_dropout_t;

/*
 * attn_fwd -- exact tiled masked attention forward ([P1] paragraphs 1-2,
 * [P3] "Rescale earlier mass before adding a new tile").
 *
 *   Y_i   = sum_{j in A_i} e^{s_ij} V_j / sum_{j in A_i} e^{s_ij},
 *   s_ij  = scale * sum_r Q_ir K_jr,   LSE_i = ln sum_{j in A_i} e^{s_ij}.
 *
 * Keys are streamed in blocks with the running summary (m, l, z) started in
 * the empty state; empty allowed blocks leave it unchanged; the full score grid
 * is never stored.
 *
 *   dt        ATTN_F32, ATTN_F16 or ATTN_BF16 (Q, K, V, Y); LSE is always fp32
 *   Q         [B][H][n_q][d]
 *   K         [B][H_kv][n_k][d]      query head h reads K/V head h / (H / H_kv)
 *   V         [B][H_kv][n_k][dv]
 *   mask      allowed sets (see attn_mask_t), may be NULL
 *   scale     c >= 0, finite
 *   block_b   key-block size b: fp32 honours any b >= 1 exactly; the bf16/fp16
 *             kernels use b = 64 and accept 0 or 64; 0 = the kernel default
 *   dropout   may be NULL
 *   Y         [B][H][n_q][dv] output, same dtype as Q
 *   LSE       [B][H][n_q] fp32 output (natural log)
 * Shapes: fp32 needs d, dv <= 128; bf16/fp16 need d == dv in {64, 128}.
 */
attn_status attn_fwd(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d, int dv,
                     const void* Q, const void* K, const void* V, const attn_mask_t* mask,
                     float scale, int block_b, const attn_dropout_t* dropout,
                     void* Y, float* LSE, void* stream);

/* Bytes of device workspace attn_bwd needs (fp32 D_i, stored negated, and the
 * base-2 LSE of every query row, plus padding). */
size_t attn_bwd_workspace_size(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d,
                               int dv);

/*
 * Bytes of workspace with which attn_bwd takes its stored-gamma form for this
 * mask and dropout, or attn_bwd_workspace_size() when the call has none.  The
 * form exists for bf16/fp16 with dropout (rate > 0) and a causal and / or
 * window mask only (no block mask, dense mask, lengths or starts): the dK/dV
 * kernel, which forms every gamma_ij = p_ij (kappa_ij G_i . V_j - D_i) of the
 * reverse pass ([P1] paragraphs 4-6) anyway, also writes them (rounded to the
 * input dtype, as its own products use them) to the workspace, and the dQ
 * product dQ_i = c sum_j gamma_ij K_j reads them back instead of recomputing
 * s_ij, G_i . V_j and the dropout draws.  The extra space is 16 KiB per
 * 64-key x 128-query tile that the mask reaches, per (batch, query head):
 * B H ceil(n/128) (ceil(n/128) + 1) tiles for a causal mask, e.g. 1.09 GB for
 * B = 1, H = 16, n = 8192.  attn_bwd (and attn_bwd_phase) take this form
 * whenever the call has it and workspace_bytes is at least this size; the
 * gradients agree with the recomputing form to rounding.  (Without dropout
 * the form is slower than the recomputation on MI355X, so it is not offered.)
 */
size_t attn_bwd_workspace_size_fast(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d,
                                    int dv, const attn_mask_t* mask, const attn_dropout_t* dropout);

/*
 * attn_bwd -- block-recomputed reverse pass ([P1] paragraphs 4-6, [P3]
 * "Reconstruct probabilities when a gradient needs them"): the exact gradient
 * of Phi = sum_i sum_a G_ia Y_ia,
 *
 *   D_i = sum_a G_ia Y_ia,   p_ij = e^{s_ij - LSE_i} on A_i,
 *   gamma_ij = p_ij (kappa_ij G_i . V_j - D_i),  kappa = xi / (1 - rate),
 *   dQ_i = c sum_j gamma_ij K_j,  dK_j = c sum_i gamma_ij Q_i,
 *   dV_j = sum_i p_ij kappa_ij G_i,
 *
 * with dK, dV of all query heads of a group summed into the shared head.
 * Arguments as attn_fwd, plus
 *   Y, LSE    exactly what attn_fwd wrote for the same inputs
 *   G         [B][H][n_q][dv] upstream gradient
 *   dQ, dK, dV  outputs shaped like Q, K, V
 *   workspace   device memory of at least attn_bwd_workspace_size() bytes,
 *               16-byte aligned; contents on entry are ignored.  With at
 *               least attn_bwd_workspace_size_fast() bytes (dropout with a
 *               causal / window mask) the stored-gamma form runs
 */
attn_status attn_bwd(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d, int dv,
                     const void* Q, const void* K, const void* V, const void* Y, const float* LSE,
                     const void* G, const attn_mask_t* mask, float scale, int block_b,
                     const attn_dropout_t* dropout, void* dQ, void* dK, void* dV,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_phase -- the three launches of attn_bwd, selectable, for callers
 * that schedule them themselves (for instance the dK/dV and dQ phases on two
 * streams once the prepass is done) or time them one by one.  `phases` is a
 * bit set: 1 = the prepass D_i = G_i . Y_i into the workspace, 2 = dK and dV,
 * 4 = dQ; phases 2 and 4 read the D_i a completed phase 1 left in the same
 * workspace and are independent of each other, except in the stored-gamma
 * form (a workspace of attn_bwd_workspace_size_fast() bytes), where phase 4
 * reads the gamma tiles phase 2 wrote and must follow it.  attn_bwd is
 * phases = 7.
 * Pointers a selected phase does not use may be NULL (phase 1 reads Y and G;
 * phases 2 and 4 read Q, K, V, LSE and G; phase 2 writes dK, dV; phase 4
 * writes dQ).  Other arguments and errors as attn_bwd; phases outside 1..7
 * is ATTN_ERR_INVALID_ARG.
 */
attn_status attn_bwd_phase(int phases, attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k,
                           int d, int dv, const void* Q, const void* K, const void* V,
                           const void* Y, const float* LSE, const void* G,
                           const attn_mask_t* mask, float scale, int block_b,
                           const attn_dropout_t* dropout, void* dQ, void* dK, void* dV,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and results as attn_bwd, without the
 * workspace arguments: the workspace is a fixed 16 MiB device array inside the
 * library (each GPU holds its own copy until the process ends).  Nothing is
 * allocated or freed.  Limit: attn_bwd_workspace_size() of the call at most
 * 16 MiB, i.e. B * H * n_q <= 2,097,088 query rows; beyond it the call returns
 * ATTN_ERR_WORKSPACE and launches nothing.  Every call on one GPU uses that
 * GPU's array: calls ordered on one stream are safe (each writes the array
 * before reading it), but calls that overlap in time on one GPU (other streams
 * or threads) race and give wrong gradients.
 */
attn_status attn_bwd_noalloc(attn_dtype dt, int B, int H, int H_kv, int n_q, int n_k, int d, int dv,
                             const void* Q, const void* K, const void* V, const void* Y, const float* LSE,
                             const void* G, const attn_mask_t* mask, float scale, int block_b,
                             const attn_dropout_t* dropout, void* dQ, void* dK, void* dV, void* stream);

/*
 * attn_sparse_fwd -- shared-KV top-k sparse attention with sink ([P5]
 * sections 1, 2 and 7.1).  For token t and head h, with the selected rows
 * I = topk_idx[t][0 : L_t] (L_t = topk_length[t], or topk when NULL):
 *
 *   s_u = scale * KV[I_u][0:d_qk] . Q[t][h],   Z = e^{z_h} + sum_u e^{s_u},
 *   O[t][h] = sum_u (e^{s_u} / Z) KV[I_u][0:d_v],   LSE[t][h] = ln Z,
 *
 * where z_h = attn_sink[h] (no sink when attn_sink is NULL: z = -inf).  The
 * exported LSE is sink-inclusive.
 *   dt           ATTN_BF16 or ATTN_F16
 *   Q            [Tq][H][d_qk];  KV [Tkv][d_qk] (the value is its first d_v columns)
 *   topk_idx     int32 [Tq][topk]; entries < L_t must lie in [0, Tkv), the
 *                rest are never read; duplicates are allowed.  An entry
 *                outside [0, Tkv) is not checked on the normal path: it
 *                reads as an all-zero row (score 0, value 0), no memory
 *                outside KV is touched and the backward drops its dKV
 *                contribution (the debug checks reject it)
 *   topk_length  int32 [Tq], values in [0, topk] (clamped into it; rejected by
 *                the debug checks), or NULL
 *   attn_sink    fp32 [H] or NULL
 *   O            [Tq][H][d_v] output;  LSE fp32 [Tq][H] output
 * Shapes: H == 64, d_qk == 576, d_v == 512.  A token with no selected row
 * gets O = 0 and LSE = z_h (-inf without a sink).
 */
attn_status attn_sparse_fwd(attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v, int topk,
                            const void* Q, const void* KV, const int32_t* topk_idx,
                            const int32_t* topk_length, const float* attn_sink, float scale,
                            void* O, float* LSE, void* stream);

/*
 * LSE conventions of the sparse path ([P5] sections 7.1-7.2).  ATTN_LSE_TOTAL:
 * ln(e^{z_h} + sum_u e^{s_u}), the sink included (attn_sparse_fwd's export).
 * ATTN_LSE_KV: ln sum_u e^{s_u} over the selected KV logits only (-inf for a
 * token with no selected row), as some sparse forward contracts return it; a
 * backward pass given it first forms LSE_total = logaddexp(LSE_kv, z_h) and
 * reconstructs every probability from that.
 */
typedef enum { ATTN_LSE_TOTAL = 0, ATTN_LSE_KV = 1 } attn_lse_kind;

/*
 * attn_sparse_fwd_lse -- attn_sparse_fwd with the LSE exported in convention
 * `kind` (O is the same either way).  INVALID_ARG for any other kind.
 */
attn_status attn_sparse_fwd_lse(attn_lse_kind kind, attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v,
                                int topk, const void* Q, const void* KV, const int32_t* topk_idx,
                                const int32_t* topk_length, const float* attn_sink, float scale, void* O,
                                float* LSE, void* stream);

/* Bytes of device workspace attn_sparse_bwd needs (fp32 D and sink-gradient
 * terms per (token, head), and an fp32 [Tkv][d_qk] dKV accumulator). */
size_t attn_sparse_bwd_workspace_size(int Tq, int H, int Tkv, int d_qk, int d_v, int topk);

/*
 * attn_sparse_bwd -- gradients of the sparse operator ([P5] sections 3 and
 * 8):  D = dO . O;  dS_u = p_u (dO . v_u - D);  dQ = scale sum_u dS_u k_u;
 * dKV[I_u][:] += scale dS_u q and dKV[I_u][0:d_v] += p_u dO (the tied K/V row),
 * summed over every token and head in fp32 and rounded once;
 * dSink[h] = -sum_t p_sink(t, h) D(t, h).
 * Arguments as attn_sparse_fwd, plus O and LSE as attn_sparse_fwd wrote them,
 * dO [Tq][H][d_v], outputs dQ [Tq][H][d_qk], dKV [Tkv][d_qk] and dSink fp32 [H]
 * (required iff attn_sink is not NULL), and the workspace (256-byte aligned,
 * at least attn_sparse_bwd_workspace_size() bytes; contents on entry are
 * ignored).  dKV is summed with fp32 atomics, so its bits may differ between
 * runs; dSink is summed over tokens in a fixed order.
 */
attn_status attn_sparse_bwd(attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v, int topk,
                            const void* Q, const void* KV, const int32_t* topk_idx,
                            const int32_t* topk_length, const float* attn_sink, float scale,
                            const void* O, const float* LSE, const void* dO, void* dQ, void* dKV,
                            float* dSink, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_sparse_bwd_lse -- attn_sparse_bwd for an LSE saved in convention
 * `kind` (see attn_lse_kind); with ATTN_LSE_KV and a sink, LSE_total =
 * logaddexp(LSE_kv, z_h) is formed per (token, head) before any probability
 * is reconstructed ([P5] section 7.2).  INVALID_ARG for any other kind.
 */
attn_status attn_sparse_bwd_lse(attn_lse_kind kind, attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v,
                                int topk, const void* Q, const void* KV, const int32_t* topk_idx,
                                const int32_t* topk_length, const float* attn_sink, float scale,
                                const void* O, const float* LSE, const void* dO, void* dQ, void* dKV,
                                float* dSink, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_sparse_bwd_det needs (as
 * attn_sparse_bwd_workspace_size, with a 64-bit [Tkv][d_qk] accumulator). */
size_t attn_sparse_bwd_det_workspace_size(int Tq, int H, int Tkv, int d_qk, int d_v, int topk);

/*
 * attn_sparse_bwd_det -- attn_sparse_bwd_lse with a bit-reproducible dKV
 * ([P5] section 9 notes that fp32 atomics make dKV order dependent; here the
 * order stops mattering instead of being fixed): every contribution
 * alpha dS_u q + p_u dO to
 * dKV[I_u] is rounded to a multiple of 2^-32 and added as a 64-bit integer, so
 * the total is the same for any order of the additions and dKV is bit
 * reproducible from run to run; it is converted to fp32 and then rounded once
 * to the storage dtype.  Requires |dKV| < 2^31 element-wise.  dQ and dSink
 * are as attn_sparse_bwd (already deterministic).  The workspace must hold
 * attn_sparse_bwd_det_workspace_size() bytes.
 */
attn_status attn_sparse_bwd_det(attn_lse_kind kind, attn_dtype dt, int Tq, int H, int Tkv, int d_qk, int d_v,
                                int topk, const void* Q, const void* KV, const int32_t* topk_idx,
                                const int32_t* topk_length, const float* attn_sink, float scale,
                                const void* O, const float* LSE, const void* dO, void* dQ, void* dKV,
                                float* dSink, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_dropout_mask -- writes the dropout realisation xi that attn_fwd and
 * attn_bwd use (see attn_dropout_t) as uint8 [B][H][n_q][n_k] (1 = kept), for
 * inspection and tests.
 */
attn_status attn_dropout_mask(float rate, uint64_t seed, int B, int H, int n_q, int n_k,
                              uint8_t* xi, void* stream);

/*
 * attn_mfma_probe -- measurement aid, not part of the method: launches one
 * workgroup of 4 * waves_per_simd waves (1 or 2) on every compute unit, each
 * wave issuing iters x 8 dense bf16 v_mfma_f32_32x32x16 with no memory
 * traffic, so that the caller can time the launch and report the MFMA rate
 * the device sustains beside the datasheet peak.  sink: device float buffer of
 * sink_len >= number of compute units (receives one value per workgroup).
 * *mfmas (host) receives the number of MFMA instructions issued
 * (32x32x16x2 = 32768 flops each).  INVALID_ARG for waves_per_simd outside
 * {1, 2}, iters < 1, null pointers or a sink shorter than the CU count.
 */
attn_status attn_mfma_probe(int waves_per_simd, int iters, float* sink, int sink_len, long long* mfmas,
                            void* stream);

/*
 * attn_issue_probe -- measurement aid, not part of the method: as
 * attn_mfma_probe (one workgroup of 4 * waves_per_simd waves per compute unit,
 * iters x 8 bf16 v_mfma_f32_32x32x16 per wave, four accumulators), with
 * valu_per_mfma (0, 2, 4, 6, 8 or 12) independent vector instructions issued
 * after each MFMA: fp32 FMAs (trans = 0) or base-2 exponentials, v_exp_f32
 * (trans = 1), so that the caller can measure how much vector-ALU work the
 * device hides under matrix instructions.  *mfmas receives the MFMA count.
 * INVALID_ARG for other valu_per_mfma or trans values and as attn_mfma_probe.
 */
attn_status attn_issue_probe(int waves_per_simd, int valu_per_mfma, int trans, int iters, float* sink, int sink_len,
                             long long* mfmas, void* stream);

/*
 * attn_atomic_probe -- measurement aid, not part of the method: fp32 atomic
 * adds of 1.0 into rows of `table` (device, [rows][576] floats, caller-owned
 * and -initialised), in the sparse dKV scatter's pattern (each instruction
 * covers 4 rows x 16 consecutive floats; 576 adds per row visit).  blocks
 * workgroups of 4 waves each visit groups_per_wave x 4 rows per wave, row
 * numbers taken cyclically from idx[0 .. n_idx) (device int32; entries outside
 * [0, rows) are skipped).  *adds (host) receives the number of adds issued.
 */
attn_status attn_atomic_probe(float* table, int rows, const int32_t* idx, int n_idx, int blocks, int groups_per_wave,
                              long long* adds, void* stream);

/*
 * attn_lds_probe -- measurement aid, not part of the method: one workgroup of
 * waves_per_cu (4, 8 or 16) waves on every compute unit fills 64 KiB of LDS,
 * then each wave issues iters x 16 conflict-free 16-byte-per-lane LDS reads,
 * so that the caller can time the launch and report the LDS read bandwidth
 * the device sustains.  sink: device uint32 buffer of sink_len >= number of
 * compute units.  *bytes (host) receives the bytes read from LDS.
 * INVALID_ARG for other wave counts, iters < 1, null pointers or a short sink.
 */
attn_status attn_lds_probe(int waves_per_cu, int iters, uint32_t* sink, int sink_len, long long* bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* attn_status_string(attn_status status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TILED_SOFTMAX_ATTN_H */
