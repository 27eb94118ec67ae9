/*
 * dar.h -- C ABI of the DAR (Distance-Adaptive Representation) attention
 * forward pass for AMD Instinct MI355X (gfx950).
 *
 * Method: "Dual Dimensionality for Local and Global Attention".
 *   Eq. (1)  h^D_j = h_j W_down                     (W_down in R^{d x d_down})
 *   Eq. (2)  h'_j  = h^D_j W_up                     (W_up   in R^{d_down x d})
 *   Eq. (3)  k_j = RoPE(h_j W_K), v_j = h_j W_V     if i - j <  w   (local path)
 *            k_j = RoPE(h'_j W_K), v_j = h'_j W_V   otherwise       (global path)
 *   Eq. (4)  o_i = softmax(q_i K_i^T / sqrt(d_k)) V_i, q_i = h_i W_Q, causal j <= i
 * The paper writes one head; several heads apply the one-head form head by
 * head (the paragraph before Eq. (2)); one W_down / W_up serves all heads.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers are DEVICE pointers, owned by the caller.  The library
 *    never allocates, keeps no state between calls and is re-entrant.
 *  - Work is enqueued on `stream` (NULL = the default stream); calls return
 *    after enqueue.  Device faults surface at the caller's next sync.
 *  - Activations are row-major with the innermost index contiguous.
 *  - WEIGHTS ARE COLUMN-MAJOR: a matrix W in R^{r x c} of the equations is
 *    stored with element (row k, column n) at offset n*r + k, i.e. each
 *    output column is contiguous.  These are the same bytes as a row-major
 *    [c, r] array (the layout of a torch.nn.Linear weight).  The MFMA GEMMs
 *    read both operands along the contraction index, so no transpose runs.
 *    A caller holding the equations' matrices row-major (W in R^{in x out}
 *    with each row contiguous, right-multiplied by row vectors h) packs each
 *    one once with dar_pack_weight.
 *  - Internal formats: the prefill intermediates dar_project writes and
 *    dar_attn_prefill reads are the library's own format, not the
 *    equations' layout: V_loc and V_glob are stored transposed per head
 *    ([B, heads, d_k, N], token innermost, the operand order of the
 *    attention's value product) and, in DAR_BF16 mode, all six are fp16.
 *  - dtype DAR_BF16: the layer's inputs and outputs (h, the weights, the
 *    folded weights, o, and the decode cache q / K_win / V_win / h_D) are
 *    bfloat16.  The six prefill intermediates that dar_project hands to
 *    dar_attn_prefill (Q, K_loc, V_loc, h_D, K_glob, V_glob) are IEEE fp16:
 *    same size and MFMA rate, 3 more mantissa bits, which keeps the
 *    end-to-end error several times inside 2e-2.  Their range is fp16's:
 *    an intermediate element of magnitude >= 65520 is stored as +-inf
 *    (round to nearest even), and the attention rows that read it come out
 *    inf or NaN; no status reports it, since the values exist only on the
 *    device.  Magnitudes up to 65504 are exact to fp16 rounding.  (The
 *    fp32 mode has no such limit.)  Arithmetic is MFMA with fp32 accumulation,
 *    softmax in fp32.  DAR_FP32: every float tensor is float32 and every
 *    step is computed in fp32 (no 16-bit rounding anywhere).
 *  - Positions are 0-based: token n of a prefill sits at position pos0 + n.
 *    RoPE uses rotate-half pairs (t, t + d_k/2) over the full head width with
 *    theta_t = rope_base^(-2t/d_k), applied to queries and keys alike.
 *  - Workspace protocol: if `workspace` is NULL the call writes the bytes it
 *    needs to *workspace_bytes and returns DAR_OK without touching the
 *    device.  Otherwise *workspace_bytes must be at least that size
 *    (DAR_ERR_WORKSPACE if not).  Workspace must be 256-byte aligned.
 *  - Validation happens before any device work; on an error nothing is
 *    launched and no output is written.  DAR_ERR_INVALID_ARG: null or
 *    misaligned (16 B) pointer, a size < 1 (w < 0, pos0 < 0), an odd d_k.
 *    DAR_ERR_UNSUPPORTED: outside the kernels' limits (d_k in {64, 128};
 *    d % 64 == 0; d_down % 32 == 0, d_down <= 1024; heads*d_k % 64 == 0).
 *    DAR_ERR_HIP: a launch reported an error.
 */
#ifndef DAR_H
#define DAR_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DAR_OK = 0,
  DAR_ERR_INVALID_ARG = 1,
  DAR_ERR_UNSUPPORTED = 2,
  DAR_ERR_WORKSPACE = 3,
  DAR_ERR_HIP = 4
} dar_status;

typedef enum { DAR_FP32 = 0, DAR_BF16 = 1 } dar_dtype;

/* Version of this ABI (bumped on any signature or layout change). */
int dar_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* dar_status_string(dar_status s);

/*
 * dar_pack_weight -- one of the equations' weight matrices in the library's
 * layout.  W is W in R^{rows x cols} row-major (element (k, n) at
 * k*cols + n: W_down [d x d_down], W_up [d_down x d], W_Q / W_K / W_V
 * [d x heads*d_k] as Eqs. (1)-(4) write them); W_packed receives the same
 * matrix column-major (element (k, n) at n*rows + k), the layout every other
 * entry point reads.  A transpose, bit-exact, in dtype (bf16 or fp32).
 * W_packed must not overlap W.  No workspace.
 */
dar_status dar_pack_weight(const void* W, int rows, int cols, dar_dtype dtype, void* W_packed,
                           hipStream_t stream);

/*
 * dar_fold -- fold the up-projection into the shared key/value weights.
 *
 * Eqs. (2)-(3): the global path applies W_K and W_V to h'_j = h^D_j W_up, so
 * h'_j W_K = h^D_j (W_up W_K).  This computes
 *     W_upK = W_up W_K,   W_upV = W_up W_V      (both d_down x heads*d_k)
 * in fp32 and stores them in `dtype`, column-major like every weight (i.e.
 * as row-major [heads*d_k, d_down]).  Run once per weight set.
 *   W_up [d_down x d], W_K, W_V [d x heads*d_k]      (column-major, dtype)
 * No workspace.
 */
dar_status dar_fold(const void* W_up, const void* W_K, const void* W_V, int d, int d_down,
                    int heads, int d_k, dar_dtype dtype, void* W_upK, void* W_upV,
                    hipStream_t stream);

/*
 * dar_project -- the projections of Eqs. (1)-(3) and q_i = h_i W_Q (Eq. 4).
 *
 *   h      [B, N, d]                       hidden states, token n at pos0+n
 *   W_down [d x d_down], W_Q, W_K, W_V [d x heads*d_k]      (column-major)
 *   W_up   [d_down x d]                    used only when W_upK/W_upV are NULL
 *   W_upK, W_upV [d_down x heads*d_k]      folded weights from dar_fold, or
 *                                          both NULL: the call folds them into
 *                                          its workspace first
 * Outputs (each written in full; fp16 in DAR_BF16 mode, fp32 in DAR_FP32):
 *   Q      [B, heads, N, d_k]   RoPE(h W_Q) at the token's position
 *   K_loc  [B, heads, N, d_k]   RoPE(h W_K)                 (Eq. 3, local)
 *   V_loc  [B, heads, d_k, N]   h W_V, TRANSPOSED per head (token innermost)
 *   h_D    [B, N, d_down]       h W_down                    (Eq. 1)
 *   K_glob [B, heads, N, d_k]   RoPE(h^D W_upK) = RoPE(h' W_K)  (Eq. 3, global)
 *   V_glob [B, heads, d_k, N]   h^D W_upV = h' W_V, transposed like V_loc
 * In bf16 mode h^D is rounded to fp16 before the global GEMM (it is the
 * stored latent).  Outputs must not alias inputs or each other.
 */
dar_status dar_project(const void* h, const void* W_down, const void* W_up, const void* W_Q,
                       const void* W_K, const void* W_V, const void* W_upK, const void* W_upV,
                       int B, int N, int d, int d_down, int heads, int d_k, int pos0,
                       float rope_base, dar_dtype dtype, void* Q, void* K_loc, void* V_loc,
                       void* h_D, void* K_glob, void* V_glob, void* workspace,
                       size_t* workspace_bytes, hipStream_t stream);

/*
 * dar_project_sigmoid -- dar_project for the variant that applies a sigmoid
 * after the down-projection of Eq. (1) ("Dual Dimensionality for Local and
 * Global Attention", the paragraph after Eq. (1): evaluated by the authors,
 * found comparable to the linear form, not adopted):
 *   h_D    [B, N, d_down]       sigma(h W_down),  sigma(x) = 1 / (1 + e^-x)
 *   K_glob, V_glob              from that h^D through the same folded weights
 * elementwise, in fp32, before h^D is rounded to its storage type.  Q, K_loc
 * and V_loc are those of dar_project.  Arguments, layouts, workspace and
 * errors are those of dar_project.  A model with this variant builds its
 * decode cache from this call's h_D (dar_cache_from_prefill) and extends it
 * with the *_sigmoid forms of dar_decode_append(_varlen) and
 * dar_prefill_chunk, which store sigma(h W_down) as the latent row; the
 * decode attention itself (dar_attn_decode) reads whatever latent is stored.
 */
dar_status dar_project_sigmoid(const void* h, const void* W_down, const void* W_up,
                               const void* W_Q, const void* W_K, const void* W_V,
                               const void* W_upK, const void* W_upV, int B, int N, int d,
                               int d_down, int heads, int d_k, int pos0, float rope_base,
                               dar_dtype dtype, void* Q, void* K_loc, void* V_loc, void* h_D,
                               void* K_glob, void* V_glob, void* workspace,
                               size_t* workspace_bytes, hipStream_t stream);

/*
 * dar_attn_prefill -- Eq. (4) with the Eq. (3) distance selection, causal.
 *
 * For query i and key j <= i of the same sequence and head, the key/value
 * pair comes from (K_loc, V_loc) when i - j < w and from (K_glob, V_glob)
 * otherwise; w = 0 sends every pair (j = i included) to the global path,
 * w >= N every pair to the local path.
 *   Q, K_loc, K_glob   [B, heads, N, d_k]   (fp16 in DAR_BF16 mode)
 *   V_loc, V_glob      [B, heads, d_k, N]   (token innermost, as dar_project writes)
 *   o                  [B, N, heads*d_k]    heads concatenated, before W_O
 *                                           (bf16 in DAR_BF16 mode)
 * The kernel needs no workspace: with workspace NULL and workspace_bytes
 * non-NULL the call validates, writes 0 and launches nothing (the size
 * query of the protocol); otherwise it launches, and workspace_bytes may be
 * NULL.
 */
dar_status dar_attn_prefill(const void* Q, const void* K_loc, const void* V_loc,
                            const void* K_glob, const void* V_glob, int B, int N, int heads,
                            int d_k, int w, dar_dtype dtype, void* o, void* workspace,
                            size_t* workspace_bytes, hipStream_t stream);

/*
 * Ragged prefill: a batch of B prompts of different lengths without padding
 * (the inference remark after Eq. (5): a serving batch holds prompts of
 * several lengths).  cu_seqlens (device, int32, B + 1 entries, nondecreasing,
 * cu_seqlens[0] = 0, cu_seqlens[B] = T) puts prompt b at rows
 * cu_seqlens[b] .. cu_seqlens[b+1]-1 of the packed input; its tokens sit at
 * positions 0, 1, ... of their own prompt; max_len bounds every length (the
 * RoPE tables' reach).  The packed intermediates hold one block per prompt,
 * at element offset cu_seqlens[b] * heads * d_k, laid out as a one-prompt
 * dar_project would (Q, K_loc, K_glob [heads, len_b, d_k]; V_loc, V_glob
 * [heads, d_k, len_b]); h_D is [T, d_down].  bf16 mode only.  The lengths are
 * read on the device only: inconsistent values are clamped so that every
 * access stays in bounds, and the rows they describe are not computed.
 *
 * dar_project_varlen -- Eqs. (1)-(3) and q = h W_Q over h [T, d]; weights,
 * folded weights and workspace as for dar_project (the query covers max_len
 * positions).
 */
dar_status dar_project_varlen(const void* h, const void* W_down, const void* W_up,
                              const void* W_Q, const void* W_K, const void* W_V,
                              const void* W_upK, const void* W_upV, const int* cu_seqlens, int B,
                              int T, int max_len, int d, int d_down, int heads, int d_k,
                              float rope_base, dar_dtype dtype, void* Q, void* K_loc,
                              void* V_loc, void* h_D, void* K_glob, void* V_glob,
                              void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * dar_attn_prefill_varlen -- Eq. (4) with the Eq. (3) selection for every
 * prompt of a ragged batch, from dar_project_varlen's packed outputs;
 * o [T, heads*d_k] (bf16), row t the query at packed row t.  No workspace.
 */
dar_status dar_attn_prefill_varlen(const void* Q, const void* K_loc, const void* V_loc,
                                   const void* K_glob, const void* V_glob, const int* cu_seqlens,
                                   int B, int T, int max_len, int heads, int d_k, int w,
                                   dar_dtype dtype, void* o, hipStream_t stream);

/*
 * dar_cache_from_prefill_packed -- the decode cache of a ragged batch
 * prefilled without padding (the inference remark after Eq. (5)): from
 * dar_project_varlen's packed h_D [T, d_down], K_loc and V_loc (fp16, one
 * block per prompt as above), for every prompt b of length
 * len_b = cu_seqlens[b+1] - cu_seqlens[b]:
 *   h_D_cache[b, n, :]       <- h_D[cu_seqlens[b] + n, :]   for n < len_b
 *   K_win[b, :, j mod w, :]  <- prompt b's K_loc[:, j, :]   for max(0, len_b-w) <= j < len_b
 *   V_win[b, :, j mod w, :]  <- prompt b's V_loc[:, :, j]
 * leaving every other row and slot untouched; h_D_cache [B, cap, d_down]
 * with cap >= max_len, K_win and V_win [B, heads, w, d_k] (bf16; ignored, may
 * be NULL, when w = 0).  Values are rounded fp16 -> bf16 (nearest even).  The
 * next token of prompt b sits at position len_b (dar_decode_append_varlen with
 * pos[b] = len_b, then dar_attn_decode_varlen with ctx_lens[b] = len_b + 1).
 * DAR_BF16 only; d_down a multiple of 8.  No workspace.
 */
dar_status dar_cache_from_prefill_packed(const void* h_D, const void* K_loc, const void* V_loc,
                                         const int* cu_seqlens, int B, int T, int max_len,
                                         int heads, int d_k, int d_down, int w, int cap,
                                         dar_dtype dtype, void* h_D_cache, void* K_win,
                                         void* V_win, hipStream_t stream);

/*
 * dar_attn_prefill_lse -- dar_attn_prefill that also stores, for training,
 * each query's softmax normaliser of Eq. (4):
 *   lse [B, heads, N] float32, lse_i = log sum_{j <= i} exp(q_i . k_j / sqrt(d_k))
 * (natural log, keys chosen by Eq. (3)).  o is identical to dar_attn_prefill's.
 * lse must be 16-byte aligned and must not alias an input or o.
 */
dar_status dar_attn_prefill_lse(const void* Q, const void* K_loc, const void* V_loc,
                                const void* K_glob, const void* V_glob, int B, int N, int heads,
                                int d_k, int w, dar_dtype dtype, void* o, float* lse,
                                hipStream_t stream);

/*
 * dar_attn_prefill_backward -- gradients of dar_attn_prefill for dL/do = dO.
 *
 * Training remark after Eq. (4): each past token keeps both representations
 * and each (i, j) pair is served by the one Eq. (3) selects, so its gradient
 * reaches only that source (the bottleneck weights learn from global pairs).
 * With s_ij = q_i . k_j / sqrt(d_k), p_ij = softmax over j <= i,
 * dp_ij = dO_i . v_j, D_i = dO_i . o_i and ds_ij = p_ij (dp_ij - D_i):
 *   dQ_i = sum_j ds_ij k_j / sqrt(d_k);  dK_j += ds_ij q_i / sqrt(d_k);
 *   dV_j += p_ij dO_i   (K, V, dK, dV of the pair's source).
 *   Q, K_loc, V_loc, K_glob, V_glob, w   exactly as given to dar_attn_prefill
 *                                        (fp16 in DAR_BF16 mode; V transposed)
 *   o, dO   [B, N, heads*d_k]            the forward output and its gradient
 *                                        (bf16 in DAR_BF16 mode; dO within the
 *                                        fp16 range: it enters fp16 products)
 *   lse     [B, heads, N] float32 or NULL  the forward's normaliser from
 *                                        dar_attn_prefill_lse; NULL: recomputed
 *                                        here (one more pass over the scores)
 * Outputs, float32 in both modes, each written in full:
 *   dQ, dK_loc, dK_glob, dV_loc, dV_glob [B, heads, N, d_k]  (dV NOT transposed)
 * Workspace: 8*B*heads*N bytes (rounded) for the per-query log-sum-exp and D.
 * Outputs must not alias inputs, each other or the workspace.  Supported:
 * d_k in {64, 128}.  DAR_BF16 runs fp16 MFMAs with fp32 accumulation (P and
 * dS rounded to fp16); DAR_FP32 runs fp32 on the VALU.
 */
dar_status dar_attn_prefill_backward(const void* Q, const void* K_loc, const void* V_loc,
                                     const void* K_glob, const void* V_glob, const void* o,
                                     const void* dO, const float* lse, int B, int N, int heads,
                                     int d_k, int w, dar_dtype dtype, float* dQ, float* dK_loc,
                                     float* dV_loc, float* dK_glob, float* dV_glob,
                                     void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream);

/*
 * dar_decode_append -- project one new token per sequence into the mixed cache.
 *
 * The inference remark after Eq. (5) (each past token is used through exactly
 * one path) and the O(T d_down + w d) cache of the efficiency analysis: for
 * the new token at position `pos` of every sequence (all sequences share pos)
 *   q   [B, heads, d_k]       <- RoPE_pos(h W_Q)             (Eq. 4 text)
 *   K_win[b, :, pos mod w, :] <- RoPE_pos(h W_K)             (Eq. 3, local)
 *   V_win[b, :, pos mod w, :] <- h W_V
 *   h_D [b, pos, :]           <- h W_down                    (Eq. 1)
 * leaving every other slot and row untouched.  h [B, d]; weights column-major;
 * K_win, V_win [B, heads, w, d_k] (ignored when w = 0); h_D [B, cap, d_down]
 * with pos < cap.  bf16 only; workspace holds the RoPE tables (query with
 * workspace = NULL).  Then dar_attn_decode(ctx_len = pos + 1) attends.
 */
dar_status dar_decode_append(const void* h, const void* W_down, const void* W_Q, const void* W_K,
                             const void* W_V, int B, int d, int d_down, int heads, int d_k,
                             int pos, int w, int cap, float rope_base, dar_dtype dtype, void* q,
                             void* K_win, void* V_win, void* h_D, void* workspace,
                             size_t* workspace_bytes, hipStream_t stream);

/*
 * dar_decode_append_sigmoid -- dar_decode_append for the sigmoid-bottleneck
 * variant (the paragraph after Eq. (1)): the latent row written at `pos` is
 * sigma(h W_down), sigma(x) = 1 / (1 + e^-x), in fp32 before its bf16
 * rounding.  q and the ring slot are those of dar_decode_append; arguments,
 * workspace and errors likewise.
 */
dar_status dar_decode_append_sigmoid(const void* h, const void* W_down, const void* W_Q,
                                     const void* W_K, const void* W_V, int B, int d, int d_down,
                                     int heads, int d_k, int pos, int w, int cap, float rope_base,
                                     dar_dtype dtype, void* q, void* K_win, void* V_win, void* h_D,
                                     void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream);

/*
 * dar_prefill_chunk -- prefill the next C tokens of every sequence over the
 * mixed cache, and extend the cache.
 *
 * The chunk holds positions p0 .. p0+C-1 (N = p0 + C); its queries attend to
 * every position j <= i as in Eqs. (3)-(4): the chunk's own keys/values from
 * its projections, the prefix's through the cache the way decode reads it --
 * local pairs (i - j < w) from the ring, global pairs from the latents,
 * k_j = RoPE_j(h^D_j W_upK), v_j = h^D_j W_upV (Eqs. 2-3 with the fold).
 * Splitting a prompt into chunks therefore gives the rows of the whole
 * prefill (up to the bf16 rounding of the cache).
 *   h       [B, C, d]                   the chunk's hidden states (bf16)
 *   W_down, W_Q, W_K, W_V               column-major, as for dar_project
 *   W_upK, W_upV [d_down x heads*d_k]   folded weights (dar_fold)
 * Cache (bf16, updated in place; the layout of dar_cache_from_prefill):
 *   h_D_cache [B, cap, d_down]   rows 0 .. p0-1 read, rows p0 .. N-1 written
 *                                (cap >= N)
 *   K_win, V_win [B, heads, w, d_k]  positions max(0,p0-w) .. p0-1 read; on
 *                                return they hold positions max(0,N-w) .. N-1
 *                                (slot = position mod w; NULL when w = 0)
 *   o [B, C, heads*d_k]           the chunk's output rows (bf16)
 * Start from an empty cache with p0 = 0.  The workspace (query with NULL)
 * holds the chunk's projections and the prefix's rebuilt global keys and
 * values (O(B heads d_k N) fp16).  DAR_BF16 only; limits as dar_project.
 */
dar_status dar_prefill_chunk(const void* h, const void* W_down, const void* W_Q, const void* W_K,
                             const void* W_V, const void* W_upK, const void* W_upV, int B, int C,
                             int d, int d_down, int heads, int d_k, int p0, int w, int cap,
                             float rope_base, dar_dtype dtype, void* h_D_cache, void* K_win,
                             void* V_win, void* o, void* workspace, size_t* workspace_bytes,
                             hipStream_t stream);

/*
 * dar_prefill_chunk_sigmoid -- dar_prefill_chunk for the sigmoid-bottleneck
 * variant (the paragraph after Eq. (1)): the chunk's latents are
 * sigma(h W_down) (fp32, then stored), both in the latent cache and as the
 * source of the chunk's global keys and values; the prefix's latents are read
 * from the cache as stored.  Everything else is dar_prefill_chunk's.
 */
dar_status dar_prefill_chunk_sigmoid(const void* h, const void* W_down, const void* W_Q,
                                     const void* W_K, const void* W_V, const void* W_upK,
                                     const void* W_upV, int B, int C, int d, int d_down, int heads,
                                     int d_k, int p0, int w, int cap, float rope_base,
                                     dar_dtype dtype, void* h_D_cache, void* K_win, void* V_win,
                                     void* o, void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream);

/*
 * dar_cache_from_prefill -- the decode cache of a prefilled prompt.
 *
 * After a prompt of N tokens is prefilled, generation keeps the latent h^D of
 * every position (Eq. 1) and full keys/values for the w most recent positions
 * only (the inference remark after Eq. (5)).  This converts dar_project's
 * outputs into the cache dar_decode_append / dar_attn_decode use:
 *   h_D_cache[b, n, :]       <- h_D[b, n, :]          for n < N
 *   K_win[b, :, j mod w, :]  <- K_loc[b, :, j, :]     for max(0, N-w) <= j < N
 *   V_win[b, :, j mod w, :]  <- V_loc[b, :, :, j]     (V_loc is token-innermost)
 * leaving every other row and slot untouched.
 *   h_D [B, N, d_down], K_loc [B, heads, N, d_k], V_loc [B, heads, d_k, N]
 *                                   (fp16: dar_project's DAR_BF16 outputs)
 *   h_D_cache [B, cap, d_down] with cap >= N; K_win, V_win [B, heads, w, d_k]
 *                                   (bf16; ignored, may be NULL, when w = 0)
 * Values are rounded fp16 -> bf16 (nearest even).  The next token sits at
 * position N: dar_decode_append(pos = N), then dar_attn_decode(ctx_len = N+1).
 * DAR_BF16 only; d_down must be a multiple of 8.  No workspace.
 */
dar_status dar_cache_from_prefill(const void* h_D, const void* K_loc, const void* V_loc, int B,
                                  int N, int heads, int d_k, int d_down, int w, int cap,
                                  dar_dtype dtype, void* h_D_cache, void* K_win, void* V_win,
                                  hipStream_t stream);

/*
 * Ragged batches: sequences of different lengths in one call.
 *
 * A batch of prompts of lengths N_b <= N is prefilled either packed without
 * padding (dar_project_varlen, dar_attn_prefill_varlen,
 * dar_cache_from_prefill_packed) or padded to N (dar_project and
 * dar_attn_prefill as usual): attention is causal, so the rows n < N_b of
 * sequence b do not depend on its padding and equal those of an unpadded
 * prefill up to rounding.  From there on each sequence moves at its own
 * position.
 * The per-sequence lengths and positions are device int32 arrays of B entries
 * (caller-owned, 4-byte aligned, read by the kernels; they are never read on
 * the host, so values are not validated: each is clamped into range, which
 * keeps every access in bounds but gives meaningless results for bad values).
 *
 * dar_cache_from_prefill_varlen -- as dar_cache_from_prefill, with sequence b
 *   ending at lens[b] (1 <= lens[b] <= N): its ring gets the positions
 *   max(0, lens[b]-w) .. lens[b]-1.  Latent rows 0 .. N-1 are copied for every
 *   sequence (rows past lens[b] are never read by decode).
 * dar_decode_append_varlen -- as dar_decode_append, with sequence b's token at
 *   position pos[b] (0 <= pos[b] < cap): RoPE at pos[b], ring slot pos[b] mod w,
 *   latent row pos[b].  The workspace holds RoPE tables up to cap - 1.
 * dar_attn_decode_varlen -- as dar_attn_decode, with sequence b's query at
 *   position ctx_lens[b] - 1 (1 <= ctx_lens[b] <= max_ctx, max_ctx - w < cap
 *   when max_ctx > w).  The work split and workspace follow max_ctx;
 *   workgroups past a sequence's end return after writing empty partials.
 */
dar_status dar_cache_from_prefill_varlen(const void* h_D, const void* K_loc, const void* V_loc,
                                         int B, int N, const int* lens, int heads, int d_k,
                                         int d_down, int w, int cap, dar_dtype dtype,
                                         void* h_D_cache, void* K_win, void* V_win,
                                         hipStream_t stream);
dar_status dar_decode_append_varlen(const void* h, const void* W_down, const void* W_Q,
                                    const void* W_K, const void* W_V, int B, int d, int d_down,
                                    int heads, int d_k, const int* pos, int w, int cap,
                                    float rope_base, dar_dtype dtype, void* q, void* K_win,
                                    void* V_win, void* h_D, void* workspace,
                                    size_t* workspace_bytes, hipStream_t stream);
/* dar_decode_append_varlen_sigmoid -- the ragged append of the sigmoid
 * variant: latent row pos[b] <- sigma(h_b W_down) (as dar_decode_append_sigmoid). */
dar_status dar_decode_append_varlen_sigmoid(const void* h, const void* W_down, const void* W_Q,
                                            const void* W_K, const void* W_V, int B, int d,
                                            int d_down, int heads, int d_k, const int* pos, int w,
                                            int cap, float rope_base, dar_dtype dtype, void* q,
                                            void* K_win, void* V_win, void* h_D, void* workspace,
                                            size_t* workspace_bytes, hipStream_t stream);
dar_status dar_attn_decode_varlen(const void* q, const void* K_win, const void* V_win,
                                  const void* h_D, const void* W_upK, const void* W_upV, int B,
                                  const int* ctx_lens, int max_ctx, int cap, int heads, int d_k,
                                  int d_down, int w, float rope_base, dar_dtype dtype, void* o,
                                  void* workspace, size_t* workspace_bytes, hipStream_t stream);

/*
 * dar_attn_decode -- one new query per sequence over the mixed cache.
 *
 * At inference a past token is seen by a query through one source only,
 * chosen by its distance (the remark after Eq. (5)), so a decode cache needs
 * full keys/values for the w most recent positions and the d_down-wide latent
 * h^D for older ones.
 * The query sits at position p = ctx_len - 1 (its own key/value already in
 * the window).
 *   q      [B, heads, d_k]          RoPE'd at p
 *   K_win  [B, heads, w, d_k]       RoPE'd keys of positions max(0,p-w+1)..p,
 *   V_win  [B, heads, w, d_k]       values; position j lives in slot j mod w
 *   h_D    [B, cap, d_down]         latents; rows 0 .. p-w are read (cap >= p-w+1)
 *   W_upK, W_upV [d_down x heads*d_k]   folded weights (dar_fold), column-major
 *   o      [B, heads*d_k]
 * Global keys are rebuilt as RoPE_j(h^D_j W_upK); values are accumulated in
 * latent space and lifted once: sum_j p_j h^D_j W_upV = (sum_j p_j h^D_j) W_upV.
 * bf16 only (fp32 returns DAR_ERR_UNSUPPORTED); d_down in {32, 64, 128, 256, 512}
 * (others return DAR_ERR_UNSUPPORTED).
 */
dar_status dar_attn_decode(const void* q, const void* K_win, const void* V_win, const void* h_D,
                           const void* W_upK, const void* W_upV, int B, int ctx_len, int cap,
                           int heads, int d_k, int d_down, int w, float rope_base,
                           dar_dtype dtype, void* o, void* workspace, size_t* workspace_bytes,
                           hipStream_t stream);

/*
 * Decoupled-RoPE variant.  "Dual Dimensionality for Local and Global
 * Attention" names MLA's decoupled rotary embedding as the route to an
 * efficient implementation (the paragraph after the inference remark)
 * without writing it out.  Reading taken (MLA's construction on Eqs. 1-4):
 * every head's query and key carry a content part and a rotary part of width
 * d_R; only the rotary part is rotated;
 *   qC_i = h_i W_Q[:, S_a],  qR_i = RoPE_i(h_i W_QR[:, R_a])   (R_a: d_R columns of head a)
 *   kC_j = h_j W_K[:, S_a] if i - j < w, else h'_j W_K[:, S_a] (Eq. 3 without RoPE)
 *   kR_j = RoPE_j(h_j W_KR)   one rotary key per token, from the full hidden
 *                             state, shared by every head and both paths
 *   v_j as Eq. 3;  s_ij = (qC_i . kC_j + qR_i . kR_j) / sqrt(d_k + d_R).
 * RoPE over the rotary part: pairs (t, t + d_R/2), theta_t = base^(-2t/d_R).
 * Supported: d_R = 64 with d_k 64 or 128, bf16 mode.
 *
 * dar_attn_decode_drope -- one query per sequence at p = ctx_len - 1 over the
 * variant's cache.  With no rotation between W_upK and the query, the content
 * score of an old position is (W_upK_a^T qC_a) . h^D_j: the fold is absorbed
 * into the query once per step and the cache is streamed as [h^D_j ; kR_j]
 * for all heads at once (latent-space value sum, one lift by W_upV).
 *   qC     [B, heads, d_k]        content query
 *   qR     [B, heads, d_R]        rotary query, rotated at p
 *   K_win  [B, heads, w, d_k]     content keys (not rotated) of positions
 *   V_win  [B, heads, w, d_k]     p-w+1 .. p and their values, slot = pos mod w
 *   KR     [B, cap, d_R]          rotary keys of every position (rows 0 .. p read)
 *   h_D    [B, cap, d_down]       latents (rows 0 .. p-w read); cap >= ctx_len
 *   W_upK, W_upV                  folded weights from dar_fold
 *   o      [B, heads*d_k]
 * bf16 only; d_down in {128, 256, 512}.  Workspace (query with NULL): the
 * absorbed queries and the softmax partials.
 */
/*
 * dar_project_drope -- the variant's projections (bf16 mode; outputs fp16
 * like dar_project's):
 *   QC     [B, heads, N, d_k]   h W_Q (not rotated)
 *   QR     [B, heads, N, d_R]   RoPE(h W_QR) at the token's position
 *   K_loc  [B, heads, N, d_k]   h W_K (not rotated)
 *   V_loc  [B, heads, d_k, N]   h W_V, token innermost
 *   h_D    [B, N, d_down]       h W_down
 *   K_glob [B, heads, N, d_k]   h^D W_upK (not rotated)
 *   V_glob [B, heads, d_k, N]   h^D W_upV, token innermost
 *   KR     [B, N, d_R]          RoPE(h W_KR), one per token
 * Weights column-major as for dar_project: W_QR [d x heads*d_R], W_KR
 * [d x d_R]; W_upK / W_upV from dar_fold, or both NULL (folded into the
 * workspace, with W_up given).  Workspace (query with NULL): RoPE tables of
 * width d_R (and the fold).
 */
dar_status dar_project_drope(const void* h, const void* W_down, const void* W_up, const void* W_Q,
                             const void* W_K, const void* W_V, const void* W_QR, const void* W_KR,
                             const void* W_upK, const void* W_upV, int B, int N, int d,
                             int d_down, int heads, int d_k, int d_R, int pos0, float rope_base,
                             dar_dtype dtype, void* QC, void* QR, void* K_loc, void* V_loc,
                             void* h_D, void* K_glob, void* V_glob, void* KR, void* workspace,
                             size_t* workspace_bytes, hipStream_t stream);

/*
 * dar_attn_prefill_drope -- Eq. (4) of the variant, causal, with the Eq. (3)
 * selection on the content part: query i and key j <= i score
 * (QC_i . K_src,j + QR_i . KR_j) / sqrt(d_k + d_R), K_src / V_src the local
 * arrays when i - j < w and the global ones otherwise; o [B, N, heads*d_k]
 * (bf16).  Inputs in dar_project_drope's layouts (fp16).  No workspace.
 */
dar_status dar_attn_prefill_drope(const void* QC, const void* QR, const void* K_loc,
                                  const void* V_loc, const void* K_glob, const void* V_glob,
                                  const void* KR, int B, int N, int heads, int d_k, int d_R, int w,
                                  dar_dtype dtype, void* o, hipStream_t stream);

/*
 * dar_cache_from_prefill_drope -- the variant's decode cache of a prefilled
 * prompt: latent rows and ring slots as dar_cache_from_prefill (the ring holds
 * the content keys K_loc), plus KR_cache[b, n, :] <- KR[b, n, :] for n < N
 * (fp16 -> bf16).  KR_cache [B, cap, d_R].
 */
dar_status dar_cache_from_prefill_drope(const void* h_D, const void* K_loc, const void* V_loc,
                                        const void* KR, int B, int N, int heads, int d_k,
                                        int d_down, int d_R, int w, int cap, dar_dtype dtype,
                                        void* h_D_cache, void* K_win, void* V_win, void* KR_cache,
                                        hipStream_t stream);

/*
 * dar_decode_append_drope -- the variant's new token at position `pos` of
 * every sequence: qC <- h W_Q, qR <- RoPE_pos(h W_QR) ([B, heads, d_R]), the
 * ring slot pos mod w of K_win / V_win <- h W_K, h W_V (content keys, not
 * rotated), h_D[b, pos] <- h W_down, KR[b, pos] <- RoPE_pos(h W_KR).  bf16;
 * workspace: RoPE tables of width d_R.
 */
dar_status dar_decode_append_drope(const void* h, const void* W_down, const void* W_Q,
                                   const void* W_K, const void* W_V, const void* W_QR,
                                   const void* W_KR, int B, int d, int d_down, int heads, int d_k,
                                   int d_R, int pos, int w, int cap, float rope_base,
                                   dar_dtype dtype, void* qC, void* qR, void* K_win, void* V_win,
                                   void* h_D, void* KR, void* workspace, size_t* workspace_bytes,
                                   hipStream_t stream);

dar_status dar_attn_decode_drope(const void* qC, const void* qR, const void* K_win,
                                 const void* V_win, const void* KR, const void* h_D,
                                 const void* W_upK, const void* W_upV, int B, int ctx_len, int cap,
                                 int heads, int d_k, int d_R, int d_down, int w, dar_dtype dtype,
                                 void* o, void* workspace, size_t* workspace_bytes,
                                 hipStream_t stream);

/*
 * dar_attn_decode_noalloc -- dar_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * Arguments, layouts, results and errors are those of dar_attn_decode, minus
 * the workspace: the call allocates nothing and takes its scratch memory (the
 * RoPE tables and the per-chunk softmax partials) from a static device array
 * of 32 MiB that the library holds on each GPU it runs on until the process
 * ends.  A problem whose dar_attn_decode workspace exceeds 32 MiB returns
 * DAR_ERR_WORKSPACE without launching (about 4.7 MiB at batch 16, context
 * 32768, 16 heads of 128, d_down 256; the RoPE tables add 256 KiB per 64k
 * positions of context).  Every call on one GPU shares that GPU's array and
 * rewrites all of it that it reads, so nothing carries over between calls;
 * calls that overlap in time on one GPU (several streams or threads) race on
 * it and must be serialised by the caller.  DAR_ERR_HIP if the array's
 * device address cannot be obtained.
 */
dar_status dar_attn_decode_noalloc(const void* q, const void* K_win, const void* V_win,
                                   const void* h_D, const void* W_upK, const void* W_upV, int B,
                                   int ctx_len, int cap, int heads, int d_k, int d_down, int w,
                                   float rope_base, dar_dtype dtype, void* o,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DAR_H */
