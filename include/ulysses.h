/*
 * ulysses.h -- C ABI of the per-rank hot path of Ulysses sequence parallelism
 * on MI355X (gfx950).
 *
 * What the operations are (sources are the pages' titles and sections):
 *   - HF Transformers docs, "Ulysses sequence parallelism" (deepspeed_alst),
 *     opening paragraph and layout diagram: sp ranks each hold N/sp tokens of
 *     all H heads; an all-to-all moves them to all N tokens of H/sp heads per
 *     rank; attention runs there; a second all-to-all moves back.
 *   - congresoia365 article "Nuevo método Ulysses ...", section "Cómo Funciona
 *     Ulysses": the local attention is the standard mechanism, and heads are
 *     independent of one another.
 *   - The same guide, "sp_attn_implementation" paragraph: samples packed into
 *     one row must not attend across their boundaries.
 *   - congresoia365 article, section "El Desafío del Entrenamiento de
 *     Secuencias Largas": memory-efficient attention keeps O(N) state and
 *     never stores the N x N score matrix.
 *   - ColossalAI docs, "Sequence Parallelism": ring attention, the other
 *     sequence-parallel mode (the ulysses_ring_attn_* calls).
 *   - jianying88 guide to DeepSpeed Ulysses in Transformers, section on the
 *     work Trainer does by itself: the count-weighted loss across SP ranks
 *     (ulysses_sp_loss).
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is device memory owned by the caller, contiguous
 *     and row-major in the layout stated at the call. The library allocates
 *     no memory and keeps no state, except the fixed per-GPU scratch of
 *     ulysses_attn_bwd_noalloc (see there); every other call is safe to call
 *     from several host threads on different streams.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns; results are ready when
 *     the stream is.
 *   - Arguments are checked on the host before anything is enqueued; a call
 *     that returns an error has enqueued nothing. The contents of device
 *     buffers (e.g. cu_seqlens) are never read on the host.
 *   - For the permute and attention calls, dtype is ULY_F32 (float) or
 *     ULY_BF16 (bfloat16, round-to-nearest-even outputs); accumulation is
 *     always in fp32 or wider. Head width d must be 64 or 128.
 */
#ifndef ULYSSES_H
#define ULYSSES_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define ULY_OK 0
#define ULY_EINVAL 1       /* null pointer where one is required, or a size <= 0 */
#define ULY_ESHAPE 2       /* a size condition fails (each call lists its own) */
#define ULY_EUNSUPPORTED 3 /* dtype not ULY_F32/ULY_BF16, or d not in {64, 128} */
#define ULY_EWORKSPACE 4   /* workspace pointer NULL or smaller than required */
#define ULY_EHIP 5         /* the HIP runtime refused a launch */

/* Element types. */
#define ULY_F32 0
#define ULY_BF16 1

/*
 * Layout change of all-to-all #1 (sequence-sharded -> head-sharded) for sp
 * virtual ranks held on one device (guide, layout diagram, upper half).
 *   x_seq  [sp][B][N/sp][H][d]   shard s holds tokens [s*N/sp, (s+1)*N/sp) of all H heads
 *   x_head [sp][B][N][H/sp][d]   shard r holds all N tokens of heads [r*H/sp, (r+1)*H/sp)
 *   x_head[r][b][s*N/sp + t][h][:] = x_seq[s][b][t][r*H/sp + h][:]
 * N is the full sequence length. Elements are copied as raw bits (bit-exact,
 * NaN payloads and -0 kept). x_seq and x_head must not overlap and must be
 * 16-byte aligned.
 * Errors: ULY_EINVAL (null, size <= 0, overlap, misaligned); ULY_ESHAPE when
 * N % sp != 0, H % sp != 0, sp > 65535, sp * B >= 2^32, or one shard's
 * output counts 2^32 - 512 or more 16-byte chunks: (N/sp) * (H/sp) * d *
 * esize / 16 here, N * (H/sp) * d * esize / 16 for ulysses_head_to_seq
 * (esize = 4 for ULY_F32, 2 for ULY_BF16); ULY_EUNSUPPORTED (dtype, d);
 * ULY_EHIP.
 */
int ulysses_seq_to_head(const void* x_seq, void* x_head, int B, int N, int H, int d, int sp,
                        int dtype, void* stream);

/*
 * Layout change of all-to-all #2 (head-sharded -> sequence-sharded), the
 * inverse of ulysses_seq_to_head (guide, layout diagram, lower half). It is
 * also the backward of ulysses_seq_to_head (the transpose of a permutation is
 * its inverse), and ulysses_seq_to_head is the backward of this call.
 *   x_head [sp][B][N][H/sp][d]  ->  x_seq [sp][B][N/sp][H][d]
 * Same argument meaning and errors as ulysses_seq_to_head.
 */
int ulysses_head_to_seq(const void* x_head, void* x_seq, int B, int N, int H, int d, int sp,
                        int dtype, void* stream);

/*
 * The same two layout changes for n tensors of one shape in one launch (q, k
 * and v going into an exchange, dq, dk and dv coming out of it; the guide's
 * layout diagram applies to each): x_seq[i] -> x_head[i] (resp. x_head[i] ->
 * x_seq[i]) for i < n, each exactly as one ulysses_seq_to_head
 * (ulysses_head_to_seq) call. x_seq and x_head are host arrays of n device
 * pointers, read during the call only; 1 <= n <= 4.
 * Errors: ULY_EINVAL also when n is out of range, an array or one of its
 * pointers is null, or an output overlaps any input or another output;
 * ULY_ESHAPE also when n * sp > 65535; otherwise as ulysses_seq_to_head.
 */
int ulysses_seq_to_head_n(const void* const* x_seq, void* const* x_head, int n, int B, int N, int H,
                          int d, int sp, int dtype, void* stream);
int ulysses_head_to_seq_n(const void* const* x_head, void* const* x_seq, int n, int B, int N, int H,
                          int d, int sp, int dtype, void* stream);

/*
 * Attention forward over the head-sharded shares of sp virtual ranks
 * (congresoia365 article, "Cómo Funciona Ulysses", local attention step).
 * For every (rank, batch row, head), with scale = 1/sqrt(d):
 *   S = scale * Q K^T, masked to allowed(i, j) = same document and
 *   (causal == 0 or j <= i); O = softmax_rows(S) V;
 *   lse_i = ln sum_{allowed j} exp(S_ij).
 *   q, k, v, o  [sp][B][N][Hl][d] of dtype; o is fully overwritten.
 *   lse         [sp][B][Hl][N] float (natural log), fully overwritten; it is
 *               the only state the backward needs besides the inputs.
 *   cu_seqlens  device int32 [ndoc+1], cu[0] = 0, non-decreasing,
 *               cu[ndoc] = N: document boundaries shared by every row; or
 *               NULL for one document [0, N) per row (ndoc, max_doc_len
 *               ignored). Empty documents are allowed.
 *   max_doc_len host int >= the longest document (sizes the launch; a
 *               smaller value leaves rows uncomputed).
 * Errors: ULY_EINVAL (null pointer, size <= 0, ndoc < 1 or max_doc_len < 1
 * with cu_seqlens); ULY_ESHAPE when
 *   - max_doc_len > N (with cu_seqlens),
 *   - sp * B * Hl > 2^24 (the (row, head) units of one call),
 *   - N * Hl * d * esize >= 2^31 (one (row, head) sequence spans 2 GiB or
 *     more: buffer offsets are 32-bit), or
 *   - bf16: ceil(L / 256) * ndoc * max(sp * B * Hl, 8) > 2^31 - 1 with L =
 *     max_doc_len (N without cu_seqlens): the launch's tile index;
 * ULY_EUNSUPPORTED (dtype, d); ULY_EHIP.
 */
int ulysses_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int* cu_seqlens, int ndoc, int max_doc_len, int sp, int B, int N,
                     int Hl, int d, int causal, int dtype, void* stream);

/*
 * ulysses_attn_fwd with a persistent launch, for callers that can lend it
 * ulysses_attn_fwd_workspace_bytes() (1152) bytes of device memory: one
 * workgroup per compute unit takes the 256-query tiles from eight queues,
 * one per XCD (an XCD's own heads first, so its L2 keeps serving them, then
 * the other XCDs' remaining tiles), instead of the hardware's fixed
 * round-robin of one workgroup per tile. XCDs that run at a higher clock
 * then take over work of the slower ones, empty tiles of short documents
 * cost no dispatch, and no workgroup waits to be launched. Same arguments,
 * results (bit for bit: every tile is still computed whole by one
 * workgroup) and errors as ulysses_attn_fwd, plus
 *   workspace        device memory, >= ulysses_attn_fwd_workspace_bytes()
 *                    bytes, 4-byte aligned; contents on entry ignored (a
 *                    small kernel on the stream clears the counters first),
 *                    left zeroed. Calls that overlap in time need their own.
 * Errors: as ulysses_attn_fwd; ULY_EWORKSPACE (workspace NULL or too small).
 * The fp32 path ignores the workspace.
 */
size_t ulysses_attn_fwd_workspace_bytes(void);
int ulysses_attn_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, const int* cu_seqlens, int ndoc, int max_doc_len, int sp, int B,
                        int N, int Hl, int d, int causal, int dtype, void* stream);

/*
 * Bytes of device workspace ulysses_attn_bwd needs: two floats per (rank,
 * batch row, head, token) (the row sums D = rowsum(dO * O), stored negated,
 * and lse in log2 units), i.e. O(N), never O(N^2), rounded up to 256 bytes,
 * plus 2304 bytes of tile-queue counters for the bf16 kernels (they run one
 * workgroup per compute unit, each taking tiles until none is left; the
 * pre-pass clears the counters and every kernel leaves them cleared).
 * Returns 0 for invalid arguments.
 */
size_t ulysses_attn_bwd_workspace_bytes(int sp, int B, int N, int Hl, int d, int dtype);

/*
 * Attention backward (the adjoint of ulysses_attn_fwd). With P recomputed
 * tile by tile from lse, D_i = sum_c dO_ic O_ic and the same mask:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q.
 *   q, k, v, o, dout  [sp][B][N][Hl][d] of dtype (o and lse from the forward)
 *   lse               [sp][B][Hl][N] float
 *   dq, dk, dv        [sp][B][N][Hl][d] of dtype, fully overwritten
 *   workspace         device memory of workspace_bytes >=
 *                     ulysses_attn_bwd_workspace_bytes(...); contents on
 *                     entry are ignored, on return unspecified.
 * cu_seqlens, ndoc, max_doc_len, causal as in ulysses_attn_fwd.
 * Errors: as ulysses_attn_fwd, with the bf16 tile condition taken with
 * 128-token tiles, ceil(L / 128) * ndoc * max(sp * B * Hl, 8) > 2^31 - 1;
 * plus ULY_EWORKSPACE.
 */
int ulysses_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, const int* cu_seqlens, int ndoc, int max_doc_len,
                     int sp, int B, int N, int Hl, int d, int causal, int dtype, void* stream);

/*
 * ulysses_attn_bwd in its two steps, for callers that time or schedule them
 * apart; ulysses_attn_bwd is exactly ulysses_attn_bwd_prepare followed by
 * ulysses_attn_bwd_prepared on the same workspace (same kernels, same bits).
 *   ulysses_attn_bwd_prepare: the D pre-pass alone, from o, dout
 *     [sp][B][N][Hl][d] and lse [sp][B][Hl][N]: fills the workspace with the
 *     row sums D_i = sum_c dO_ic O_ic (stored negated for bf16) and, for
 *     bf16, lse in log2 units. One document per row is assumed for sizing
 *     only; the values do not depend on the packing.
 *   ulysses_attn_bwd_prepared: the dK/dV and dQ kernels, reading the
 *     workspace a prepare call of the same sizes and dtype filled (its
 *     contents are not checked; the kernels claim their tiles through the
 *     counters at its end and leave them cleared, so one prepare may serve
 *     several prepared calls in turn); q, k, v, dout, lse, dq, dk, dv,
 *     cu_seqlens, ndoc, max_doc_len, causal as in ulysses_attn_bwd.
 * Errors: as ulysses_attn_bwd.
 */
int ulysses_attn_bwd_prepare(const void* o, const void* dout, const float* lse, void* workspace,
                             size_t workspace_bytes, int sp, int B, int N, int Hl, int d, int dtype, void* stream);
int ulysses_attn_bwd_prepared(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                              void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                              const int* cu_seqlens, int ndoc, int max_doc_len, int sp, int B, int N, int Hl,
                              int d, int causal, int dtype, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * computation, arguments and results as ulysses_attn_bwd, without the
 * workspace: its contents (-D and lse in log2 units, two floats per (rank,
 * batch row, head, token)) go to a scratch array of ULY_NOALLOC_SCRATCH_BYTES
 * that the library holds in device memory, one per GPU, from the first call
 * on that GPU until the process ends. The call allocates nothing.
 *   - The scratch of the calling thread's current device is used: make it the
 *     device of the stream and the tensors.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents (nothing in it needs to start at zero). Calls that
 *     overlap in time on one GPU (on different streams, or from different
 *     host threads) race and give wrong results: serialise them on one
 *     stream, or give each its own workspace through ulysses_attn_bwd.
 *   - Limit: ulysses_attn_bwd_workspace_bytes(...) <= ULY_NOALLOC_SCRATCH_BYTES,
 *     i.e. sp * B * Hl * N <= 8388608 (token, head) rows.
 * Errors: as ulysses_attn_bwd; ULY_EWORKSPACE when the problem needs more
 * scratch than the limit; ULY_EHIP when the scratch's device address cannot
 * be looked up.
 */
#define ULY_NOALLOC_SCRATCH_BYTES (((size_t)64 << 20) + 2304)
int ulysses_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens, int ndoc,
                             int max_doc_len, int sp, int B, int N, int Hl, int d, int causal, int dtype,
                             void* stream);

/*
 * Ring attention, the other sequence-parallel mode (ColossalAI docs,
 * "Sequence Parallelism": sequence_parallelism_mode="ring_attn", related
 * paper "Ring Attention with Blockwise Transformers"; the closing comparison
 * notes it has no head-count condition). sp virtual ranks on one device:
 * rank r keeps token chunk r (Ns = N/sp tokens) of all H heads. At ring step
 * i = 0 .. sp-1 rank r holds key/value chunk j = (r - i) mod sp (passed one
 * rank along the ring per step), attends its queries to that block and
 * merges the block's partial result with its running one by log-sum-exp:
 *   lse' = log(exp(lse) + exp(lse_blk)),
 *   O'   = exp(lse - lse') O + exp(lse_blk - lse') O_blk.
 * Block mask, in global positions: causal -> j < r every key, j == r the
 * causal diagonal, j > r none (the rank idles); causal == 0 -> every key.
 * After sp steps O and lse are softmax attention over the whole sequence.
 * Only ULY_BF16 is supported; d is 64 or 128.
 *
 * Forward step i:
 *   q, k, v  [sp][B][Ns][H][d] bf16, the sequence-sharded layout (k, v of
 *            every chunk; the step picks chunk j for rank r)
 *   o_acc    [sp][B][Ns][H][d] float: running normalised output; read at
 *            step i > 0, written at every step
 *   lse      [sp][B][H][Ns] float: running log-sum-exp (natural log); read
 *            at step i > 0, written at every step
 *   o        [sp][B][Ns][H][d] bf16: rank r's rows are written at its last
 *            step (i == r when causal, i == sp-1 otherwise)
 * Steps run in order 0, 1, .., sp-1 (step 0 ignores o_acc and lse on entry).
 * Errors: ULY_EINVAL (null pointer, size <= 0, step outside [0, sp));
 * ULY_EUNSUPPORTED (dtype, d); ULY_ESHAPE when sp * B * H > 2^24,
 * Ns * H * d * 2 >= 2^31, or ceil(Ns / 128) * max(sp * B * H, 8) > 2^31 - 1
 * (as for ulysses_attn_bwd, with Ns tokens, H heads, one document);
 * ULY_EHIP.
 */
int ulysses_ring_attn_fwd_step(const void* q, const void* k, const void* v, void* o, float* o_acc,
                               float* lse, int step, int sp, int B, int Ns, int H, int d, int causal,
                               int dtype, void* stream);

/*
 * ulysses_ring_attn_fwd_step as a persistent launch, like ulysses_attn_fwd_ws:
 * the caller lends ulysses_attn_fwd_workspace_bytes() (1152) bytes of device
 * memory for the step's tile-queue counters (cleared on the stream before the
 * kernel; contents on entry ignored; steps that share one workspace must not
 * overlap). Same results, bit for bit.
 * Errors: as ulysses_ring_attn_fwd_step; ULY_EWORKSPACE (workspace NULL or
 * too small).
 */
int ulysses_ring_attn_fwd_step_ws(const void* q, const void* k, const void* v, void* o, float* o_acc,
                                  float* lse, void* workspace, size_t workspace_bytes, int step, int sp,
                                  int B, int Ns, int H, int d, int causal, int dtype, void* stream);

/*
 * Bytes of workspace the ring backward needs: two floats per (rank, batch
 * row, head, token) (-D = -rowsum(dO * O) and lse in log2 units), then 2304
 * bytes of tile-queue counters for the steps' persistent kernels (as in
 * ulysses_attn_bwd_workspace_bytes). Returns 0 for invalid arguments.
 */
size_t ulysses_ring_attn_bwd_workspace_bytes(int sp, int B, int Ns, int H, int d, int dtype);

/*
 * Before the backward steps: -D = -rowsum(dO * O) and lse * log2(e) of every
 * query row into the workspace, from the forward's final o and lse; also
 * clears the workspace's queue counters.
 *   o, dout [sp][B][Ns][H][d] bf16; lse [sp][B][H][Ns] float.
 * Errors: as ulysses_ring_attn_fwd_step, plus ULY_EWORKSPACE.
 */
int ulysses_ring_attn_bwd_prepare(const void* o, const void* dout, const float* lse, void* workspace,
                                  size_t workspace_bytes, int sp, int B, int Ns, int H, int d,
                                  int dtype, void* stream);

/*
 * Backward step i (the adjoint of the forward's block of rank r and chunk
 * j = (r - i) mod sp). With P = exp(S - lse) of the block, dP = dO V_j^T and
 * dS = P * (dP - D):
 *   dQ_r += scale dS K_j,  dK_j += scale dS^T Q_r,  dV_j += P^T dO_r.
 *   q, k, v, dout        [sp][B][Ns][H][d] bf16; lse the forward's final one
 *   workspace            as filled by ulysses_ring_attn_bwd_prepare; the
 *                        step's kernels claim tiles from its queue counters
 *                        and leave them cleared for the next step, so steps
 *                        on one workspace must not overlap
 *   dq_acc, dk_acc,      [sp][B][Ns][H][d] float running sums, indexed by the
 *   dv_acc               chunk they belong to (set at step 0, added to later)
 *   dq, dk, dv           [sp][B][Ns][H][d] bf16: a query chunk's dq is written
 *                        at its rank's last step, a key/value chunk's dk, dv at
 *                        its last visit (i == sp-1-j when causal, sp-1 otherwise)
 * Steps run in order 0, 1, .., sp-1 after one prepare call.
 * Errors: as ulysses_ring_attn_bwd_prepare.
 */
int ulysses_ring_attn_bwd_step(const void* q, const void* k, const void* v, const void* dout,
                               const float* lse, void* workspace, size_t workspace_bytes,
                               float* dq_acc, float* dk_acc, float* dv_acc, void* dq, void* dk, void* dv,
                               int step, int sp, int B, int Ns, int H, int d, int causal, int dtype,
                               void* stream);

/*
 * Sequence-parallel loss aggregation (jianying88 guide to DeepSpeed Ulysses
 * in Transformers, section on the work Trainer does by itself, item 3), for
 * sp virtual ranks held on one device. Rank r's loss is the mean of its
 * per-token losses over its counted tokens (label != ignore_index), good_r
 * their number; the batch loss is
 *   loss = sum_r loss_r * good_r / sum_r good_r   over ranks with good_r > 0,
 * the mean over every counted token of the batch. A rank without counted
 * tokens gets loss_r = 0 and drops out; with none anywhere loss = 0. Tokens
 * that do not count contribute nothing, whatever their loss value holds.
 *   token_loss   [sp][B][Ns] float, each rank's per-token losses
 *   labels       [sp][B][Ns] int64, the shifted labels (ignore_index = not counted)
 *   rank_loss    [sp] float out;  good_tokens [sp] int64 out;  loss [1] float out
 *   workspace    >= ulysses_sp_loss_workspace_bytes(sp, B, Ns) bytes, 8-byte
 *                aligned; contents on entry ignored
 * Sums are fp64 in a fixed order (bit-reproducible). sp <= 4096.
 * Errors: ULY_EINVAL (null pointer, size <= 0, B * Ns >= 2^40), ULY_ESHAPE
 * (sp > 4096), ULY_EWORKSPACE, ULY_EHIP.
 */
size_t ulysses_sp_loss_workspace_bytes(int sp, int B, int Ns);
int ulysses_sp_loss(const float* token_loss, const long long* labels, float* rank_loss,
                    long long* good_tokens, float* loss, void* workspace, size_t workspace_bytes,
                    int sp, int B, int Ns, int ignore_index, void* stream);

/*
 * Tiled MLP of ALST (HF guide "Ulysses sequence parallelism", the paragraph
 * after the layout diagram: Arctic Long Sequence Training pairs Ulysses with
 * TiledMLP; jianying88 guide, its account of the layout: after the second
 * all-to-all the FFN runs locally on each rank's token shard). The FFN is the
 * Llama-style SwiGLU MLP of one rank's tokens,
 *   G = X Wg^T,  U = X Wu^T,  A = silu(G) * U,  Y = A Wd^T,  silu(z) = z / (1 + e^-z),
 * computed over tiles of `tile` tokens so that only one tile's [tile, inter]
 * intermediates exist (in the workspace) at a time; the backward recomputes
 * them per tile and accumulates the weight gradients over the tiles:
 *   dA = dY Wd,  dWd = sum dY^T A,  dG = dA * U * silu'(G),  dU = dA * silu(G),
 *   dX = dG Wg + dU Wu,  dWg = sum dG^T X,  dWu = sum dU^T X.
 * The result equals the MLP over all tokens at once (up to rounding).
 *   x, dy, y, dx   [tokens][hidden] bf16 (y, dx fully overwritten)
 *   w_gate, w_up   [inter][hidden] bf16;  w_down [hidden][inter] bf16
 *   dw_gate, dw_up [inter][hidden] float; dw_down [hidden][inter] float:
 *                  fully overwritten with the sums over every token
 *   workspace      >= ulysses_tiled_mlp_workspace_bytes(...) bytes: three
 *                  [tile][inter] bf16 arrays of one tile (A, and the backward's
 *                  U * silu'(G) and silu(G)); contents on entry ignored
 * bf16 only. hidden and inter must be multiples of 256 (Llama-7B: 4096 and
 * 11008); tokens and tile are any positive sizes (the last tile may be short).
 * Pointers (workspace included) must be 16-byte aligned.
 * Errors: ULY_EINVAL (null pointer, size <= 0, a pointer not 16-byte
 * aligned), ULY_ESHAPE (hidden or inter
 * not a multiple of 256, or 512 * max(hidden, inter) >= 2^31),
 * ULY_EWORKSPACE, ULY_EHIP.
 */
size_t ulysses_tiled_mlp_workspace_bytes(int tokens, int hidden, int inter, int tile);
int ulysses_tiled_mlp_fwd(const void* x, const void* w_gate, const void* w_up, const void* w_down, void* y,
                          void* workspace, size_t workspace_bytes, int tokens, int hidden, int inter, int tile,
                          void* stream);
int ulysses_tiled_mlp_bwd(const void* x, const void* w_gate, const void* w_up, const void* w_down, const void* dy,
                          void* dx, float* dw_gate, float* dw_up, float* dw_down, void* workspace,
                          size_t workspace_bytes, int tokens, int hidden, int inter, int tile, void* stream);

/* Static English text for a status code (never NULL). */
const char* ulysses_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ULYSSES_H */
