/*
 * attn.h - exact attention forward pass on AMD Instinct MI355X (gfx950).
 *
 * Operation.  For every batch entry b < B and head h < H, with Q, K, V each
 * holding N rows of d features, the library writes
 *
 *     O = softmax(scale * Q K^T [+ causal mask]) V,
 *     LSE_i = m_i + ln(l_i),  m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i),
 *
 * where s_ij = scale * q_i . k_j, and a causal call hides key j from query i
 * whenever j > i.  This is exact attention as defined on the page
 * "FlashAttention: Fast and Memory-Efficient Exact Attention with
 * IO-Awareness" (reading notes at notes.yuuk.io), section "problem setting";
 * the kernel follows that page's section "proposed method": it walks K and
 * V in tiles, keeps a running row max and row sum (tiling), never writes the
 * N x N score or probability matrices to device memory (kernel fusion), and
 * keeps the softmax statistics for a backward pass (recomputation) in the
 * form of LSE.  The result matches the plain definition up to rounding.
 *
 * Conventions shared by every entry point:
 *   - Layout: q, k, v, o are contiguous row-major [B][H][N][d] (d fastest);
 *     lse is contiguous [B][H][N].  All pointers are device pointers.
 *   - Ownership: the caller owns every buffer.  q, k, v are only read;
 *     o and lse are only written, and must not overlap q, k, v or each other.
 *     The library keeps no pointer after the call returns, allocates no
 *     device memory and holds no per-call state: the forward entry points
 *     need no workspace at any size (attn_fwd_split optionally takes the
 *     caller's to run faster), attn_bwd takes the caller's, and only
 *     attn_bwd_noalloc uses memory of the library's own (a static device
 *     array, see there).  Calls are reentrant and may come from several host
 *     threads (attn_bwd_noalloc calls on one device must not overlap).
 *   - Stream: `stream` is a hipStream_t passed as void*; NULL means the
 *     default stream.  The call only enqueues work: it returns before the
 *     kernel runs, and the caller synchronises.
 *   - scale: any finite float; scale < 0 is allowed.  The usual choice is
 *     1/sqrt(d).
 *   - causal: 0 = every query sees all N keys; non-zero = query i sees keys
 *     0..i (the diagonal included, so no row is empty without a key mask).
 *   - Numerics: scores, the online softmax and both products accumulate in
 *     fp32 (the fp32 entry points form scores in fp64).  Non-finite inputs
 *     are not scrubbed: a NaN in the K row of a key a query sees, or in that
 *     query, makes the query's O row and LSE NaN; a NaN in feature f of a
 *     seen key's V row makes feature f of O NaN (an infinite one, +-inf).
 *     A hidden key's score never enters the softmax.  The bf16 paths
 *     multiply whole 32-key blocks of V by their probabilities, a hidden
 *     key's being exactly 0, so a non-finite V value of a hidden key can
 *     still reach the rows that visit its block, as NaN (0 * NaN, 0 * inf);
 *     and when N is not a multiple of 32 the slots past N of the last block
 *     hold copies of key N-1's V row, so a non-finite V value of key N-1
 *     reaches every row that visits that block as NaN (an infinite value
 *     then gives NaN, not +-inf).  The fp32 paths skip hidden keys.
 *   - Errors are reported synchronously, before anything is enqueued; on an
 *     error the outputs are untouched (except ATTN_E_LAUNCH from a later
 *     kernel of attn_bwd, whose earlier kernels are then enqueued and leave
 *     dq, dk, dv undefined).  A fault inside the kernel surfaces at
 *     the caller's next synchronisation (HIP convention).  No C++ exception
 *     crosses this interface.
 */
#ifndef EXACT_ATTENTION_29_AMD_ATTN_H
#define EXACT_ATTENTION_29_AMD_ATTN_H

#include <stddef.h> /* size_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    /* A null pointer; B, H or N below 1; d other than 64; a non-finite
     * scale; N at or above 2^24 (16,777,216); or B*H*ceil(N/32) at or above
     * 2^31.  (The tensors themselves may hold more than 2^31 elements:
     * offsets between heads and batch entries are 64-bit.) */
    ATTN_E_INVALID = 1,
    /* q, k, v or o not 16-byte aligned (the kernels move 128-bit vectors;
     * rows of 64 features keep every row aligned), or lse not 4-byte
     * aligned. */
    ATTN_E_ALIGN = 2,
    /* No HIP device is current, or the current device is not gfx950. */
    ATTN_E_DEVICE = 3,
    /* The kernel launch was rejected by the runtime (its error is also
     * cleared from the runtime's last-error state). */
    ATTN_E_LAUNCH = 4,
    /* attn_bwd_noalloc only: the call needs more workspace than the
     * library's static scratch holds (ATTN_BWD_NOALLOC_SCRATCH_BYTES). */
    ATTN_E_SCRATCH = 5
} attn_status;

/*
 * attn_fwd: bf16 input and output, the main path.
 *   q, k, v : const bf16 [B][H][N][d]   (bf16 = 16-bit bfloat, raw bits)
 *   o       : bf16 [B][H][N][d], rounded to nearest-even from fp32
 *   lse     : float [B][H][N], natural-log log-sum-exp of the scaled,
 *             masked scores of each query row
 *   B, H, N : batch, heads, sequence length (queries = keys = N); N may be
 *             any value >= 1, not only a multiple of the tile size
 *   d       : head size; 64 is the only size built
 * The probabilities multiplying V are rounded to bf16 (nearest-even) before
 * that product; the row sum l adds up the unrounded fp32 probabilities.
 */
attn_status attn_fwd(const void *q, const void *k, const void *v, void *o,
                     float *lse, int B, int H, int N, int d, float scale,
                     int causal, void *stream);

/*
 * attn_fwd_fp32: the same operation with fp32 input and output and no bf16
 * or reduced-precision products: scores, the running row max and their
 * difference are formed in fp64 (products of fp32 values are exact there),
 * exp2 in fp32, the row sum of P and the sums P V in fp64, O rounded to fp32
 * once at the end.  Same layout, ownership, stream and error rules as
 * attn_fwd; q, k, v, o are float.
 */
attn_status attn_fwd_fp32(const float *q, const float *k, const float *v,
                          float *o, float *lse, int B, int H, int N, int d,
                          float scale, int causal, void *stream);

/*
 * attn_fwd_masked: attn_fwd with a key-padding mask.  The Qiita page on the
 * patch-attention layer ("flash-attnの代役がVRAMを18GB溶かしていたので87%削った
 * 話"), sections 4 and 6, describes the mask as a per-key additive bias: 0
 * for a key that takes part, -inf for a padded key, the same for every query
 * of a batch entry.  Two forms, either or both (a key must pass both):
 *   key_len  : const int [B] device array, or NULL.  Key j of batch entry b
 *              takes part only when j < key_len[b] (the usual right
 *              padding).  Values are clamped to [0, N].  4-byte aligned.
 *              This form costs nothing: it only shortens the key loop.
 *   key_bits : const unsigned [B][ceil(N/32)] device array, or NULL: bit
 *              j % 32 of word j / 32 of row b set = key j of entry b takes
 *              part (bits past N are ignored).  4-byte aligned.  Any
 *              pattern is allowed; attn_pack_key_mask builds it from one
 *              byte per key.  Every key tile then takes the masked path.
 * Causal masking, when asked for, applies on top.
 * A query row that sees no key at all (every key padded) gets O = 0 and
 * LSE = -inf: its row sum is the empty sum.  These are the values under
 * which the blockwise combination of the FlashAttention reading notes
 * (section "proposed method") leaves another key set's result unchanged.
 * With both masks NULL this is exactly attn_fwd.  Errors as attn_fwd, plus
 * ATTN_E_ALIGN for a key_len or key_bits not 4-byte aligned.
 */
attn_status attn_fwd_masked(const void *q, const void *k, const void *v,
                            void *o, float *lse, int B, int H, int N, int d,
                            float scale, int causal, const int *key_len,
                            const unsigned *key_bits, void *stream);

/* attn_fwd_masked for fp32 tensors: attn_fwd_fp32 with the same two mask
 * forms and the same empty-row result. */
attn_status attn_fwd_fp32_masked(const float *q, const float *k,
                                 const float *v, float *o, float *lse, int B,
                                 int H, int N, int d, float scale, int causal,
                                 const int *key_len, const unsigned *key_bits,
                                 void *stream);

/*
 * Element strides of one [B][H][N][d] tensor whose d features are
 * contiguous: element (b, h, n, f) sits at b*batch + h*head + n*row + f.
 */
typedef struct attn_layout {
    long long batch;
    long long head;
    long long row;
} attn_layout;

/*
 * attn_fwd_strided: attn_fwd_masked on strided tensors, so that Q, K and V
 * can be read where an input projection left them.  The Qiita page on the
 * patch-attention layer, section 4 (its CPU reproduction of the layer's
 * sdpa path), shows the usual route: one packed projection writes
 * [B][N][3][H][d], it is split into q, k, v, viewed per head and
 * transposed to [B][H][N][d] for the sdpa call, which then needs contiguous
 * copies or strided reads.  With
 * layouts q = {N*3*H*d, d, 3*H*d}, k and v the same (their base pointers d*H
 * and 2*d*H elements further), this call reads the projection output as it
 * is.  o may be strided too (e.g. [B][N][H][d] for the output projection);
 * lse stays contiguous [B][H][N].
 *   *_layout : element strides of q, k, v, o, or NULL for the contiguous
 *              [B][H][N][d] layout.  Every stride must be >= 0 and a
 *              multiple of 8 elements (16 bytes), o's row stride at least
 *              d, and (N-1) * row * 2 + 128 below 2^31 for k and v
 *              (ATTN_E_ALIGN / ATTN_E_INVALID otherwise).  Zero head or
 *              batch strides are allowed for q, k, v (one K/V shared by
 *              several heads); o's rows must not overlap each other (not
 *              checked beyond the row stride).
 *   key_len, key_bits : as attn_fwd_masked (NULL for none).
 * With all layouts NULL this is exactly attn_fwd_masked.
 */
attn_status attn_fwd_strided(const void *q, const void *k, const void *v,
                             void *o, float *lse, int B, int H, int N, int d,
                             float scale, int causal,
                             const attn_layout *q_layout,
                             const attn_layout *k_layout,
                             const attn_layout *v_layout,
                             const attn_layout *o_layout, const int *key_len,
                             const unsigned *key_bits, void *stream);

/*
 * attn_fwd_split: attn_fwd_strided, faster when the query tiles leave the
 * last round of workgroups mostly empty.  A non-causal call runs query
 * tiles of 256 rows, one workgroup per compute unit at a time; when the
 * tiles left after the whole rounds fill at most half of a round (8 MP
 * patches at 16 heads: 2,400 tiles = 9 rounds of 256 CUs and 96 left; 16
 * heads at N = 5,120: 320 tiles = 1 round and 64 left), the workgroups of
 * that round instead share the leftover tiles' keys: each takes an equal,
 * contiguous run of (tile, 64-key tile) pairs -- one or two pieces of
 * query tiles, done one after the other -- and the pieces of one query
 * tile are combined from their row maxima, row sums and unnormalised
 * outputs: the blockwise softmax identity of the FlashAttention reading
 * notes (section "proposed method", tiling), applied across workgroups.
 * The result is the same attention up to rounding (the bf16 product and
 * fp32 sums are split at different keys); it is deterministic (pieces are
 * merged in a fixed order whichever finishes last).  A nearly full last
 * round is left alone: the part is power-limited, and with a few CUs idle
 * the others clock higher, so splitting it gains nothing.
 *   workspace       : device memory owned by the caller, 256-byte aligned
 *                     (ATTN_E_ALIGN otherwise), of at least the bytes
 *                     attn_fwd_split_workspace_size reports for the call:
 *                     0 when the call is not split (then NULL is fine), else
 *                     about 35.7 MB on a 256-CU device, the same for every
 *                     split call (ATTN_E_INVALID when NULL or smaller).  Its
 *                     first 256 * ceil(32 * (CUs/8) / 256) bytes are arrival
 *                     counters that must be zero when a call starts: zero
 *                     the whole workspace once after allocating it; every
 *                     call leaves the counters zero when it completes.  The
 *                     rest holds partial results and needs no clearing.
 *                     Calls that overlap in time (two streams) need separate
 *                     workspaces.
 * Causal calls, calls whose last round is more than half full, calls with
 * no whole round and rows shorter than 10,240 keys (there the 4-wave
 * launch of attn_fwd_strided already spreads the rows over every CU), and
 * rows shorter than 64 * (CUs / 8) keys run exactly as attn_fwd_strided
 * and do not touch the workspace.  Other arguments, layouts, masks and
 * errors as attn_fwd_strided.
 */
attn_status attn_fwd_split(const void *q, const void *k, const void *v,
                           void *o, float *lse, int B, int H, int N, int d,
                           float scale, int causal,
                           const attn_layout *q_layout,
                           const attn_layout *k_layout,
                           const attn_layout *v_layout,
                           const attn_layout *o_layout, const int *key_len,
                           const unsigned *key_bits, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace attn_fwd_split needs for a B x H x N call (causal or
 * not) on the current device, into *bytes: 0 when that call is not split,
 * otherwise a size that depends only on the device's compute-unit count.
 * ATTN_E_INVALID for a NULL bytes or sizes attn_fwd rejects, ATTN_E_DEVICE
 * as attn_fwd.
 */
attn_status attn_fwd_split_workspace_size(int B, int H, int N, int causal,
                                          size_t *bytes);

/*
 * attn_fwd_block_sparse: block-sparse attention, the variant described on
 * the FlashAttention reading notes page, section "block-sparse
 * FlashAttention": a predefined 0/1 matrix M over (query block, key block)
 * pairs; only the blocks where M is 1 are computed, so compute and K/V
 * traffic shrink with the fraction of set blocks.  Key j is hidden from
 * query i when M[i / 128][j / 64] == 0 (query blocks of 128 rows, key
 * blocks of 64 keys; the same M for every batch entry and head).  Causal
 * masking, when asked for, applies on top.
 *   block_mask : const unsigned char [ceil(N/128)][ceil(N/64)] device array,
 *                row-major, non-zero = the block takes part.
 * A query row that sees no key gets O = 0 and LSE = -inf (as
 * attn_fwd_masked).  Same layout, ownership, stream and error rules as
 * attn_fwd; N may be at most 262144 (ATTN_E_INVALID above).
 */
attn_status attn_fwd_block_sparse(const void *q, const void *k, const void *v,
                                  void *o, float *lse, int B, int H, int N,
                                  int d, float scale, int causal,
                                  const unsigned char *block_mask,
                                  void *stream);

/*
 * attn_pack_key_mask: one byte per key -> the bit form attn_fwd_masked
 * reads.  key_valid: const unsigned char [B][N] device array (non-zero =
 * the key takes part); key_bits: unsigned [B][ceil(N/32)] device array,
 * 4-byte aligned, written in full (bits past N are 0).  Enqueued on
 * `stream` like the attention calls; the caller owns both buffers.
 * ATTN_E_INVALID for a null pointer, B or N below 1, N >= 2^24 or
 * B*ceil(N/32) >= 2^31;
 * ATTN_E_ALIGN for a misaligned key_bits; ATTN_E_DEVICE, ATTN_E_LAUNCH as
 * attn_fwd.
 */
attn_status attn_pack_key_mask(const unsigned char *key_valid,
                               unsigned *key_bits, int B, int N,
                               void *stream);

/*
 * attn_bwd: gradients of attn_fwd (bf16, contiguous [B][H][N][d], optional
 * causal mask) by recomputation, as on the FlashAttention reading notes
 * page, section "recomputation": from Q, K, V, the forward output O and its
 * LSE, and the upstream gradient dO = dL/dO, the probabilities are rebuilt
 * tile by tile (never stored) and
 *     dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
 *     dQ = scale * dS K,  dK = scale * dS^T Q.
 *   q, k, v, o, dout : const bf16 [B][H][N][d] (o and lse as attn_fwd wrote
 *                      them for the same q, k, v, scale and causal)
 *   lse              : const float [B][H][N]
 *   dq, dk, dv       : bf16 [B][H][N][d], written in full (rounded to
 *                      nearest-even from fp32 accumulators)
 *   workspace        : scratch owned by the caller, at least
 *                      attn_bwd_workspace_size(B, H, N) bytes, 16-byte
 *                      aligned; overwritten (it holds LSE * log2(e) and -D
 *                      per row, rows padded to a multiple of 256), so calls
 *                      that overlap in time need separate workspaces.
 * Two kernels are enqueued on `stream` (dQ, which also leaves the per-row
 * terms in the workspace, then dK and dV); no atomics, so the result is
 * deterministic.  Errors as attn_fwd
 * (every bf16 pointer and workspace 16-byte aligned, lse 4-byte aligned).
 */
attn_status attn_bwd(const void *q, const void *k, const void *v,
                     const void *o, const float *lse, const void *dout,
                     void *dq, void *dk, void *dv, void *workspace, int B,
                     int H, int N, int d, float scale, int causal,
                     void *stream);

/*
 * attn_bwd_masked: attn_bwd for a forward that hid keys (attn_fwd_masked
 * with the same key_len and key_bits) -- the padded batches the Qiita page's
 * layer passes a key_padding_mask for, in training.  A hidden key takes no
 * part in any query's softmax, so by the same recomputation (FlashAttention
 * reading notes, section "recomputation") its probabilities are 0 in every
 * row:
 *   - dK and dV of a hidden key are exactly 0, and it adds nothing to dQ;
 *   - a query that sees no key has the constant output O = 0 (LSE = -inf):
 *     its dQ is 0 and it adds nothing to any dK or dV.
 *   key_len  : const int [B] device array or NULL, as attn_fwd_masked (keys
 *              j >= key_len[b] hidden; clamped to [0, N]);
 *   key_bits : const unsigned [B][ceil(N/32)] device array or NULL, as
 *              attn_fwd_masked (bit j%32 of word j/32 clear hides key j);
 *              both NULL is exactly attn_bwd.
 * O and LSE must come from the forward with the same masks.  Lengths skip
 * the hidden keys' work; bits compute it and drop it (a select per
 * probability), so a bit mask costs a little more than no mask at any
 * density.  Other arguments,
 * layout, ownership, workspace and errors as attn_bwd (ATTN_E_ALIGN also
 * for a key_len or key_bits not 4-byte aligned).
 */
attn_status attn_bwd_masked(const void *q, const void *k, const void *v,
                            const void *o, const float *lse,
                            const void *dout, void *dq, void *dk, void *dv,
                            void *workspace, int B, int H, int N, int d,
                            float scale, int causal, const int *key_len,
                            const unsigned *key_bits, void *stream);

/*
 * attn_bwd_strided: attn_bwd_masked on strided tensors, the backward of
 * attn_fwd_strided: q, k, v, o, dout may be read where a packed projection
 * (or the forward) left them, and dq, dk, dv written straight into the
 * gradient of a packed projection (the layout the Qiita page's patch
 * layer, section 4, gives its sdpa call: [B][N][3][H][d] split into heads).
 *   *_layout : element strides of q, k, v, o, dout, dq, dk, dv, or NULL for
 *              the contiguous [B][H][N][d] layout.  Every stride must be
 *              >= 0 and a multiple of 8 elements (16 bytes); dq, dk and dv
 *              need a row stride of at least d, and their rows must not
 *              overlap across heads or batch entries (not checked beyond
 *              the row stride); (N-1) * row * 2 + 128 must stay below 2^31
 *              for q, dout, k and v (ATTN_E_ALIGN / ATTN_E_INVALID
 *              otherwise).  Zero head or batch strides are allowed for the
 *              inputs.
 *   key_len, key_bits : as attn_bwd_masked (NULL for none).
 * lse stays contiguous [B][H][N]; the workspace is attn_bwd's.  With every
 * layout NULL this is exactly attn_bwd_masked; otherwise separate kernel
 * instances that form each row's address from its strides run (4-wave
 * workgroups), with the same arithmetic, so the gradients are bitwise those
 * of the contiguous call on the same values.
 */
attn_status attn_bwd_strided(const void *q, const void *k, const void *v,
                             const void *o, const float *lse,
                             const void *dout, void *dq, void *dk, void *dv,
                             void *workspace, int B, int H, int N, int d,
                             float scale, int causal,
                             const attn_layout *q_layout,
                             const attn_layout *k_layout,
                             const attn_layout *v_layout,
                             const attn_layout *o_layout,
                             const attn_layout *dout_layout,
                             const attn_layout *dq_layout,
                             const attn_layout *dk_layout,
                             const attn_layout *dv_layout, const int *key_len,
                             const unsigned *key_bits, void *stream);

/*
 * attn_bwd_block_sparse: attn_bwd for a forward run by
 * attn_fwd_block_sparse with the same block_mask (FlashAttention reading
 * notes, section on block-sparse FlashAttention: the backward skips the
 * same zero blocks).  A (query, key) pair whose block of M is 0 has
 * probability 0, so it passes no gradient between them; a query whose row
 * of M (with the causal mask) leaves no key has dQ = 0.
 *   block_mask : const unsigned char [ceil(N/128)][ceil(N/64)] device array,
 *                as attn_fwd_block_sparse (one M for every batch entry and
 *                head; query block i / 128, key block j / 64).
 * Work follows M: the dQ kernel visits only the key tiles its query block's
 * row sets, the dK/dV kernel (128 keys, two columns of M) the query tiles
 * whose blocks set either of its columns; both pipeline the listed tiles as
 * attn_bwd does, so an all-ones M costs about what attn_bwd does.  A key
 * whose own block of a listed tile is 0 takes probability exactly 0 there
 * (exp2 of -inf), so a NaN in that tile's Q rows still reaches its dK and
 * dV (NaN - inf is NaN).  Other arguments and errors
 * as attn_bwd, plus ATTN_E_INVALID for a NULL block_mask or N > 262144.
 */
attn_status attn_bwd_block_sparse(const void *q, const void *k, const void *v,
                                  const void *o, const float *lse,
                                  const void *dout, void *dq, void *dk,
                                  void *dv, void *workspace, int B, int H,
                                  int N, int d, float scale, int causal,
                                  const unsigned char *block_mask,
                                  void *stream);

/*
 * Bytes of workspace attn_bwd needs: 8 * B * H * ceil(N / 256) * 256 (two
 * fp32 values per padded row of every head); 0 when B, H or N is below 1.
 */
size_t attn_bwd_workspace_size(int B, int H, int N);

/*
 * attn_bwd_noalloc: attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, layout, results and errors as attn_bwd, minus
 * the workspace: the per-row terms go to a static device array of
 * ATTN_BWD_NOALLOC_SCRATCH_BYTES (16 MiB) inside the library, one copy per
 * device, held until the process ends.  The call allocates nothing and needs
 * no set-up; its first call on a device looks up that device's copy.
 *   - Size: attn_bwd_workspace_size(B, H, N) must fit the array, i.e.
 *     B * H * ceil(N / 256) <= 8192 (e.g. 16 heads up to N = 131,072);
 *     larger calls return ATTN_E_SCRATCH and enqueue nothing.
 *   - Every call on a device shares that device's array: calls that overlap
 *     in time on one device (two streams, two host threads) race and give
 *     wrong gradients.  Serialise them, or use attn_bwd with separate
 *     workspaces.  The array keeps the last call's contents; every entry a
 *     call reads is written by the same call first, so nothing needs
 *     clearing.
 */
#define ATTN_BWD_NOALLOC_SCRATCH_BYTES (16u << 20)
attn_status attn_bwd_noalloc(const void *q, const void *k, const void *v,
                             const void *o, const float *lse,
                             const void *dout, void *dq, void *dk, void *dv,
                             int B, int H, int N, int d, float scale,
                             int causal, void *stream);

/* Static, human-readable text for a status code; never NULL. */
const char *attn_strerror(attn_status status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_29_AMD_ATTN_H */
