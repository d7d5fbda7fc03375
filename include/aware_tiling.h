/*
 * aware_tiling.h -- C ABI of the MI355X (gfx950) exact-attention library.
 *
 * The library computes exact single-head attention
 *     O = softmax(scale * Q K^T) V        (row-wise softmax)
 * for a batch of independent heads, as defined on the page "The I/O
 * Complexity of Attention, or How Optimal is Flash Attention?" (exposition),
 * section "Attention as a mathematical problem": the score of query i and key
 * j is scale * <q_i, k_j>, each row of scores is normalised by a row-wise
 * softmax into weights summing to one, and output row i is the average of
 * the value rows under row i's weights.  That page omits
 * the 1/sqrt(d) factor; here it is the explicit `scale` argument.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Layout: Q, K, V, dO, O, dQ, dK, dV are contiguous row-major tensors of
 *    shape [bh, n, d] (bh = batch x heads, n = sequence length, d = head
 *    dimension, d fastest).  lse is [bh, n].  Queries and keys have the same
 *    count n.  Strides are not supported.
 *  - Pointers are DEVICE pointers (hipMalloc'd or from a framework allocator)
 *    on the device that is current for the calling thread.  Q, K, V, dO must
 *    be 16-byte aligned; O, lse, dQ, dK, dV 16-byte aligned as well.
 *  - Ownership: the caller owns every buffer.  No entry point allocates
 *    device memory; scratch space is passed in as `workspace`, sized by the
 *    matching *_workspace_size function.
 *  - dtype: ATTN_BF16 (bfloat16 inputs, fp32 accumulation, bf16 MFMA) or
 *    ATTN_F32 (fp32 inputs and arithmetic; forward only).  Outputs are fp32.
 *  - stream: a hipStream_t passed as void*; NULL means the null stream.
 *    Calls only enqueue work and return without synchronising the host.
 *  - scale must be finite and > 0 (callers pass 1/sqrt(d)).
 *  - Sizes: n <= 2^24, n * d < 2^31, bh <= 2^20 and bh * n <= 2^29 (more
 *    rows than Q, K, V and an fp32 O take in the 288 GB of one GPU at
 *    d >= 64); a larger size is ATTN_ERR_INVALID_ARG.
 *  - Errors: validation happens before any HIP call; on an error nothing is
 *    enqueued and no output is touched.  ATTN_ERR_LAUNCH reports a HIP error
 *    seen right after enqueueing (its text is in attn_last_hip_error()).
 *  - Non-finite inputs propagate to the outputs; they are not detected.  For
 *    the forward entry points a NaN in query row i gives NaN in O row i and
 *    lse i; in key row j, NaN in every row of that head; in V[j][c], NaN in
 *    column c of every row of that head, lse unchanged.  Other rows, columns
 *    and heads are computed as if the NaN were absent.
 */
#ifndef AWARE_TILING_H_
#define AWARE_TILING_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Both enums carry two range sentinels (never returned or accepted) so that
 * every 32-bit integer is a representable value: a caller may pass any int
 * as a dtype and get ATTN_ERR_UNSUPPORTED, and attn_status_string accepts
 * any int. */
typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or scale */
  ATTN_ERR_UNSUPPORTED = 2, /* head dimension or dtype not built */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  ATTN_ERR_LAUNCH = 4,      /* HIP reported an error when enqueueing */
  ATTN_STATUS_RANGE_MIN_ = -2147483647 - 1,
  ATTN_STATUS_RANGE_MAX_ = 2147483647
} attn_status;

typedef enum {
  ATTN_F32 = 0,
  ATTN_BF16 = 1,
  ATTN_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  ATTN_DTYPE_RANGE_MAX_ = 2147483647
} attn_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char* attn_status_string(attn_status s);

/* Text of the last HIP error seen by this thread's calls ("" if none). */
const char* attn_last_hip_error(void);

/* Library version as "major.minor.patch" (static storage). */
const char* attn_version(void);

/*
 * attn_fwd -- fused streaming forward for the large-cache regime.
 *
 * Follows the exposition's sections "Softmax without storing the score
 * matrix" and "Large caches: where FlashAttention's I/O comes from": each
 * workgroup keeps a block of queries and, per query, the running maximum m,
 * the running normaliser l and the unnormalised output u on chip, scans all
 * key/value tiles once, folds each tile in with the rescaling rule
 * (m' = max(m, tile max); l and u multiplied by exp(m - m') before the tile's
 * terms are added), and writes o = u / l.  The N x N score matrix is never
 * stored.
 *
 *   Q, K, V : [bh, n, d] dtype `dtype` (device, read only)
 *   O       : [bh, n, d] float (device, written)
 *   lse     : [bh, n] float, natural-log log-sum-exp of each row of scaled
 *             scores, log(sum_j exp(scale <q_i,k_j>)); may be NULL.
 *   bh >= 0, n >= 0 (bh*n == 0 is a no-op), d in {64, 128, 256} for bf16
 *   and for f32.
 */
attn_status attn_fwd(const void* Q, const void* K, const void* V, float* O,
                     float* lse, int64_t bh, int64_t n, int64_t d, float scale,
                     attn_dtype dtype, void* stream);

/*
 * On-chip elements M held by one workgroup of attn_fwd for head dimension d
 * (query block, its accumulators and statistics, the key/value tiles of
 * every pipeline slot and the score tiles in flight, each element counted
 * once whatever its width), the quantity the exposition calls the
 * fast-memory size M; and the query-block rows B.
 * Returns 0 for unsupported (d, dtype).
 */
int64_t attn_fwd_onchip_elems(int64_t d, attn_dtype dtype);
int64_t attn_fwd_query_block(int64_t d, attn_dtype dtype);

/*
 * attn_fwd_tile -- attn_fwd with the bf16 kernel's tile shape named
 * explicitly, for tile sweeps and tests of every compiled shape.  The
 * fast-memory size M of the exposition's section "Large caches: where
 * FlashAttention's I/O comes from" is set by the query-block rows B and
 * the key tile; this call lets a caller measure the schedule's traffic at
 * each compiled (B, key tile) pair.  attn_fwd itself always uses the first
 * (default) shape for d and reads no environment.
 *
 *   attn_fwd_tiles(d) : space-separated names of the shapes compiled for
 *             head dimension d, the default first; "" if none (static
 *             storage).
 *   attn_fwd_tile_info : query-block rows, keys per tile and on-chip
 *             elements (as attn_fwd_onchip_elems) of shape `tile` at d;
 *             any output pointer may be NULL.  ATTN_ERR_UNSUPPORTED for an
 *             unknown (tile, d), ATTN_ERR_INVALID_ARG for a NULL name.
 *   attn_fwd_tile : same arguments, result and errors as attn_fwd (bf16
 *             only), computed with shape `tile`; ATTN_ERR_UNSUPPORTED for
 *             an unknown (tile, d).
 */
const char* attn_fwd_tiles(int64_t d);
attn_status attn_fwd_tile_info(const char* tile, int64_t d, int64_t* block_rows,
                               int64_t* key_tile, int64_t* onchip_elems);
attn_status attn_fwd_tile(const char* tile, const void* Q, const void* K,
                          const void* V, float* O, float* lse, int64_t bh,
                          int64_t n, int64_t d, float scale, attn_dtype dtype,
                          void* stream);

/*
 * attn_fwd_budget -- the fused streaming forward held to an on-chip budget
 * below d^2, for comparing the two forward schedules at the same M.
 *
 * Follows the exposition's sections "Softmax without storing the score
 * matrix" and "Large caches: where FlashAttention's I/O comes from": the
 * same streaming recurrence as attn_fwd, but each workgroup keeps only a
 * 32-row query block (the smallest the matrix cores take) with 32-key
 * tiles, so its on-chip footprint fits a budget below d^2 at d = 256 and
 * K and V are read once per 32 query rows.  The result is the same
 * function as attn_fwd.
 *
 *   m_elems : on-chip budget M in elements (> 0); the call returns
 *             ATTN_ERR_UNSUPPORTED when attn_fwd_budget_onchip_elems(d)
 *             exceeds it.
 *   Other arguments as attn_fwd; bf16 only, d in {128, 256};
 *   bh * ceil(n / 32) must not exceed 2^31 - 1.
 */
attn_status attn_fwd_budget(const void* Q, const void* K, const void* V,
                            float* O, float* lse, int64_t bh, int64_t n,
                            int64_t d, float scale, attn_dtype dtype,
                            int64_t m_elems, void* stream);
/* On-chip elements of one attn_fwd_budget workgroup at head dimension d
 * (every buffer counted once whatever its width: the Q and U blocks, (m, l),
 * two slots each of the K and V tiles, the four partial score tiles and
 * the summed one); 54,336 at d = 256.  0 for unsupported d. */
int64_t attn_fwd_budget_onchip_elems(int64_t d);

/*
 * attn_fwd_splitk -- fused forward for rectangular shapes, nq queries against
 * nk keys per head (nq much smaller than nk: decoding, chunked prefill).
 *
 * The exposition's closing section notes that single-token decoding (query
 * length one) is outside the square N x N analysis and needs a rectangular
 * account.  This entry point cuts the keys of every head into `splits`
 * contiguous chunks, runs the streaming computation of attn_fwd on each
 * (query block, chunk) pair in its own workgroup, and merges the per-chunk
 * results with the same rescaling rule the streaming recurrence uses within
 * a chunk ("Softmax without storing the score matrix"): with lse_s and o_s
 * the log-sum-exp and normalised output of chunk s,
 *     lse = log sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) o_s.
 * The result is the same function as attn_fwd (bit for bit the same when
 * nq == nk > 32 and one chunk is used: at most 32 queries with d <= 128 run
 * a one-wave form with 32-key tiles, whose rounding order differs).
 *
 *   Q       : [bh, nq, d] bf16;  K, V : [bh, nk, d] bf16 (device, read only)
 *   O       : [bh, nq, d] float; lse : [bh, nq] float or NULL (as attn_fwd)
 *   splits  : requested chunk count, 1..256, or 0 for an automatic choice
 *             (one round of workgroups over the device for more than 128
 *             queries a head, two rounds for fewer, 512 one-wave
 *             workgroups for at most 32 queries with d <= 128; >= 256 keys
 *             a chunk).
 *             Chunks are whole 64-key tiles, so fewer may be used; see
 *             attn_fwd_splitk_splits().
 *   workspace, workspace_bytes : device scratch of at least
 *             attn_fwd_splitk_workspace_size(bh, nq, nk, d, splits) bytes,
 *             256-byte aligned (0 bytes, and NULL allowed, when one chunk
 *             is used).  It holds the per-chunk o_s and lse_s; contents on
 *             return are unspecified.
 *   bh*nq == 0 is a no-op; nk must be >= 1 otherwise (ATTN_ERR_INVALID_ARG).
 *   bf16 only, d in {64, 128, 256}.
 */
int64_t attn_fwd_splitk_splits(int64_t bh, int64_t nq, int64_t nk, int64_t d,
                               int64_t splits);
size_t attn_fwd_splitk_workspace_size(int64_t bh, int64_t nq, int64_t nk,
                                      int64_t d, int64_t splits);
attn_status attn_fwd_splitk(const void* Q, const void* K, const void* V,
                            float* O, float* lse, int64_t bh, int64_t nq,
                            int64_t nk, int64_t d, float scale,
                            attn_dtype dtype, int64_t splits, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * attn_fwd_splitk_noalloc -- attn_fwd_splitk for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * (decoding) loops, harnesses that forbid allocation.  Same arguments,
 * result and errors as attn_fwd_splitk, without the workspace: the
 * per-chunk partial outputs live in a device array inside the library of
 * ATTN_SPLITK_NOALLOC_SCRATCH_BYTES bytes (16 MiB), one per GPU, held from
 * the library's load until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); its first call on
 * a device looks up that device's array address once.
 *
 *   Requests whose partials need more than the array holds, i.e.
 *   attn_fwd_splitk_workspace_size(bh, nq, nk, d, splits) >
 *   ATTN_SPLITK_NOALLOC_SCRATCH_BYTES, return ATTN_ERR_WORKSPACE (pass a
 *   smaller `splits`, or use attn_fwd_splitk).  With one chunk the array
 *   is not used.
 *   Every call on one GPU shares that GPU's array: calls that overlap in
 *   time on one GPU (different streams, or host threads without stream
 *   order between them) race and give undefined results.  Calls ordered on
 *   one stream are safe; the array's contents between calls are
 *   unspecified and nothing in it needs clearing.
 */
#define ATTN_SPLITK_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
attn_status attn_fwd_splitk_noalloc(const void* Q, const void* K, const void* V,
                                    float* O, float* lse, int64_t bh,
                                    int64_t nq, int64_t nk, int64_t d,
                                    float scale, attn_dtype dtype,
                                    int64_t splits, void* stream);

/*
 * attn_fwd_blocksparse -- fused forward restricted to the query/key blocks a
 * block mask keeps (block-sparse attention).
 *
 * The explainer's "Sparse Attention Extension" and its result 2 bound the
 * I/O of sparse attention by the number of kept entries; it gives no
 * algorithm.  Here the kept pairs are square blocks of ATTN_SPARSE_BLOCK
 * queries x ATTN_SPARSE_BLOCK keys: query i and key j interact iff
 * block_mask[hm][i / B][j / B] != 0 (B = ATTN_SPARSE_BLOCK).  Each workgroup
 * runs the streaming computation of attn_fwd over only the key tiles of its
 * kept blocks (the others are neither read nor computed), so
 *     o_i = sum_{j kept} exp(s_ij) v_j / sum_{j kept} exp(s_ij),
 *     lse_i = log sum_{j kept} exp(s_ij);
 * a row with no kept key gets o_i = 0 and lse_i = -inf.
 *
 *   block_mask : device bytes [mask_heads][nb][nb], nb = ceil(n / B),
 *                nonzero = kept; mask_heads is 1 (one mask for all heads,
 *                hm = 0) or bh (hm = head).
 *   workspace, workspace_bytes : at least
 *                attn_fwd_blocksparse_workspace_size(bh, n, mask_heads)
 *                bytes, 256-byte aligned (per-row tile lists built from the
 *                mask on the device).  Contents on return unspecified.
 *   Other arguments as attn_fwd; bf16 only, d in {64, 128, 256}.
 */
#define ATTN_SPARSE_BLOCK 128
size_t attn_fwd_blocksparse_workspace_size(int64_t bh, int64_t n,
                                           int64_t mask_heads);
attn_status attn_fwd_blocksparse(const void* Q, const void* K, const void* V,
                                 float* O, float* lse, int64_t bh, int64_t n,
                                 int64_t d, float scale, attn_dtype dtype,
                                 const uint8_t* block_mask, int64_t mask_heads,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * attn_fwd_smallcache -- square-tile forward for the small-cache regime.
 *
 * Follows the exposition's section "Small caches: when storing an
 * intermediate matrix helps": square tiles of side b (two input tiles and
 * an output tile fit in an on-chip budget of m_elems elements) compute the
 * exponentiated score matrix and write it to device memory (the N x N
 * intermediate, kept in bf16), then a second tiled product multiplies it by
 * V.  The page does not say how the exponentials are kept in range; this
 * library shifts each (row, key tile) by that tile's own maximum, keeps the
 * per-tile sums, merges the per-tile statistics with the same rescaling
 * rule as the streaming recurrence, and applies the merged factors in the
 * second product.  The result is the same function as attn_fwd.
 *
 *   m_elems : on-chip budget M in elements; must satisfy m_elems < d*d
 *             (otherwise the large-cache path applies and the call returns
 *             ATTN_ERR_INVALID_ARG).  The tile side b is the largest
 *             supported side whose footprint fits in m_elems
 *             (ATTN_ERR_UNSUPPORTED if none fits); see
 *             attn_smallcache_tile().
 *   workspace, workspace_bytes : device scratch of at least
 *             attn_fwd_smallcache_workspace_size(bh, n, d, m_elems) bytes,
 *             256-byte aligned.  Its contents on return are unspecified.
 *   Other arguments as attn_fwd; bf16 only, d in {128, 256} (at d = 64 no
 *             tile fits below d^2: ATTN_ERR_UNSUPPORTED).
 */
size_t attn_fwd_smallcache_workspace_size(int64_t bh, int64_t n, int64_t d,
                                          int64_t m_elems);
attn_status attn_fwd_smallcache(const void* Q, const void* K, const void* V,
                                float* O, float* lse, int64_t bh, int64_t n,
                                int64_t d, float scale, attn_dtype dtype,
                                int64_t m_elems, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Tile side b chosen for (d, m_elems), 0 if none fits or m_elems >= d*d;
 * and the on-chip elements one workgroup of that tile actually holds. */
int64_t attn_smallcache_tile(int64_t d, int64_t m_elems);
int64_t attn_smallcache_onchip_elems(int64_t b);

/*
 * attn_bwd -- gradients of attn_fwd.
 *
 * The backward problem is the one the page "On Fine-Grained I/O Complexity
 * of Attention Backward Passes" (explainer) analyses; it prints no formulas.
 * This entry point computes the exact derivatives of O with respect to Q, K
 * and V for an upstream gradient dO, in the blockwise large-cache schedule
 * that page says is optimal when M >= d^2: the weights P are recomputed
 * tile by tile from Q, K and the saved log-sum-exp, never stored, and
 *     dV = P^T dO,  dP = dO V^T,  D_i = <dO_i, o_i>,  dS = P o (dP - D),
 *     dQ = scale dS K,  dK = scale dS^T Q.
 *
 *   Q, K, V, dO : [bh, n, d] bf16 (device, read only)
 *   O           : [bh, n, d] float, the output of attn_fwd on the same Q,K,V
 *   lse         : [bh, n] float, the lse of that attn_fwd call (required)
 *   dQ, dK, dV  : [bh, n, d] float (device, written)
 *   workspace   : at least attn_bwd_workspace_size(bh, n, d) bytes,
 *                 256-byte aligned; contents on return unspecified.
 *   bf16 only, d in {64, 128, 256} (at d = 256 four waves, one per SIMD, of
 *   128 keys or queries per workgroup).
 */
size_t attn_bwd_workspace_size(int64_t bh, int64_t n, int64_t d);

/*
 * attn_bwd_tile -- attn_bwd with the tile shape named explicitly, for tile
 * sweeps and tests of every compiled shape (attn_bwd always takes the
 * default).  A shape is keys per dK/dV workgroup (k), queries per dQ
 * workgroup (q) and keys per dQ tile (c); every shape gives the same bits.
 *
 *   attn_bwd_tiles(d) : space-separated names of the shapes compiled for
 *             head dimension d, the default first; "" if none (static
 *             storage).
 *   attn_bwd_tile_info : keys per dK/dV workgroup, queries per dQ
 *             workgroup, keys per dQ tile and on-chip elements (as
 *             attn_bwd_onchip_elems) of shape `tile` at d; any output
 *             pointer may be NULL.  ATTN_ERR_UNSUPPORTED for an unknown
 *             (tile, d), ATTN_ERR_INVALID_ARG for a NULL name.
 *   attn_bwd_tile : arguments, results and errors as attn_bwd, plus
 *             ATTN_ERR_INVALID_ARG for a NULL name and ATTN_ERR_UNSUPPORTED
 *             for an unknown one.
 */
const char* attn_bwd_tiles(int64_t d);
attn_status attn_bwd_tile_info(const char* tile, int64_t d, int64_t* keys_per_block,
                               int64_t* queries_per_block, int64_t* key_tile,
                               int64_t* onchip_elems);
attn_status attn_bwd_tile(const char* tile, const void* Q, const void* K,
                          const void* V, const float* O, const void* dO,
                          const float* lse, float* dQ, float* dK, float* dV,
                          int64_t bh, int64_t n, int64_t d, float scale,
                          attn_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * On-chip elements M held by one workgroup of attn_bwd for head dimension d:
 * the larger of its two kernels' resident sets (the dK/dV kernel's key rows,
 * accumulators, one query tile and score tiles; the dQ kernel's query rows,
 * accumulator, one key tile and score tiles), each element counted once
 * whatever its width and every pipeline slot counted, as for
 * attn_fwd_onchip_elems: the M of Theorem 1.1 on the page "On Fine-Grained
 * I/O Complexity of Attention Backward Passes".  0 for an unsupported d.
 */
int64_t attn_bwd_onchip_elems(int64_t d);
attn_status attn_bwd(const void* Q, const void* K, const void* V,
                     const float* O, const void* dO, const float* lse,
                     float* dQ, float* dK, float* dV, int64_t bh, int64_t n,
                     int64_t d, float scale, attn_dtype dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * attn_bwd_smallcache -- gradients of attn_fwd for the small-cache regime.
 *
 * The page "On Fine-Grained I/O Complexity of Attention Backward Passes"
 * (explainer), sections "Methodology" and "Key Contributions and Results"
 * (Theorem 1.1): when the on-chip budget M is below d^2 the blockwise
 * schedule of attn_bwd is not optimal, and the page's Algorithm 6 writes the
 * n x n attention matrices and the n x d intermediates to device memory and
 * works on square tiles sized to M, for Theta((n^2 d + n d^2)/sqrt(M))
 * transfers.  The page gives no further steps; this entry point computes the
 * same gradients as attn_bwd (same formulas) in that form: square tiles of
 * side b write P^T and dS^T (bf16, key-major) to the workspace, then three
 * square-tile products give dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K.
 *
 *   m_elems : on-chip budget M in elements, m_elems < d*d (otherwise
 *             ATTN_ERR_INVALID_ARG).  The tile side b in {128, 64} and the
 *             number of staged panels are the largest whose footprint
 *             (accumulators plus staged panels, see
 *             attn_bwd_smallcache_onchip_elems) fits m_elems
 *             (ATTN_ERR_UNSUPPORTED if none fits).
 *   workspace, workspace_bytes : at least
 *             attn_bwd_smallcache_workspace_size(bh, n, d, m_elems) bytes,
 *             256-byte aligned: D, P^T and dS^T, about 4 bh ceil(n/b)^2 b^2
 *             bytes.  Contents on return unspecified.
 *   Other arguments as attn_bwd.  bf16 only, d in {128, 256};
 *   ceil(n/b) b <= 2^20.
 */
int64_t attn_bwd_smallcache_tile(int64_t d, int64_t m_elems);
int64_t attn_bwd_smallcache_onchip_elems(int64_t d, int64_t m_elems);
size_t attn_bwd_smallcache_workspace_size(int64_t bh, int64_t n, int64_t d,
                                          int64_t m_elems);
attn_status attn_bwd_smallcache(const void* Q, const void* K, const void* V,
                                const float* O, const void* dO,
                                const float* lse, float* dQ, float* dK,
                                float* dV, int64_t bh, int64_t n, int64_t d,
                                float scale, attn_dtype dtype, int64_t m_elems,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * attn_calib_mfma_loop -- calibration, not part of the attention method: a
 * matrix-core loop with no memory traffic, timed by the caller for the bf16
 * MFMA rate this device reaches (the published dense peak assumes the top
 * clock; the card lowers its clock with the matrix core's switching load).
 * Each of `workgroups` workgroups of four waves runs `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 chains on register operands drawn
 * in [-amp, amp) (all zero when amp = 0): 4 * 4 * 2 * 32 * 32 * 16 flops
 * per workgroup per round.
 *
 *   out : workgroups * 256 floats (device, written; 16-byte aligned).
 *   ATTN_ERR_INVALID_ARG for a null or unaligned out, workgroups outside
 *   [1, 2^31), iters < 1 or a non-finite amp.  Asynchronous on `stream`.
 */
attn_status attn_calib_mfma_loop(float* out, int64_t workgroups, int32_t iters, float amp,
                                 void* stream);

/*
 * attn_calib_stream_read -- calibration, not part of the attention method: a
 * streaming read of `bytes` bytes of device memory, timed by the caller for
 * the HBM read bandwidth this device reaches (the ceiling of the decoding
 * path, which reads K and V once).  `workgroups` workgroups of 256 threads;
 * thread t reads the 16-byte chunks t, t + T, t + 2T, ... (T = 256
 * workgroups) with non-temporal loads and writes the XOR of their words.
 *
 *   src : bytes bytes (device, read; 16-byte aligned).
 *   out : workgroups * 256 uint32 (device, written; 16-byte aligned).
 *   ATTN_ERR_INVALID_ARG for a null or unaligned pointer, bytes not a
 *   positive multiple of 16, or workgroups outside [1, 2^31 / 256).
 *   Asynchronous on `stream`.
 */
attn_status attn_calib_stream_read(const void* src, int64_t bytes, uint32_t* out,
                                   int64_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AWARE_TILING_H_ */
