/*
 * sa.h -- C ABI of libsa: block-sparse causal factorized self-attention
 * (Sparse Transformer strided and fixed patterns) on AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (sources, by page title and section):
 *   - "OpenAI Sparse Transformer" (agentlenshq.com), "Sparse Attention and
 *     Algorithmic Complexity": each output position attends only a subset of
 *     the input positions, so the cost falls from O(N^2) to O(N sqrt N).
 *   - same page, "Factorized Attention Patterns", and "Генеративное
 *     моделирование с разреженными трансформерами" (pcnews.ru),
 *     "Разреженное внимание": the strided pattern (row and column) and the
 *     fixed pattern (a fixed column plus the elements after the latest column
 *     element), each split over two heads.  With i the query position and
 *     j <= i the key position:
 *         SA_STRIDED_A   0 <= i - j < l
 *         SA_STRIDED_B   (i - j) mod l == 0
 *         SA_FIXED_A     floor(j / l) == floor(i / l)
 *         SA_FIXED_B     j mod l >= l - c
 *         SA_DENSE_CAUSAL  every j <= i (the full attention the pages compare
 *                          sparse attention against)
 *   - "OpenAI Sparse Transformer", "Implementation and Limitations", and
 *     pcnews.ru, "Релиз кода": the query and key matrices are sliced into
 *     blocks and only the needed blocks are computed; the block size sets
 *     the granularity of the sparsity ("희소 어텐션 (Sparse Attention)",
 *     molayo1419.me).
 *   - "희소 어텐션 (Sparse Attention)": scores are query-key dot products,
 *     normalised by a softmax so that each row of weights sums to one.
 *   - "[논문 리뷰] Generating Long Sequences with Sparse Transformers"
 *     (nubint.ai), ABSTRACT item (b): the backward pass recomputes the
 *     attention matrix rather than storing it; only O and the row
 *     log-sum-exp are kept from the forward pass.
 *
 * Forward, per (batch b, head h, query row i), with S_i the allowed keys of
 * row i under head h's layout:
 *     s_ij  = scale * (q_i . k_j)
 *     lse_i = log(sum_{j in S_i} exp(s_ij))           (natural log, fp32)
 *     o_i   = sum_{j in S_i} exp(s_ij - lse_i) v_j
 * A row with S_i empty gets o_i = 0 and lse_i = -inf.  Backward returns the
 * gradients of L = sum(dO * O) with respect to q, k and v.
 *
 * Tensors.  q, k, v, o, dout, dq, dk, dv are device pointers to contiguous
 * row-major [B][H][n][d] arrays of the call's dtype (16-byte aligned); lse is
 * a device pointer to fp32 [B][H][n].  All tensor memory is owned by the
 * caller.  Layouts are owned by the library.
 *
 * Execution.  sa_fwd and sa_bwd validate their arguments on the host and
 * return a negative status without launching anything when a check fails.
 * Otherwise they enqueue kernels on `stream` (a hipStream_t; NULL is the
 * default stream) and return SA_OK; device faults surface at the caller's
 * next synchronisation.  The first call with a new (B, H, layouts)
 * combination allocates and uploads a small work list (synchronously), as
 * does the first use of a layout on a device; later calls reuse them and
 * only enqueue kernels, so they may be captured into a HIP graph (make one
 * uncaptured call of each kind first: a call on a stream being captured
 * allocates and copies nothing, and returns SA_ERR_UNSUPPORTED, with nothing
 * enqueued, when its layouts or work list are not on the device yet).  Calls
 * are thread-safe.
 *
 * Compiled (dtype, block, d) combinations:
 *     forward   (SA_F32, 16, 64), (SA_BF16, 64, 64), (SA_BF16, 64, 128)
 *     backward  (SA_BF16, 64, 64), (SA_BF16, 64, 128)
 * Others return SA_ERR_UNSUPPORTED.  bf16 calls accumulate in fp32 and
 * round results to bf16 (nearest even); the softmax weights are rounded to
 * bf16 before they multiply V.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_pattern {
    SA_STRIDED_A = 0,
    SA_STRIDED_B = 1,
    SA_FIXED_A = 2,
    SA_FIXED_B = 3,
    SA_DENSE_CAUSAL = 4
} sa_pattern_t;

typedef enum sa_dtype { SA_F32 = 0, SA_BF16 = 1 } sa_dtype_t;

enum {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = -1, /* a bad value, shape, pointer or alignment */
    SA_ERR_UNSUPPORTED = -2, /* a valid request with no compiled kernel  */
    SA_ERR_HIP = -3,         /* the HIP runtime reported an error        */
    SA_ERR_ALLOC = -4        /* host or device allocation failed         */
};

/* Opaque block layout of one pattern at one sequence length. */
typedef struct sa_layout sa_layout_t;

/*
 * Build the block layout of `pattern` for sequence length n, stride l,
 * summary width c (used by SA_FIXED_B only) and block size `block`.
 * Source: "OpenAI Sparse Transformer", "Implementation and Limitations", and
 * pcnews.ru, "Релиз кода": the query and key matrices are cut into blocks
 * and only the blocks the pattern needs are computed; "희소 어텐션 (Sparse
 * Attention)": the block size is the granularity of the sparsity; the
 * predicates themselves are those of "Factorized Attention Patterns" (file
 * head).  Host only.  For every query block qb (rows qb*block .. qb*block+block-1)
 * it lists, in ascending order, every key block kb holding at least one
 * allowed (i, j), and gives each listed block an element mask: -1 when every
 * element is allowed ("full"), else the index of a T*T-bit mask in a
 * deduplicated table (ids in order of first appearance in the listing).
 * It also builds the transpose (per key block, its query blocks).
 *
 * Errors (SA_ERR_INVALID_ARG): out == NULL; unknown pattern; n < 1;
 * block not in {8, 16, 32, 64, 128}; n % block != 0; l < 1; for SA_FIXED_B
 * c < 1 or c > l; nqb*nqb (the block grid) beyond 2^31.  SA_ERR_ALLOC when
 * memory runs out.  On success *out owns the layout until sa_layout_destroy.
 */
int sa_layout_build(int pattern, int64_t n, int64_t l, int64_t c, int32_t block,
                    sa_layout_t** out);

/*
 * Sizes of a layout: number of query blocks, listed blocks (nnz), distinct
 * partial masks, and allowed (i, j) pairs in total.  Any output pointer may
 * be NULL.  SA_ERR_INVALID_ARG when lay == NULL.
 */
int sa_layout_info(const sa_layout_t* lay, int64_t* nqb, int64_t* nnz, int64_t* n_masks,
                   int64_t* allowed_pairs);

/*
 * Copy a layout into caller-allocated host arrays (any may be NULL):
 *   row_ptr[nqb+1], col_idx[nnz], mask_id[nnz]          listing by query block
 *   mask_words[n_masks * block*block/64]                 mask table; element
 *        (r, s) of a block (query row r, key column s) is bit (r*block+s)%64
 *        of word (r*block+s)/64 of its mask, row-major
 *   col_ptr[nqb+1], row_idx[nnz], csr_pos[nnz]          transpose: for key
 *        block kb, its query blocks ascending and their positions in the
 *        listing by query block
 */
int sa_layout_export(const sa_layout_t* lay, int32_t* row_ptr, int32_t* col_idx,
                     int32_t* mask_id, uint64_t* mask_words, int32_t* col_ptr,
                     int32_t* row_idx, int32_t* csr_pos);

/*
 * Residue view of a strided-B layout ("Генеративное моделирование с
 * разреженными трансформерами", "Разреженное внимание": attention along a
 * column is attention along a row of the transposed matrix).  Under
 * strided B with stride l, position i attends exactly the earlier positions
 * of its residue class i mod l, so a head is l independent dense causal
 * attentions of length n/l over rows r, r+l, r+2l, ...  With the view on,
 * sa_fwd and the sa_bwd calls run this layout's heads that way: each
 * residue class as a dense causal attention (blocks of 64 rows taken l rows
 * apart, a ragged last block padded): at n = 12288, l = 128 that is 384
 * blocks per head against the raster layout's 9312.  The results are those
 * of the raster layout (same pairs; only the rounding order differs).  The layout itself (sa_layout_info, sa_layout_export) is
 * unchanged.  enable = 0 turns the view off.
 *
 * Must not be called while an enqueued sa_fwd/sa_bwd uses the layout.
 * Errors: SA_ERR_INVALID_ARG when lay == NULL; SA_ERR_UNSUPPORTED unless the
 * pattern is SA_STRIDED_B, the block is 64 (the bf16 kernels) and n is a
 * multiple of l; SA_ERR_ALLOC when memory runs out.
 */
int sa_layout_set_residue_view(sa_layout_t* lay, int enable);

/*
 * Compact view of a fixed-B layout ("OpenAI Sparse Transformer", "Factorized
 * Attention Patterns", and pcnews.ru, "Разреженное внимание": fixed B lets a
 * position attend a fixed set of summary columns, the last c of every block
 * of l).  Numbered consecutively, the (n/l)·c summary positions are keys
 * t = 0, 1, ... at sequence position (t / c)·l + (l - c) + t mod c, in
 * increasing order, so the keys a query sees are a prefix of them.  With
 * the view on, sa_fwd and the sa_bwd calls run this layout's heads against
 * 64-key blocks of the summary keys (read in place, no copy): at n = 12288,
 * l = 128, c = 32 that is 4656 blocks per head, almost all full, against the
 * raster layout's 9216 half-empty ones.  Every stage walks the view.  In the
 * view the first key blocks are listed by nearly every query block, so the
 * dK/dV stage walks each pair of key blocks in chunks of at most 96 query
 * blocks, each chunk leaving fp32 partial sums in device memory the library
 * keeps with the call's work list, and a second kernel adds each pair's
 * chunks in a fixed order (deterministic) and writes dK, dV, with zeros on
 * the positions no query reaches.  The results are those of the raster
 * layout (same pairs; only the rounding order differs).  The layout itself (sa_layout_info,
 * sa_layout_export) is unchanged.  enable = 0 turns the view off.
 *
 * Must not be called while an enqueued sa_fwd/sa_bwd uses the layout.
 * Errors: SA_ERR_INVALID_ARG when lay == NULL; SA_ERR_UNSUPPORTED unless the
 * pattern is SA_FIXED_B, the block is 64, n is a multiple of l and c is a
 * power of two; SA_ERR_ALLOC when memory runs out.
 */
int sa_layout_set_compact_view(sa_layout_t* lay, int enable);

/*
 * What the kernels walk for this layout: *kind = 0 (the layout itself),
 * 1 (residue view: a dense causal layout walked once per residue class,
 * l times per head) or 2 (compact view), and that layout's query blocks,
 * key blocks, listed blocks and allowed (query, key) pairs.  Any output
 * pointer may be NULL.  Errors: SA_ERR_INVALID_ARG when lay == NULL.
 */
int sa_layout_view_info(const sa_layout_t* lay, int* kind, int64_t* nqb, int64_t* nkb, int64_t* nnz,
                        int64_t* allowed_pairs);

/* Free a layout, its device copies and the cached work lists of every call
 * that used it.  NULL is ignored.  The caller must make sure no enqueued
 * sa_fwd/sa_bwd still uses it. */
void sa_layout_destroy(sa_layout_t* lay);

/*
 * Forward pass.  Source: "희소 어텐션 (Sparse Attention)": per head, the
 * scores are dot products of the queries with the keys and a softmax turns
 * each row of scores into weights that sum to one, which average the
 * values; "OpenAI Sparse Transformer", "Sparse Attention and Algorithmic
 * Complexity": only the layout's allowed (query, key) pairs enter a row;
 * "[논문 리뷰] Generating Long Sequences with Sparse Transformers", ABSTRACT
 * (b): the row log-sum-exp is kept so that the backward pass can rebuild
 * the weights.  head_layout[h] (h < H) is the layout of head h; several
 * heads may share one layout, at most 8 distinct layouts per call, H <= 256.
 * Every layout must have sequence length n and the call's block size
 * (16 for SA_F32, 64 for SA_BF16).  scale must be finite and > 0.
 * Writes o [B][H][n][d] (dtype) and lse [B][H][n] (fp32).
 * Errors: SA_ERR_INVALID_ARG for NULL/misaligned pointers, B < 1, H < 1,
 * H > 256, a layout whose n differs, a bad scale, more than 8 distinct
 * layouts; SA_ERR_UNSUPPORTED for a (dtype, block, d) not compiled;
 * SA_ERR_HIP if a HIP call or the launch fails; SA_ERR_ALLOC when memory
 * for the work list runs out.  One kernel, or two when long lists are
 * walked in chunks (sa_set_split).  The work list of (head_layout, B, H, d)
 * is built and kept on the device on the first call, with a partial-result
 * buffer per stream that runs it; calls on different streams may overlap.
 * Under graph capture nothing is allocated: the layouts and the work list
 * must be on the device already (else SA_ERR_UNSUPPORTED), and a stream
 * being captured that has no buffer of its own uses one made for another
 * stream by an earlier uncaptured call (SA_ERR_UNSUPPORTED if there is
 * none); the captured work must not overlap that stream's calls.
 */
int sa_fwd(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d,
           int dtype, float scale, const void* q, const void* k, const void* v, void* o,
           float* lse, void* stream);

/* Bytes of device workspace sa_bwd needs: two fp32 row terms per row,
 * -D_i = -sum_t dO_it O_it and -lse_i * log2(e).  Source: "[논문 리뷰]
 * Generating Long Sequences with Sparse Transformers", ABSTRACT (b): the
 * backward pass rebuilds the weights from what the forward pass kept (O and
 * lse) instead of storing them; these two per-row terms are all it derives
 * from O and lse, 8 bytes per row (0 when B, H or n < 1). */
size_t sa_bwd_workspace_size(int32_t B, int32_t H, int64_t n, int32_t d);

/*
 * Backward pass (recomputes the attention weights from q, k and lse).
 * Source: "[논문 리뷰] Generating Long Sequences with Sparse Transformers"
 * (nubint.ai), ABSTRACT (b) and "제안 방법", and pcnews.ru, "Глубокое
 * внимание": the attention matrices are recomputed during backpropagation
 * rather than stored; the gradients are those of the forward's definition
 * over the same allowed pairs.
 * o and lse are sa_fwd's outputs for the same inputs; dout is dL/dO.
 * Writes dq, dk, dv [B][H][n][d] (dtype).  workspace: device memory of at
 * least sa_bwd_workspace_size(...) bytes, 16-byte aligned, owned by the
 * caller, contents ignored on entry.  Same errors as sa_fwd, plus
 * SA_ERR_INVALID_ARG when ws_bytes is too small.  Deterministic: no atomics,
 * so equal inputs give bitwise equal outputs.  Runs sa_bwd_dq_rowterms then
 * sa_bwd_dkdv: two kernels, and a combining kernel after each whose long
 * lists are walked in chunks (sa_set_split) or, for dK/dV, after a compact
 * view's chunks.  Partial results are kept per stream, as for sa_fwd.
 */
int sa_bwd(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d,
           int dtype, float scale, const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
           size_t ws_bytes, void* stream);

/*
 * sa_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * row terms go to a scratch array inside the library (one per device, held
 * until the process ends) instead of a caller workspace; otherwise arguments,
 * results and errors are sa_bwd's, and so are the kernels (bitwise the same
 * gradients).  The call allocates nothing: the layouts and the work lists of
 * (head_layout, B, H) must already be on the current device, which one
 * earlier sa_bwd call with the same head_layout, B and H on that device
 * ensures; else SA_ERR_UNSUPPORTED, launching nothing.  Limit: B*H*n <=
 * 2^21 rows (16 MiB of scratch), else SA_ERR_INVALID_ARG.  Every call on a
 * device shares that device's scratch: calls that overlap on one device (on
 * different streams, or from several threads without ordering) race and
 * give wrong gradients; calls ordered on one stream are safe.  The scratch
 * needs no clearing (the first kernel writes every row term the second
 * reads).  The chunks' partial results (sa_set_split, compact views) use a
 * buffer cached with the work list: the one made for this stream by an
 * earlier sa_bwd, else the one made for another stream, under the same
 * rule.
 */
int sa_bwd_noalloc(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d,
                   int dtype, float scale, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv, void* stream);

/*
 * The stages of the backward pass as separate calls, for callers that
 * schedule them themselves.  Arguments mean what they mean for sa_bwd; each
 * call reads and writes only the pointers it takes.
 *   sa_bwd_dq_rowterms  dQ, and the row terms -D_i = -sum_t dO_it O_it and
 *                       -lse_i log2(e) of every row into the workspace, one
 *                       workgroup per pair of query blocks walking their
 *                       key blocks (sa_bwd's first kernel)
 *   sa_bwd_dkdv         dK, dV (reads the row terms from the workspace), one
 *                       workgroup per pair of key blocks walking their query
 *                       blocks (sa_bwd's second kernel)
 *   sa_bwd_rowterms     the row terms alone into the workspace
 *   sa_bwd_dq           dQ (reads the row terms from the workspace)
 * sa_bwd_dkdv and sa_bwd_dq must be ordered on the device after a call that
 * wrote the row terms (sa_bwd_dq_rowterms or sa_bwd_rowterms).  The two
 * routes give the same dQ, dK, dV up to the summation order of D_i (so not
 * always bitwise); sa_bwd_dq_rowterms + sa_bwd_dkdv is bitwise sa_bwd.
 * Same errors as sa_bwd.
 */
int sa_bwd_dq_rowterms(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d,
                       int dtype, float scale, const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* workspace, size_t ws_bytes,
                       void* stream);
int sa_bwd_rowterms(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d,
                    int dtype, float scale, const void* o, const float* lse, const void* dout,
                    void* workspace, size_t ws_bytes, void* stream);
int sa_bwd_dkdv(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d,
                int dtype, float scale, const void* q, const void* k, const void* v, const void* dout,
                void* dk, void* dv, const void* workspace, size_t ws_bytes, void* stream);
int sa_bwd_dq(const sa_layout_t* const* head_layout, int32_t B, int32_t H, int64_t n, int32_t d,
              int dtype, float scale, const void* q, const void* k, const void* v, const void* dout,
              void* dq, const void* workspace, size_t ws_bytes, void* stream);

/*
 * Forward kernel form, process-wide: a tuning and testing switch (both forms
 * compute the same attention; their results differ only in rounding order).
 *   0  chosen per call (default): the two-half form when most wave-steps of
 *      the call's walk have both 32-key halves of a block live, else the
 *      per-half form
 *   1  the per-half form: each live 32-key half is scored and folded into
 *      the running softmax on its own
 *   2  the two-half form: a step's live halves are scored together and the
 *      running reference is checked once per step
 * Applies to bf16 calls (the fp32 kernel has one form).  Returns the
 * previous setting, or SA_ERR_INVALID_ARG (setting unchanged) for another
 * value.  Calls of sa_fwd that are already enqueued are not affected.
 */
int sa_set_fwd_form(int form);

/*
 * Chunking of long lists, process-wide: a tuning and testing switch.  The
 * bf16 forward, dQ and dK/dV kernels run one workgroup per pair of blocks,
 * longest list first, and the workgroups of a compute unit share its
 * SIMDs, so a unit's time follows the steps it is given.  When one pair's
 * list is longer than whole units' loads (a batch of one and few heads)
 * that list would set the launch's end while other units idle; such a list
 * is walked in chunks by several workgroups, each leaving fp32 partial
 * results in a device buffer the library keeps with the call's work list
 * (one per stream that runs it), and a combining kernel adds each list's
 * chunks in list order and writes the pair's rows: the forward's chunks
 * carry their running reference and row sum, and are rescaled to the
 * largest reference before they are added, as the online softmax does
 * between key blocks ("OpenAI Sparse Transformer", "Implementation and
 * Limitations": the kernels split the work by blocks).  Results are
 * deterministic (fixed order, no atomics) and equal to those of an
 * unchunked walk up to rounding order.  Residue views are never chunked;
 * compact views' dK/dV chunks (96 steps) are not affected.
 *   0   chosen per call (default): lists are cut into chunks of about
 *       the average number of steps per compute unit (at least 16): in a
 *       call with at most 1.25 lists per unit every list longer than that,
 *       else lists longer than twice that average; calls whose every unit
 *       holds many lists' worth of steps get no chunks
 *   -1  no chunks
 *   k>0 every list longer than k steps in ceil(len / k) near-equal chunks
 * *previous (if not NULL) receives the setting before the call.  Returns
 * SA_OK, or SA_ERR_INVALID_ARG (setting unchanged) for a value below -1.
 * Work lists built before the change keep their chunks; later calls use
 * lists built under the new setting.
 */
int sa_set_split(int steps, int* previous);

/*
 * One-exponential paths, process-wide: a testing and comparison switch.
 * Where a 32 x 32 quadrant of a block leaves each lane of the forward's
 * (and dQ's) tile at most one allowed element -- strided B's diagonal
 * blocks, fixed B with one summary column -- those kernels take that
 * element alone: one exponential per lane instead of sixteen, its weight
 * placed back into the tile (the dK/dV kernel, whose lanes are keys, has no
 * such path: there the selection chains cost more than the exponentials
 * they save).  enable = 1 (default) takes them where the quadrants allow,
 * 0 never; both give the same results up to rounding.  *previous (if not
 * NULL) receives the setting before the call.  Returns SA_OK, or
 * SA_ERR_INVALID_ARG (setting unchanged) for another value.  Calls already
 * enqueued are not affected.
 */
int sa_set_one_paths(int enable, int* previous);

/* Static text of a status code. */
const char* sa_status_string(int status);

/* Text of the last error raised on the calling thread ("" if none). */
const char* sa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
