/*
 * poem.h - C ABI of libpoem: output-relative (POEM-style) block-sparse causal
 * attention prefill for AMD Instinct MI355X (gfx950).
 *
 * The operation follows the POEM note on attention deletion error (Wu et al.,
 * "POEM: Output-Relative Block-Sparse Attention for Long-Context Prefilling",
 * arXiv:2611.13578): for one query and one head, a visible key block b carries
 * the dense attention mass m_b and the weighted mean value v_b, the dense output
 * is o = sum_b m_b v_b, dropping a set D of mass delta leaves an output error of
 * exactly sum_D m_b (v_b - o) / (1 - delta) (its Section 4.1, Equation (3)), and
 * the triangle inequality bounds its norm by sum_D I_b / (1 - delta) with the
 * block score I_b = m_b ||v_b - o|| (Equation (4)). Head grouping, chunk
 * positions, mandatory sink/local blocks and the tie rule follow "BFLA:
 * Block-Filtered Long-Context Attention Mechanism" (Sections 3.3, 3.6, 5.1 and
 * Appendix A, "Block ordering").
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers are DEVICE pointers unless the name ends in _host. Every call is
 * asynchronous on the given HIP stream (pass a hipStream_t as void*; NULL is the
 * default stream) and never synchronises the host. The library allocates no
 * device memory and keeps no state between calls: the caller owns every buffer,
 * including the selector workspace. Host arrays are read during the call only.
 *
 * Layout is packed "THD", token-major and contiguous in d:
 *   Q [sum N_q][H_q][d], K and V [sum N_k][H_kv][d], sequences concatenated.
 * Query head h reads KV head h / (H_q / H_kv) (BFLA Section 3.3).
 * The N_q queries of a sequence sit at absolute positions N_k - N_q .. N_k - 1
 * (BFLA Section 3.6); (N_k - N_q) must be a multiple of block_size. A query tile is
 * block_size consecutive queries of ONE query head (the last one of a sequence may
 * be shorter); key block b of a sequence holds keys b*B .. b*B+B-1. Tile t of a
 * sequence has diagonal block T_t = (N_k - N_q)/B + t and sees blocks 0 .. T_t.
 * Global tile index = sum over earlier sequences of ceil(N_q/B) + t.
 * CSR row of (h, global tile) = h * num_tiles + global tile.
 *
 * Errors: every argument is validated on the host before anything is enqueued.
 * A failing call returns a negative poem_status, writes nothing, and sets a
 * thread-local message readable with poem_last_error(). A failed launch returns
 * POEM_ERR_HIP. Nothing is thrown across the ABI. Calls are reentrant; calls on
 * different streams may overlap.
 */
#ifndef POEM_H
#define POEM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  POEM_OK = 0,
  POEM_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad enum, inconsistent shape */
  POEM_ERR_UNSUPPORTED = -2, /* valid but outside the built kernels (head_dim, block_size, limits) */
  POEM_ERR_WORKSPACE = -3,   /* workspace missing or smaller than poem_select_workspace_bytes() */
  POEM_ERR_CAPACITY = -4,    /* block_idx capacity smaller than poem_csr_capacity() */
  POEM_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed */
} poem_status;

typedef enum { POEM_BF16 = 0, POEM_FP32 = 1 } poem_dtype;

/* Limits of the built kernels (exceeding one returns POEM_ERR_UNSUPPORTED). */
#define POEM_MAX_SEQS 64          /* sequences per call */
#define POEM_MAX_ROWS_PER_TILE 32 /* sampled rows per tile in the selector */
#define POEM_MAX_VISIBLE_BLOCKS 4096 /* key blocks visible to one tile in the selector */
#define POEM_MAX_HEADS_Q 128       /* query heads in the selector (thresholds travel by value) */

typedef struct {
  int32_t num_seqs;              /* 1 .. POEM_MAX_SEQS */
  const int32_t* seqlens_q_host; /* host [num_seqs]: N_q >= 0 per sequence */
  const int32_t* seqlens_k_host; /* host [num_seqs]: N_k >= N_q, (N_k - N_q) % block_size == 0 */
  int32_t num_heads_q;           /* H_q >= 1, a multiple of num_heads_kv */
  int32_t num_heads_kv;          /* H_kv >= 1 */
  int32_t head_dim;              /* d: 64 or 128 */
  int32_t block_size;            /* B: 64 or 128 (query tile = key block) */
  float softmax_scale;           /* <= 0 selects 1/sqrt(head_dim); must be finite */
  int32_t in_dtype;              /* poem_dtype of Q, K and V */
} poem_problem;

/* Number of query tiles over all sequences (sum of ceil(N_q / B)); < 0 on error. */
int64_t poem_num_tiles(const poem_problem* problem);

/* Sum over (query head, tile) of the tile's visible blocks T_t + 1: the most ids a
 * CSR produced by poem_select can hold. < 0 on error. */
int64_t poem_csr_capacity(const poem_problem* problem);

/* Largest T_t + 1 over all tiles (the row length of the selector's score outputs). */
int64_t poem_max_visible_blocks(const poem_problem* problem);

/* Bytes of device workspace the selectors need (256-byte aligned start): enough for
 * poem_select, poem_select_mass, poem_select_practical and poem_select_group at this
 * rows_per_tile; < 0 on error. It holds per-row softmax statistics, partial
 * statistics when the first pass splits tile groups into block chunks (problems with
 * too few tile groups to fill the GPU otherwise), per-block masses and scores,
 * retained-id slots and, for bf16 inputs, an fp16 copy of V (the size of V) with one
 * scale per (key block, KV head) for the second pass. */
int64_t poem_select_workspace_bytes(const poem_problem* problem, int32_t rows_per_tile);

/*
 * poem_select: the output-relative block selector.
 *
 * For every (query head h, tile t) it samples S_t = min(rows_per_tile, n_t) rows
 * r_j = ceil((j+1) n_t / S_t) - 1 of the tile (n_t = rows in the tile) and, for
 * each sampled row i over the visible keys j <= its position, computes the dense
 * softmax p_ij (scale * q.k, max subtracted), the dense output o_i, and per
 * visible block b the mass m_ib = sum_{j in b} p_ij, the sum u_ib = sum_{j in b}
 * p_ij v_j and the score I_ib = ||u_ib - m_ib o_i|| (= m_ib ||v_ib - o_i||; POEM
 * note Section 4.1 and Equation (4)). The tile score is Ibar_b = mean_i I_ib.
 * Mandatory blocks {b < n_sink_blocks} and {T_t - n_local_blocks < b <= T_t} are
 * always kept (BFLA Sections 4 and 5.1). The other visible blocks are put in
 * discard order: ascending Ibar_b, and among equal scores the larger id first (so
 * the smaller id is retained first; BFLA Appendix A). With A_i(k), Delta_i(k) the
 * sums of I_ib and m_ib over the first k blocks of that order, the bound is
 * B(k) = max_i A_i(k) / (1 - Delta_i(k)) (+inf when 1 - Delta_i(k) <= 0), and the
 * cut k* is the largest k with B(k') <= tau_host[h] for all k' <= k. The first k*
 * blocks are discarded; the rest, with the mandatory blocks, form the tile's CSR
 * row, in ascending id order (BFLA Appendix A).
 *
 *   q, k, v          device, in_dtype, THD layout above.
 *   tau_host         host [H_q]: per-head threshold, finite and >= 0, in the units of V.
 *   n_sink_blocks    >= 0;  n_local_blocks >= 1 (counts the diagonal block).
 *   rows_per_tile    S, 1 .. POEM_MAX_ROWS_PER_TILE.
 *   row_ptr          device int32 [H_q * num_tiles + 1]: CSR offsets (written).
 *   block_idx        device int32 [block_idx_capacity]: CSR ids, local to the sequence (written).
 *   block_idx_capacity  >= poem_csr_capacity(problem).
 *   tile_scores      nullable device fp32 [H_q][num_tiles][max_visible]: Ibar_b; entries
 *                    b > T_t are written as -1.
 *   tile_mass        nullable, same shape: mean_i m_ib (-1 beyond T_t).
 *   row_bound        nullable device fp32 [H_q][num_tiles][rows_per_tile]: the per-row bound
 *                    A_i(k*) / (1 - Delta_i(k*)) at the cut (-1 for rows beyond S_t).
 *   workspace        device, >= poem_select_workspace_bytes(problem, rows_per_tile) bytes,
 *                    256-byte aligned; contents on entry are ignored.
 * Requires every tile to see at most POEM_MAX_VISIBLE_BLOCKS blocks, H_q <= POEM_MAX_HEADS_Q
 * and (H_q / H_kv) * rows_per_tile <= 128.
 */
poem_status poem_select(const poem_problem* problem, const void* q, const void* k, const void* v,
                        const float* tau_host, int32_t n_sink_blocks, int32_t n_local_blocks,
                        int32_t rows_per_tile, int32_t* row_ptr, int32_t* block_idx,
                        int64_t block_idx_capacity, float* tile_scores, float* tile_mass,
                        float* row_bound, void* workspace, size_t workspace_bytes, void* stream);

/*
 * poem_select_practical: practical POEM, the deployed form of the output-relative
 * selector (POEM note Equation (6) and its selection procedure, Appendix B).
 *
 * The same sampled rows and passes as poem_select give per visible block the pooled
 * estimates mbar_b = mean_i m_ib and Ibar_b = mean_i I_ib (Ibar_b / mbar_b is the
 * mass-weighted mean deviation ||v_ib - o_i||). Then:
 *   preselection  the shortest prefix of the candidates in (mbar descending, id
 *                 ascending) order whose mass reaches presel_fraction of the
 *                 candidates' mass; the other candidates are discarded;
 *   rerank        the preselected blocks by log mbar_b + weight * log(Ibar_b / mbar_b)
 *                 (natural logs), descending, smaller id first among equal keys; a
 *                 block with no mass, or (weight != 0) no deviation, ranks last;
 *   threshold     blocks are kept in that order while the pooled retained mass (the
 *                 mandatory blocks' included) is below (1 - eps_host[h]) of the pooled
 *                 total over the visible blocks.
 * The pages leave the estimates, the preselection rule, the weight and the threshold
 * open; these are the parameters. The CSR is as for poem_select.
 *
 * Arguments as for poem_select, except:
 *   eps_host        host [H_q]: pooled omitted-mass budget per head, finite, >= 0.
 *   weight          finite: the deviation weight w.
 *   presel_fraction (0, 1]: the preselected share of the candidates' mass.
 *   tile_scores     nullable: the rerank key of every visible block (-1 beyond T_t).
 *   row_bound       nullable: the per-row omitted mass of the final discard set.
 * Errors as for poem_select; a non-finite weight or a fraction outside (0, 1] is
 * POEM_ERR_INVALID_ARG.
 */
poem_status poem_select_practical(const poem_problem* problem, const void* q, const void* k, const void* v,
                                  const float* eps_host, int32_t n_sink_blocks, int32_t n_local_blocks,
                                  int32_t rows_per_tile, float weight, float presel_fraction, int32_t* row_ptr,
                                  int32_t* block_idx, int64_t block_idx_capacity, float* tile_scores,
                                  float* tile_mass, float* row_bound, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * poem_select_group: the output-relative selector with one list per (KV head, tile),
 * shared by the G = H_q / H_kv query heads that read that KV head (BFLA Section 3.3
 * groups query heads by KV head).
 *
 * The tile's S_t = min(rows_per_tile, n_t) sampled rows sit at the positions
 * poem_select uses, but are spread over the group: row j is taken from query head
 * g G + (j mod G), so each head contributes about S / G rows and the selector does
 * about 1 / G of poem_select's work. Per row: m_ib, u_ib, o_i and I_ib as in
 * poem_select; block score Ibar_b = mean over the S_t rows; discard order as in
 * poem_select. A prefix of the discard order is acceptable iff every sampled row's
 * bound A_i / (1 - Delta_i) is <= tau_host of that row's head; the cut is the longest
 * prefix all of whose sub-prefixes are acceptable. Each sampled row thus keeps its own
 * head's guarantee. The CSR holds the shared list under every head of the group
 * (rows h * num_tiles + tile), so poem_sparse_prefill consumes it unchanged.
 *
 * Arguments as for poem_select, except:
 *   rows_per_tile  S per (KV head, tile), 1 .. POEM_MAX_ROWS_PER_TILE (no limit on G S).
 *   tile_scores, tile_mass  nullable: the group's Ibar_b and mbar_b, repeated under each
 *                  head of the group.
 *   row_bound      nullable: the group's per-row bounds at the cut, row j of the group
 *                  sample at index j, repeated under each head of the group.
 * The workspace size is poem_select_workspace_bytes(). Errors as for poem_select.
 */
poem_status poem_select_group(const poem_problem* problem, const void* q, const void* k, const void* v,
                              const float* tau_host, int32_t n_sink_blocks, int32_t n_local_blocks,
                              int32_t rows_per_tile, int32_t* row_ptr, int32_t* block_idx,
                              int64_t block_idx_capacity, float* tile_scores, float* tile_mass,
                              float* row_bound, void* workspace, size_t workspace_bytes, void* stream);

/*
 * poem_select_mass: the mass-only selector, the baseline the POEM note compares the
 * output-relative score against (its evaluation summary: mass-only baseline at 128K).
 *
 * Same sampled rows, per-row block masses m_ib, mandatory set, tie rule and CSR
 * output as poem_select. The ranking key is the tile mass mbar_b = mean_i m_ib
 * (discard order: ascending mbar_b, larger id first among equal masses). With
 * Delta_i(k) the mass of row i over the first k blocks of that order, the cut k*
 * is the largest k with max_i Delta_i(k') <= eps_host[h] for all k' <= k: every
 * sampled row keeps all but at most eps of its dense attention mass, which bounds
 * its output error by 2 R eps for values of norm <= R (BFLA Appendix B.1). The
 * pages fix no mass threshold; eps is a parameter.
 *
 * Arguments as for poem_select, except:
 *   eps_host     host [H_q]: per-head omitted-mass budget, finite and >= 0.
 *   tile_scores  nullable: receives the ranking key mbar_b (-1 beyond T_t).
 *   row_bound    nullable: the per-row omitted mass Delta_i(k*) at the cut.
 * Neither pass computes P V (no o, u or I), and both stream K only. The workspace
 * size is poem_select_workspace_bytes(). Errors as for poem_select.
 */
poem_status poem_select_mass(const poem_problem* problem, const void* q, const void* k, const void* v,
                             const float* eps_host, int32_t n_sink_blocks, int32_t n_local_blocks,
                             int32_t rows_per_tile, int32_t* row_ptr, int32_t* block_idx,
                             int64_t block_idx_capacity, float* tile_scores, float* tile_mass,
                             float* row_bound, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the optional device workspace poem_sparse_prefill uses to schedule its rows
 * (a queue head and one int32 per CSR row); < 0 on error. */
int64_t poem_sparse_workspace_bytes(const poem_problem* problem);

/*
 * poem_sparse_prefill: causal softmax attention of each query tile over the key
 * blocks its CSR row lists, i.e. the masked softmax over {j <= position : block(j)
 * listed} with scores scale * q.k. This is the retained-block attention the POEM
 * note's sparse output o_tilde denotes (Section 4.1); the loop skips unlisted
 * blocks, as BFLA's support-restricted kernel does (Section 3.4).
 *
 *   row_ptr, block_idx  device int32 CSR as produced by poem_select (rows as above). Each
 *                    row must be strictly ascending; ids > T_t are skipped; a row with
 *                    no usable id yields O = 0 and LSE = -inf.
 *   out              device [sum N_q][H_q][d] in out_dtype (POEM_BF16 or POEM_FP32).
 *   lse              nullable device fp32 [H_q][sum N_q]: natural-log sum of exp of the scores.
 *   workspace        nullable device buffer of >= poem_sparse_workspace_bytes(problem) bytes,
 *                    256-byte aligned, contents ignored on entry. With it, a schedule kernel
 *                    orders the rows by retained count (longest first) and a persistent
 *                    kernel pulls them from a queue; without it, one workgroup per row is
 *                    launched in diagonal order. Results are identical either way. Calls that
 *                    share a workspace must not overlap.
 */
poem_status poem_sparse_prefill(const poem_problem* problem, const void* q, const void* k,
                                const void* v, const int32_t* row_ptr, const int32_t* block_idx,
                                void* out, int32_t out_dtype, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * poem_sparse_prefill_group: poem_sparse_prefill for lists shared by the query heads of
 * each GQA group, as poem_select_group writes them (BFLA Section 3.3 groups heads by
 * KV head; Section 3.4 restricts the kernel to the listed blocks). Every head of a
 * group walks the list of the group's first head, row (g G) * num_tiles + tile (the
 * schedule orders rows by that list's length); the other heads' rows are not read. With
 * bf16 inputs, an even group size and a workspace, one workgroup runs two heads of a
 * group over one tile, loading each K/V stage once for both. The result equals
 * poem_sparse_prefill on a CSR that repeats each first head's row under every head of
 * its group, bit for bit. Arguments, workspace and errors as for poem_sparse_prefill.
 */
poem_status poem_sparse_prefill_group(const poem_problem* problem, const void* q, const void* k,
                                      const void* v, const int32_t* row_ptr, const int32_t* block_idx,
                                      void* out, int32_t out_dtype, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Most CSR rows (num_heads_q * num_tiles) poem_sparse_prefill_noalloc schedules. */
#define POEM_NOALLOC_MAX_ROWS 1048576

/*
 * poem_sparse_prefill_noalloc: poem_sparse_prefill with its persistent, count-ordered
 * schedule, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). It takes no
 * workspace: the queue head and the row order live in a library-owned device array
 * of 256 + 4 * POEM_NOALLOC_MAX_ROWS bytes (about 4 MiB), one per GPU, held from the
 * first call on that GPU until the process ends. The call allocates nothing; its
 * first call on a device looks up that device's copy of the array.
 *
 * Arguments, results and errors as for poem_sparse_prefill (the results are identical),
 * except: num_heads_q * num_tiles above POEM_NOALLOC_MAX_ROWS is POEM_ERR_UNSUPPORTED,
 * and the stream must belong to the current device. Every call on one GPU shares that
 * GPU's array and it keeps the last call's contents (the schedule kernel resets the
 * queue head on the stream before use), so calls that overlap on one GPU, on any
 * streams, race: the caller must order them.
 */
poem_status poem_sparse_prefill_noalloc(const poem_problem* problem, const void* q, const void* k,
                                        const void* v, const int32_t* row_ptr, const int32_t* block_idx,
                                        void* out, int32_t out_dtype, float* lse, void* stream);

/* Bytes of the optional device workspace poem_dense_prefill uses for its tile queue. */
#define POEM_DENSE_WORKSPACE_BYTES 256

/*
 * poem_dense_prefill: the same kernel with every tile's full causal list 0 .. T_t:
 * dense causal attention, the output o the POEM note's deletion error is measured
 * against (Section 4.1), and the speedup baseline. out, lse and errors as for
 * poem_sparse_prefill.
 *
 *   workspace        nullable device buffer of >= POEM_DENSE_WORKSPACE_BYTES bytes,
 *                    256-byte aligned, contents ignored on entry. With it, a persistent
 *                    kernel pulls tiles from a queue (reset by a one-thread kernel on the
 *                    stream), one KV head after another and longest first within each;
 *                    without it, the resident workgroups take the tiles of that order in
 *                    a fixed interleave. Results are identical either way. Calls that
 *                    share a workspace must not overlap.
 */
poem_status poem_dense_prefill(const poem_problem* problem, const void* q, const void* k,
                               const void* v, void* out, int32_t out_dtype, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Message of the last failing call on this thread ("" if none); valid until the next call. */
const char* poem_last_error(void);

/* Library version string. */
const char* poem_version(void);

#ifdef __cplusplus
}
#endif

#endif /* POEM_H */
