/*
 * msa_decode.h - C ABI of libmsadecode: block-sparse (MSA-style) attention decode
 * over a paged FP8 / NVFP4 KV cache on AMD Instinct MI355X (gfx950).
 *
 * One decode step is five calls, in this order, all asynchronous on one HIP stream:
 *
 *   msa_kv_append      quantise the step's new K, V and index-K into their page slots
 *   msa_index_score    score every visible token's index key, max-pool per 128-token block
 *   msa_select_topk    pick k blocks per query row (ties to the smaller block)
 *   msa_sparse_decode  GQA flash-decode over the selected pages, split-KV partials
 *   msa_combine        fixed-order log-sum-exp merge of the partials into bf16 outputs
 *
 * Fused entry points run the same step in two launches: msa_append_score_select
 * (append + score, optionally + select) and msa_select_decode_combine (select + decode
 * + combine) or msa_sparse_decode_combine (decode + combine); msa_decode_step runs the
 * whole step in one launch where its shape allows. msa_sparse_decode_union decodes the
 * rows of a request together over the union of their selected pages.
 *
 * The operations follow three public TensorRT-LLM pull-request pages:
 *   [Rubin] "[None][feat] Add Rubin (sm_107) MiniMax-M3.1 low-latency decode targets" (#21136)
 *   [GB300] "MiniMax-M3 NVFP4 low-latency decode megakernel for modeling_v2 for Blackwell" (#20306)
 *   [P128]  "[None][perf] MiniMax-M3: native P128 draft KV view for the NVFP4 hybrid cache" (#19731)
 *
 * General rules for every entry point:
 *   - Every array argument is caller-owned DEVICE memory, except the msa_kv_pool_t and
 *     msa_step_t structs themselves, which live in HOST memory and are read during the
 *     call only (the device pointers inside them are what the kernels use).
 *   - Nothing is allocated or freed and no host synchronisation happens; calls on
 *     different streams may run concurrently if their outputs differ. The release library
 *     keeps no global state beyond the fixed per-GPU array of the allocation-free entry
 *     (msa_sparse_decode_combine_noalloc) and its address on each device; the debug
 *     library's two process-wide settings are described at msa_debug_set_error_word.
 *   - Geometry is validated on the host before any launch. A call outside the supported
 *     contract returns MSA_ERR_UNSUPPORTED and launches nothing; it never falls back to
 *     another algorithm ([GB300] "The TP4 decode target": a covered shape whose
 *     precondition is missing raises instead of falling back silently).
 *   - Device-side metadata (page ids, positions, selections) is trusted: page ids must
 *     be in [0, num_pages) and positions must be covered by the block table.
 *   - All byte offsets are computed in 64 bits ([Rubin] "Disclosures and known gaps":
 *     int32 KV offsets overflow at 1M-token contexts).
 *   - `stream` is a hipStream_t (0 = the null stream).
 */
#ifndef MSA_DECODE_H_
#define MSA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1,  /* null pointer, misaligned pointer, negative size      */
  MSA_ERR_UNSUPPORTED = -2,  /* geometry or format outside the contract              */
  MSA_ERR_LAUNCH = -3,       /* the HIP runtime rejected a kernel launch             */
  MSA_ERR_TOO_LARGE = -4     /* more than an allocation-free entry's fixed scratch   */
} msa_status_t;

typedef enum {
  MSA_KV_FP8_E4M3 = 1, /* OCP E4M3FN codes, one fp32 scale per page for K and for V     */
  MSA_KV_NVFP4 = 2     /* E2M1 codes + E4M3 scale per 16 elements + fp32 tensor scale   */
} msa_kv_format_t;

typedef enum {
  MSA_INDEX_E4M3 = 1,  /* one unscaled OCP E4M3 code per index-key element (0 means the same) */
  MSA_INDEX_NVFP4 = 2  /* E2M1 codes + E4M3 scale per 16 elements + fp32 index tensor scale  */
} msa_index_format_t;

#define MSA_PAGE_SIZE 128     /* tokens per page ([P128] Description: native P128 pages) */
#define MSA_HEAD_DIM 128
#define MSA_INDEX_DIM 64
#define MSA_HEADS_PER_KV 16   /* [Rubin] Description: 16 query heads per KV head          */
#define MSA_MAX_TOPK 64
#define MSA_MAX_BLOCKS 12288  /* blocks per sequence (1.5M tokens)                        */
#define MSA_MAX_SEL_TABLES 4  /* per-KV-head selection: at most 4 tables per row          */
#define MSA_MAX_GROUP_ROWS 4  /* msa_sparse_decode_union: rows per group (verify length)   */
/* Bit pattern of every fp32 word of an idle split-merge workspace (a signalling NaN). */
#define MSA_MERGE_IDLE_BITS 0x7fbadbadu

/*
 * One layer's paged KV pool. A page holds 128 consecutive tokens of one sequence;
 * inside a page the layout is head-major (HND). Token t of a page, KV head h:
 *
 *   NVFP4  k_codes/v_codes  u8 [num_pages][num_kv_heads][128][head_dim/2]
 *                           byte j holds element 2j in its low nibble, 2j+1 in its high nibble
 *          k_scales/v_scales u8 (E4M3) [num_pages][num_kv_heads][128][head_dim/16]
 *                           scale g covers elements 16g..16g+15 of that token and head
 *          value = E2M1(code) * E4M3(scale) * tensor_scale
 *   FP8    k_codes/v_codes  u8 (E4M3) [num_pages][num_kv_heads][128][head_dim]
 *          k_scales/v_scales fp32 [num_pages]  (one scale per page, all heads)
 *          value = E4M3(code) * page_scale
 *   index_k, MSA_INDEX_E4M3 (default): u8 [num_pages][128][index_dim], one unscaled
 *          E4M3 key per token
 *   index_k, MSA_INDEX_NVFP4: per page, token p = 16 t + n (t < 8, n < 16) and key
 *          group g (elements 16g .. 16g+15, g < index_dim/16), group-major:
 *          index_k u8 [num_pages][g][n][t][8] (low nibble = even element),
 *          index_scales u8 (E4M3) [num_pages][g][n][t]; value =
 *          E2M1(code) * E4M3(scale) * index_tensor_scale. One group of a page's 8 token
 *          rows {n, n+16, ..., n+112} is thus 64 contiguous code bytes. [Rubin] Description lists
 *          NVFP4 index-K pages (indexer_kv_dtype='nvfp4', a prototype) without a
 *          recipe; the key is encoded like the NVFP4 KV (see msa_kv_append).
 *
 * All arrays in use are required and must be 16-byte aligned.
 */
typedef struct {
  int32_t fmt;            /* msa_kv_format_t                                   */
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;       /* must be 128                                       */
  int32_t page_size;      /* must be 128                                       */
  int32_t index_dim;      /* must be 64                                        */
  void* k_codes;
  void* v_codes;
  void* k_scales;
  void* v_scales;
  float k_tensor_scale;   /* NVFP4 only; > 0                                   */
  float v_tensor_scale;   /* NVFP4 only; > 0                                   */
  void* index_k;
  int32_t index_fmt;        /* msa_index_format_t; 0 = MSA_INDEX_E4M3             */
  void* index_scales;       /* MSA_INDEX_NVFP4 only                               */
  float index_tensor_scale; /* MSA_INDEX_NVFP4 only; > 0                          */
} msa_kv_pool_t;

/*
 * Per-step metadata (device arrays). Query rows are request-major: the rows of one
 * request are contiguous. Row r belongs to request row_seq[r] and sits at absolute
 * position row_pos[r]; it attends positions [0, row_pos[r]] (causal among the verify
 * tokens of a speculative step). Its visible blocks are 0 .. row_pos[r] / 128.
 * When num_rows > 0, num_seqs must be at least 1 and every row_seq value must lie in
 * [0, num_seqs) (MSA_ERR_INVALID_ARG for num_seqs == 0; the values are trusted).
 *
 * sel_tables: selection tables per query row ([Rubin] commit messages: the indexer
 * hands KV-head-reduced scores to its selector; the prefill tile select runs per KV
 * head and writes a head-major table). 0 or 1: one table per row, shared by every KV
 * head. T > 1: one table per (row, KV head); T must equal the pool's num_kv_heads, and
 * every per-row array of the selection gains a table axis after the row:
 *   block_scores [num_rows][T][max_blocks_per_seq], sel and sel_pages [num_rows][T][k].
 * Table t is scored from index heads [t * n_idx_heads / T, (t + 1) * n_idx_heads / T)
 * (n_idx_heads must be a multiple of T), selected by the same rule, and read by KV
 * head t. At most MSA_MAX_SEL_TABLES; negative is MSA_ERR_INVALID_ARG.
 *
 * rows_per_seq: 0 = not stated. R > 0 states that every request has exactly R rows
 * (num_rows == num_seqs * R, else MSA_ERR_INVALID_ARG; negative is
 * MSA_ERR_INVALID_ARG), as in a speculative step with a fixed draft length. The index
 * scorer then launches one workgroup row per group of a request's rows instead of one
 * per row (the rows of a group share their key reads). Results are the same either
 * way. Like row_seq itself the statement is trusted; the debug library reports a wrong
 * one as MSA_DEBUG_BAD_SEQ.
 */
typedef struct {
  int32_t num_seqs;
  int32_t num_rows;
  int32_t max_blocks_per_seq;
  const int32_t* block_table; /* [num_seqs][max_blocks_per_seq] logical block -> page id */
  const int32_t* row_seq;     /* [num_rows]                                              */
  const int32_t* row_pos;     /* [num_rows]                                              */
  int32_t sel_tables;         /* 0/1: shared selection; num_kv_heads: one per KV head    */
  int32_t rows_per_seq;       /* 0: not stated; R > 0: every request has exactly R rows  */
} msa_step_t;

/*
 * KV append ([GB300] "Step-loop runtime hooks": a hook for the KV update; [Rubin]
 * Description: saturating FP8 casts). Token i is written to page slot[i] / 128, offset
 * slot[i] % 128; slot[i] < 0 skips the token and writes nothing.
 *   k_new, v_new : bf16 [n_new][num_kv_heads][head_dim]   (either may be NULL to skip)
 *   idx_k_new    : bf16 [n_new][index_dim]                (may be NULL to skip)
 * Encoding, all in correctly rounded fp32, rounding to nearest-even, saturating:
 *   NVFP4 per 16 elements: amax = max|x|; sc = E4M3(amax / (6 * t)); if E4M3(sc) == 0
 *         every code is +0, else d = E4M3(sc) * t and code_i = E2M1(x_i / d)
 *   FP8   code = E4M3(x / page_scale[page])   (the page scale is read, never written)
 *   index code = E4M3(x), or with MSA_INDEX_NVFP4 the NVFP4 rule above per 16 elements
 *         of the key with t = index_tensor_scale
 * Two tokens with the same slot in one call race. n_new may be 0.
 */
msa_status_t msa_kv_append(const msa_kv_pool_t* pool, int32_t n_new, const int64_t* slot,
                           const void* k_new, const void* v_new, const void* idx_k_new,
                           void* stream);

/*
 * Index score with block max-pool. For row r and visible token p (p <= row_pos[r]):
 *   s_p = sum_h w[r][h] * max(0, q_idx[r][h] . key(p))
 * where key(p) is the exact value of token p's index key (E4M3, or NVFP4 decoded as
 * E2M1 * E4M3 scale * index_tensor_scale).
 *   block_scores[r][b] = max over the visible tokens p of block b of s_p   (b < nb(r))
 *   block_scores[r][b] = -inf                                   (nb(r) <= b < max_blocks)
 * The pages name the scorer ([GB300] "The TP4 decode target": an index scorer over
 * index-K pages) but not its formula; this is the definition the library adopts.
 *   q_idx  : bf16 [num_rows][n_idx_heads][index_dim]
 *   w      : fp32 [num_rows][n_idx_heads]
 *   block_scores : fp32 [num_rows][max_blocks_per_seq] (output), or
 *                  [num_rows][T][max_blocks_per_seq] with T = step->sel_tables > 1, where
 *                  table t sums only the index heads of its share (see msa_step_t)
 * n_idx_heads must be 1, 2 or 4. Accumulation is fp32 in a fixed order that does not
 * depend on the token's position, so identical keys give bit-identical scores.
 */
msa_status_t msa_index_score(const msa_kv_pool_t* pool, const msa_step_t* step,
                             int32_t n_idx_heads, const void* q_idx, const float* w,
                             float* block_scores, void* stream);

/*
 * Top-k block selection ([Rubin] commit messages: the table is "ascending, -1-padded"
 * with "init / local forcing"; [GB300] "The TP4 decode target", numerics: ties go to
 * the smaller block). For row r with nb = row_pos[r] / 128 + 1 visible blocks:
 *   nb <= k : sel[r] = 0, 1, ..., nb-1, then -1 padding (identity table, [GB300]
 *             "Step-loop runtime hooks")
 *   nb >  k : blocks 0..n_init-1 and nb-n_local..nb-1 are forced and count inside k;
 *             the remaining k - |forced| slots take the best other blocks ordered by
 *             (higher score, then smaller block index). Output ascending.
 *   block_scores : fp32 [num_rows][max_blocks_per_seq]; only b < nb(r) is read
 *   sel          : int32 [num_rows][k] (output, logical block ids)
 *   sel_pages    : int32 [num_rows][k] (output, may be NULL) the physical page of each
 *                  selected block, block_table[row_seq[r]][sel[r][i]], -1 where sel is -1
 * With step->sel_tables = T > 1 every (row, table) is selected on its own from
 * block_scores [num_rows][T][max_blocks_per_seq] into sel / sel_pages [num_rows][T][k].
 * 1 <= k <= 64, n_init >= 0, n_local >= 0, n_init + n_local <= k,
 * max_blocks_per_seq <= 12288. The result is deterministic for any tie width.
 */
msa_status_t msa_select_topk(const msa_step_t* step, const float* block_scores, int32_t k,
                             int32_t n_init, int32_t n_local, int32_t* sel, int32_t* sel_pages,
                             void* stream);

/*
 * msa_kv_append + msa_index_score + msa_select_topk in one launch, with the same
 * results and outputs as the three calls in that order ([GB300] "The TP4 decode
 * target": block selection and the KV update fused into the decode megakernels; "The
 * TP8 decode target": index scoring fused with block selection). Arguments are those
 * of the three calls; additionally:
 *   counters : int32 [num_rows], all zero before the call; left zero again. Two calls
 *              that share `counters` must not run concurrently.
 * n_new <= 4096 (larger appends: call msa_kv_append first, then this with n_new = 0).
 * block_scores is written as by msa_index_score and is the selection's workspace.
 * With sel == NULL and counters == NULL the call only appends and scores (the
 * selection then runs inside msa_select_decode_combine); sel_pages is ignored.
 */
msa_status_t msa_append_score_select(const msa_kv_pool_t* pool, const msa_step_t* step,
                                     int32_t n_new, const int64_t* slot, const void* k_new,
                                     const void* v_new, const void* idx_k_new,
                                     int32_t n_idx_heads, const void* q_idx, const float* w,
                                     int32_t k, int32_t n_init, int32_t n_local,
                                     float* block_scores, int32_t* sel, int32_t* sel_pages,
                                     int32_t* counters, void* stream);

/*
 * Sparse GQA flash-decode with split-KV partials ([Rubin] commit messages: one unit of
 * work per (top-k split, KV head, query row), NVFP4 dequantised in registers). Query
 * head h reads KV head h / 16. Split s of num_splits takes the selection entries
 * [floor(s*k/S), floor((s+1)*k/S)); entry -1 is skipped; only tokens <= row_pos[r] are
 * visible. With x_p = softmax_scale * (q[r][h] . K_p) * log2(e), each split writes
 *   part_ml[r][h][s] = { m = max_p x_p, l = sum_p 2^(x_p - m) }  (m = -inf, l = 0 if empty)
 *   part_o[r][h][s][:] = sum_p 2^(x_p - m) * V_p                   (0 if empty)
 *   q         : bf16 [num_rows][num_q_heads][head_dim]
 *   sel       : int32 [num_rows][k] as written by msa_select_topk ([num_rows][T][k] with
 *               step->sel_tables = T > 1: KV head g reads table g)
 *   sel_pages : int32, the shape of sel, page ids as written by msa_select_topk, or NULL
 *               to look each block up in the block table
 *   part_o    : fp32 [num_rows][num_q_heads][num_splits][head_dim]  (output)
 *   part_ml   : fp32 [num_rows][num_q_heads][num_splits][2]         (output)
 * num_q_heads must be 16 * num_kv_heads; 1 <= num_splits <= k.
 * Accumulation is fp32 on the matrix cores; K and V are dequantised exactly to fp16.
 */
msa_status_t msa_sparse_decode(const msa_kv_pool_t* pool, const msa_step_t* step,
                               int32_t num_q_heads, const void* q, const int32_t* sel,
                               const int32_t* sel_pages, int32_t k, float softmax_scale,
                               int32_t num_splits, float* part_o, float* part_ml, void* stream);

/*
 * msa_sparse_decode followed by msa_combine in one launch: the last splits of each
 * (row, KV head) to count themselves in (the largest power of two not above num_splits,
 * each taking an equal slice of the 16 query heads) merge all splits of that row and
 * head exactly as msa_combine does ([Rubin] "Items and numerics", LC_ONEDIV: same order, same
 * arithmetic, so `out` equals msa_sparse_decode + msa_combine bit for bit) and writes
 * bf16 `out` [num_rows][num_q_heads][head_dim].
 *   part_o, part_ml, counters : the merge workspace. part_o fp32
 *     [num_rows][num_kv_heads][2][16][num_splits][head_dim] and part_ml fp32
 *     [num_rows][num_kv_heads][2][16][num_splits][2] hold two exchange buffers per
 *     (row, KV head), used by alternate calls (the layout does not depend on num_rows,
 *     so a workspace sized for R rows serves any call with num_rows <= R);
 *     counters int32 [num_rows][num_kv_heads] holds one state word
 *     per (row, KV head): bit 31 = the buffer the next call uses, bits 26..30 = the
 *     split count the workspace is set up for, bit 25 = a failure bit (below), bits
 *     8..22 = slices handed from one merging split to another and bits 0..7 = arrivals
 *     (both zero between calls). msa_merge_workspace_init sets it up for one num_splits (both buffers
 *     idle: every word MSA_MERGE_IDLE_BITS); every call with that num_splits leaves it
 *     ready for the next one. The partials pass through the buffers and are not left
 *     readable. An allocation sized for S splits serves any num_splits <= S after a
 *     set-up for that num_splits (the words are laid out for the num_splits in use). A call whose num_splits (> 1) differs from the set-up one, or that
 *     finds a state word out of range, touches no workspace word and writes bf16 NaN
 *     to that (row, KV head)'s outputs: call msa_merge_workspace_init again before
 *     changing num_splits. With num_splits == 1 the one split writes `out` itself and
 *     the workspace is neither read nor written. Two calls that share a workspace must
 *     not run concurrently. num_splits <= 16.
 *   The last split to arrive waits for the other splits' partials with a bounded poll
 *     (about 2^16 rounds; every split it waits for is already running). A merging split
 *     that arrived earlier polls for a few dozen rounds at most, then hands its slice to
 *     the last split (the outputs are the same either way). If the last split's bound is
 *     ever reached (a split held off the GPU for milliseconds), the outputs it could not
 *     merge are bf16 NaN and the pair's state word keeps the failure bit, so
 *     every later call writes NaN for that (row, KV head) as for a workspace set up for
 *     another split count, until msa_merge_workspace_init; the debug library also
 *     reports MSA_DEBUG_MERGE_TIMEOUT.
 */
msa_status_t msa_sparse_decode_combine(const msa_kv_pool_t* pool, const msa_step_t* step,
                                       int32_t num_q_heads, const void* q, const int32_t* sel,
                                       const int32_t* sel_pages, int32_t k, float softmax_scale,
                                       int32_t num_splits, float* part_o, float* part_ml,
                                       int32_t* counters, void* out, void* stream);

/*
 * msa_select_topk + msa_sparse_decode + msa_combine in one launch: every workgroup of a
 * query row runs the row's selection (the deterministic contract of msa_select_topk)
 * from block_scores itself, then decodes its split, and the last split of each
 * (row, KV head) merges as msa_sparse_decode_combine does.
 *   block_scores : fp32 [num_rows][max_blocks_per_seq] as written by msa_index_score
 *   sel, sel_pages : optional outputs (may be NULL), the selection msa_select_topk writes
 *   part_o, part_ml, counters : the idle merge workspace of msa_sparse_decode_combine
 * Other arguments as msa_sparse_decode_combine; num_splits <= 16.
 */
msa_status_t msa_select_decode_combine(const msa_kv_pool_t* pool, const msa_step_t* step,
                                       int32_t num_q_heads, const void* q,
                                       const float* block_scores, int32_t k, int32_t n_init,
                                       int32_t n_local, float softmax_scale, int32_t num_splits,
                                       float* part_o, float* part_ml, int32_t* counters,
                                       void* out, int32_t* sel, int32_t* sel_pages, void* stream);

/*
 * The whole decode step in ONE launch: msa_kv_append + msa_index_score +
 * msa_select_topk + msa_sparse_decode + msa_combine, with the results of those calls
 * ([GB300] "The TP4 decode target": the decode megakernels fuse block selection and
 * the KV update; "The TP8 decode target": index scoring fused with block selection).
 * Saves the launch between msa_append_score_select and msa_select_decode_combine.
 * The decode workgroups of each group of rows (up to 4 rows of one request) first score
 * that group's blocks, each wave at most two blocks, into the score exchange; every
 * workgroup then selects its row's blocks from the exchange as the scores land (an
 * agent-coherent poll), decodes its split and merges as msa_select_decode_combine
 * does. New tokens are encoded into the pool by the same launch; the scorer and the
 * decode take each new token's key, K and V from its bf16 source (the same encoding)
 * rather than from the pool, so out, sel and block_scores equal those of the calls
 * above bit for bit.
 *   Arguments of msa_kv_append, msa_index_score, msa_select_topk and
 *   msa_select_decode_combine, and:
 *   score_x     : fp32 [num_rows][max_blocks_per_seq], the score exchange. Every word
 *                 must be MSA_MERGE_IDLE_BITS before the call, and is so again after it
 *                 (msa_step_workspace_init sets it up).
 *   score_words : int32 [num_rows], zero before the call and again after it.
 *   block_scores : optional output (may be NULL), [num_rows][max_blocks_per_seq] as
 *                 msa_index_score writes it; sel, sel_pages : optional outputs as in
 *                 msa_select_decode_combine.
 *   part_o, part_ml, counters : the merge workspace of msa_select_decode_combine.
 * The single launch covers: n_idx_heads == 4, MSA_INDEX_E4M3 keys, one selection table
 * per row, a stated row count per request (step->rows_per_seq = R > 0), n_new <= 64,
 * the decode shape of 4 or 8 waves per workgroup (at most 2 selected blocks per split)
 * and rows of at most 64 * 2 * 8 candidate blocks, max_blocks_per_seq at most twice the
 * waves of the smallest group of rows ((R % 4, or 4) * num_kv_heads * num_splits
 * workgroups of 4 or 8 waves), and at most 256 workgroups per group. Other shapes
 * return MSA_ERR_UNSUPPORTED and launch nothing: use the two-launch entries. Two
 * calls that share score_x, score_words or the merge workspace must not run
 * concurrently. A workgroup waits only for workgroups of its own group of rows, which
 * are dispatched before it or with it; its poll is bounded (about 2^16 rounds), and if
 * the bound is ever reached its outputs are bf16 NaN (the debug library reports
 * MSA_DEBUG_SCORE_TIMEOUT).
 */
msa_status_t msa_decode_step(const msa_kv_pool_t* pool, const msa_step_t* step, int32_t n_new,
                             const int64_t* slot, const void* k_new, const void* v_new,
                             const void* idx_k_new, int32_t n_idx_heads, const void* q_idx,
                             const float* w, int32_t num_q_heads, const void* q, int32_t k,
                             int32_t n_init, int32_t n_local, float softmax_scale,
                             int32_t num_splits, float* score_x, int32_t* score_words,
                             float* part_o, float* part_ml, int32_t* counters, void* out,
                             float* block_scores, int32_t* sel, int32_t* sel_pages, void* stream);

/*
 * Set up msa_decode_step's score exchange for `rows` rows of max_blocks_per_seq
 * blocks: every word of score_x [rows][max_blocks] = MSA_MERGE_IDLE_BITS, every word of
 * score_words [rows] = 0. A fill kernel on `stream` (no memset nodes). Needed once after
 * allocation and again if anything else wrote the exchange.
 */
msa_status_t msa_step_workspace_init(int32_t rows, int32_t max_blocks, float* score_x,
                                     int32_t* score_words, void* stream);

/*
 * Sparse decode of groups of query rows over the union of their selections (query
 * pairing for speculative verify: [Rubin] commit messages name query pairing among
 * the tuned parameters of the NVFP4 sparse decode at 4 query rows per request). A
 * group is 1..max_group_rows rows of ONE request; the rows of a group that selected
 * the same block share one read of its page, and each row applies its own causal
 * mask (its visible tokens) and keeps its own softmax state, so every row's result
 * is the attention msa_sparse_decode + msa_combine compute for it (up to the order
 * of the fp32 sums).
 *   sel, sel_pages : as msa_sparse_decode ([num_rows][k], or [num_rows][T][k] with
 *     step->sel_tables = T > 1); a block is listed at most once in a row's table
 *   group_rows : int32 [num_groups + 1], ascending row offsets: group i is the rows
 *     [group_rows[i], group_rows[i + 1]), at most max_group_rows (1..MSA_MAX_GROUP_ROWS)
 *     of them, all with the same row_seq; with sel_pages, a block has the same page in
 *     every row of its group. Rows in no group are not written. The union of group i
 *     lists each selected block once, in order of its first pick (rows in order, each
 *     table in order); split s of num_splits takes its entries
 *     [s N / num_splits, (s + 1) N / num_splits) of the N entries.
 *   num_splits == 1 : writes bf16 out [num_rows][num_q_heads][head_dim] (part_o and
 *     part_ml unused, may be NULL)
 *   num_splits > 1  : writes the partials of msa_sparse_decode's layout, part_o fp32
 *     [num_rows][num_q_heads][num_splits][head_dim] and part_ml fp32
 *     [num_rows][num_q_heads][num_splits][2], for msa_combine (out unused, may be NULL);
 *     a split that holds none of a row's blocks writes m = -inf, l = 0, O = 0 for it
 * Choosing group sizes: a group's rows share each page read and V's dequantisation,
 * but every row of a group keeps its own scores, softmax and O, and the four-row
 * variant runs two waves per SIMD. Groups of several rows pay only when the rows share
 * nearly all of their blocks; groups of one row (the rounds software-pipelined) are
 * the faster one-split table-driven decode of 40 x 4 verify rows on gfx950.
 * 1 <= num_splits <= 64 (msa_combine's limit). The release library drops a table entry
 * that is neither -1 nor a visible block of its row, or whose page is negative; the
 * debug library also reports it (MSA_DEBUG_BAD_SEL) and reports a group that breaks
 * the rules above (MSA_DEBUG_BAD_GROUP), whose rows are then clamped to
 * [0, num_rows) and to max_group_rows.
 */
msa_status_t msa_sparse_decode_union(const msa_kv_pool_t* pool, const msa_step_t* step,
                                     int32_t num_q_heads, const void* q, const int32_t* sel,
                                     const int32_t* sel_pages, int32_t k, int32_t num_groups,
                                     const int32_t* group_rows, int32_t max_group_rows,
                                     float softmax_scale, int32_t num_splits, float* part_o,
                                     float* part_ml, void* out, void* stream);

/*
 * msa_sparse_decode_combine for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the merge workspace, and the same bf16 `out` bit for bit. The split
 * partials live in a fixed array of MSA_NOALLOC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends; a call whose partials,
 * num_rows * num_q_heads * num_splits * (head_dim + 2) fp32 (part_o rounded up to 256
 * bytes), exceed it returns MSA_ERR_TOO_LARGE and launches nothing. num_splits == 1
 * decodes in one launch without touching the array; num_splits > 1 (<= 16) decodes into
 * it and merges with msa_combine, two launches. Nothing is allocated or freed (the
 * first call on a device looks up the array's address; MSA_ERR_LAUNCH if the runtime
 * cannot give it). Other errors as msa_sparse_decode_combine. Every call on one GPU shares
 * that GPU's array: calls that can overlap on one GPU (on different streams, or from
 * several host threads) race and must be ordered by the caller.
 */
#define MSA_NOALLOC_SCRATCH_BYTES (8u << 20)
msa_status_t msa_sparse_decode_combine_noalloc(const msa_kv_pool_t* pool, const msa_step_t* step,
                                               int32_t num_q_heads, const void* q, const int32_t* sel,
                                               const int32_t* sel_pages, int32_t k, float softmax_scale,
                                               int32_t num_splits, void* out, void* stream);

/*
 * Set up a merge workspace of the two *_combine entries for `num_splits` splits: every
 * word of both exchange buffers, part_o [rows][num_q_heads / 16][2][16][num_splits]
 * [head_dim] and part_ml [rows][num_q_heads / 16][2][16][num_splits][2], =
 * MSA_MERGE_IDLE_BITS, and every
 * state word in counters [rows][num_q_heads / 16] = buffer 0, num_splits, no arrivals
 * (num_splits << 16). A fill kernel on `stream` (no memset nodes, so the call may be
 * captured in a graph). Needed once after allocation, again before calls with another
 * num_splits, and if anything else wrote the workspace. num_splits <= 16.
 */
msa_status_t msa_merge_workspace_init(int32_t rows, int32_t num_q_heads, int32_t head_dim,
                                      int32_t num_splits, float* part_o, float* part_ml,
                                      int32_t* counters, void* stream);

/*
 * Log-sum-exp merge of split partials ([Rubin] "Items and numerics", LC_ONEDIV: the
 * split-K merge divides once per output, in a fixed order, without atomics):
 *   M = max_s m_s,  out = (sum_s 2^(m_s - M) O_s) / (sum_s 2^(m_s - M) l_s)
 * summed over s = 0..num_splits-1 in order, rounded once to bf16 (nearest even).
 * A row/head whose splits are all empty gets 0.
 *   out : bf16 [rows][num_q_heads][head_dim] (output)
 */
msa_status_t msa_combine(int32_t rows, int32_t num_q_heads, int32_t head_dim,
                         int32_t num_splits, const float* part_o, const float* part_ml,
                         void* out, void* stream);

/* Bytes of the part_o + part_ml workspace for the given geometry (part_o first, then
 * part_ml at a 256-byte aligned offset). Returns 0 for invalid arguments. */
size_t msa_decode_workspace_bytes(int32_t rows, int32_t num_q_heads, int32_t head_dim,
                                  int32_t num_splits);

/* Exact bytes of each pool array for a geometry: out[0..4] = k_codes, v_codes,
 * k_scales, v_scales, index_k. Returns MSA_ERR_UNSUPPORTED / INVALID_ARG like the
 * entry points. */
msa_status_t msa_pool_bytes(int32_t fmt, int32_t num_pages, int32_t num_kv_heads,
                            int32_t head_dim, int32_t index_dim, size_t out[5]);

/* Exact bytes of the index-key arrays: out[0] = index_k, out[1] = index_scales (0 for
 * MSA_INDEX_E4M3). */
msa_status_t msa_index_bytes(int32_t index_fmt, int32_t num_pages, int32_t index_dim, size_t out[2]);

/* A static string naming the status. */
const char* msa_status_string(msa_status_t status);

/*
 * Device-side metadata checks. The release library trusts the device arrays (page ids,
 * requests, positions, selections). The debug library, libmsadecode_debug.so (the same
 * sources built with -DMSA_DEBUG_CHECKS), checks them where the kernels use them: a
 * failed check writes its code to the caller's error word if the word is still 0 (the
 * first failure wins) and skips the access it guards (the affected scores, selections
 * or outputs are then meaningless, but nothing is read or written out of bounds).
 *   MSA_DEBUG_BAD_PAGE : a page id from the block table or sel_pages outside [0, num_pages)
 *   MSA_DEBUG_BAD_SEQ  : a row_seq value outside [0, num_seqs)
 *   MSA_DEBUG_BAD_POS  : a row_pos whose block lies past max_blocks_per_seq
 *   MSA_DEBUG_BAD_SEL  : a selection entry neither -1 nor a visible block of its row
 *   MSA_DEBUG_BAD_SLOT : an append slot whose page lies outside [0, num_pages)
 *   MSA_DEBUG_MERGE_TIMEOUT : a merging split gave up waiting for another split's
 *                       partial (see msa_sparse_decode_combine)
 *   MSA_DEBUG_BAD_GROUP : a row group of msa_sparse_decode_union that is out of order,
 *                       outside [0, num_rows), longer than max_group_rows or mixes requests
 *   MSA_DEBUG_SCORE_TIMEOUT : a workgroup of msa_decode_step gave up waiting for its
 *                       row's scores (see msa_decode_step)
 * msa_debug_set_error_word sets the device int32 word (NULL: none) that every later
 * call of the debug library, on any stream, reports to; the caller zeroes and reads
 * it. msa_debug_set_merge_poll_limit sets the number of poll rounds after which a
 * merging split gives up (polls < 0: the release bound; 0: give up without reading,
 * which lets a test force the failure path while every kernel still exits normally).
 * msa_debug_set_merge_helper_poll_limit sets the number of poll rounds after which a
 * merging split other than the last to arrive hands its slice of the heads to the last
 * one (polls < 0: the release bound; 0: hand over at once wherever the last split has
 * not yet arrived, which lets a test force the handoff path; the outputs are the same
 * either way). All three are process-wide state of the debug library only. The release
 * library returns MSA_ERR_UNSUPPORTED for them, and msa_debug_checks_enabled tells the
 * two builds apart (1 / 0).
 */
typedef enum {
  MSA_DEBUG_OK = 0,
  MSA_DEBUG_BAD_PAGE = 1,
  MSA_DEBUG_BAD_SEQ = 2,
  MSA_DEBUG_BAD_POS = 3,
  MSA_DEBUG_BAD_SEL = 4,
  MSA_DEBUG_BAD_SLOT = 5,
  MSA_DEBUG_MERGE_TIMEOUT = 6,
  MSA_DEBUG_BAD_GROUP = 7,
  MSA_DEBUG_SCORE_TIMEOUT = 8
} msa_debug_error_t;

msa_status_t msa_debug_set_error_word(int32_t* word);
msa_status_t msa_debug_set_merge_poll_limit(int32_t polls);
msa_status_t msa_debug_set_merge_helper_poll_limit(int32_t polls);
int32_t msa_debug_checks_enabled(void);

#ifdef __cplusplus
}
#endif
#endif /* MSA_DECODE_H_ */
