/*
 * gdn_paged.h -- Gated Delta-Rule prefill and decode on a paged recurrent-state
 * pool, for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Semantics follow the flashinfer.gdn_paged API page (docs.flashinfer.ai,
 * "flashinfer.gdn_paged"): its opening paragraph, the "Page table" section and
 * the "Slot arguments of chunk_gated_delta_rule" section.  The page names the
 * Gated Delta-Rule without writing it out; this library computes, per v-head,
 * with a state S of shape [V, K]:
 *
 *     alpha_t = exp(g_t)
 *     S_t     = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T
 *     o_t     = scale * S_t q_t           (scale = 1/sqrt(K) unless given)
 *
 * Data layout (row-major, all device memory, all owned by the caller):
 *   q, k         [T, Hqk, K]  bf16 (raw 16-bit patterns)
 *   v            [T, H, V]    bf16
 *   g, beta      [T, H]       fp32 (either may be NULL: g = 0, beta = 1); g
 *                finite (the chunked prefill takes differences of decay sums
 *                within a chunk: a reset is a large negative g, not -inf).  A
 *                NaN in g, beta or k reaches at least what the recurrence
 *                would reach, and in the prefill also the earlier rows of its
 *                64-token chunk; a NaN in v reaches the state rows of its
 *                32-column group, but not the states past the segment it
 *                sits in when the sequence-parallel first pass leaves its
 *                chunk out (it may, because for finite v the decay after
 *                that chunk makes its contribution invisible at fp32)
 *   o            [T, H, V]    bf16, written for every new token
 *   state pools  [rows, H, V, K] fp32 or bf16 (gdn_dims_t.state_dtype, one type
 *                for every state buffer of a call); each row is one dense
 *                [H, V, K] block and consecutive rows sit `row_stride`
 *                elements apart (>= H*V*K).  The arithmetic is the same for
 *                both types; a bf16 buffer receives each stored state rounded
 *                to nearest even (the page requires one element type that
 *                both entry points accept; fp32 and bf16 both qualify).
 * Decode uses B (one token per sequence) in place of T.
 * v-head h reads q/k head h / (H / Hqk).
 *
 * Calls are asynchronous on `stream`, never synchronize with the host and
 * allocate nothing: the caller passes a workspace where one is needed
 * (gdn_prefill_workspace_size).  A call only launches kernels on `stream` (no
 * memset, copy or allocation), so it can be captured into a HIP graph and
 * replayed; the launch shapes are taken on the host from the sizes and
 * dims->options, the sequence-parallel plan on the device from the batch's
 * lengths, so a replay follows the lengths of its own inputs.  Return value:
 * GDN_OK or a negative status,
 * set before any launch for every check the host can make; the message is in
 * gdn_last_error() (thread-local).  Device-side contents are NOT validated
 * (the page says slots are not checked against the page table): page ids must
 * be real rows of the pool, decode sequences must hold a token before the
 * decoded one, and rows one sequence writes must be neither read nor written
 * by another sequence of the same call.  Breaking these is undefined
 * behaviour.
 *
 * Supported: K = V = 128, H a multiple of Hqk, page_size a positive multiple
 * of 64, any positive checkpoint_every_n_tokens (a checkpoint inside a 64-token
 * chunk costs one more state-update product in that chunk).  Token positions
 * are 32-bit: a sequence's prefix plus its new tokens, and the checkpoint
 * positions up to it plus checkpoint_every_n_tokens, stay below 2^31.
 */
#ifndef GDN_PAGED_H
#define GDN_PAGED_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  GDN_OK = 0,
  GDN_EINVAL = -1,        /* bad argument (null pointer, size, missing companion) */
  GDN_EUNSUPPORTED = -2,  /* valid per the page but not served by this library */
  GDN_ELAUNCH = -3,       /* a kernel launch failed */
  GDN_EWORKSPACE = -4     /* workspace missing or too small */
};

enum { GDN_INDEX_INT32 = 0, GDN_INDEX_INT64 = 1 };
enum { GDN_STATE_F32 = 0, GDN_STATE_BF16 = 1 };

/*
 * Launch choices of one call.  Every field at 0 selects the library's
 * default (what the measurements use); the other values exist for tests and
 * tuning, and every choice computes the same recurrence (decode shapes give
 * bit-identical results, prefill shapes agree within the tolerances).  The
 * library reads no environment variables and keeps no per-call settings of
 * its own: a choice is made by passing it here.  Under HIP graph capture the
 * choices in force at capture time are frozen into the graph, like any other
 * argument.
 *   prefill_split_chunks  sequence-parallel recurrence: 0 = decided on the
 *                         device from the batch's lengths (possible when
 *                         B * H <= 256); -1 = never; m > 0 = every sequence in
 *                         segments of m chunks of 64 tokens.
 *   prefill_tile_waves    waves per recurrence workgroup: 0 or 8 = whole heads;
 *                         4, 2 or 1 = V-tiles of 64, 32 or 16 state rows.
 *   decode_waves          2, 4, 8 or 16: the one-(sequence, head)-per-workgroup
 *                         decode kernel of that width; 0 = default.
 *   decode_stream_per_cu  streaming decode (16 waves) workgroups per compute
 *                         unit; -1 = the one-pair kernel; 0 = default: 6 for
 *                         fp32 state; for bf16 state (with the two other
 *                         decode fields 0) the streaming kernel with 4 waves
 *                         and one workgroup per (sequence, head).
 *   decode_stream_grid    > 0: streaming decode with exactly this many
 *                         workgroups (overrides decode_stream_per_cu).
 */
typedef struct {
  int32_t prefill_split_chunks;
  int32_t prefill_tile_waves;
  int32_t decode_waves;
  int32_t decode_stream_per_cu;
  int32_t decode_stream_grid;
  /* Debug validation (NULL = off, the default: nothing extra runs).  A
   * device int32: gdn_prefill_paged and gdn_decode_paged first run
   * gdn_check_paged into it (against a pool of check_num_pages rows), and
   * every later kernel of the call returns without reading or writing
   * anything when the word holds an error bit other than
   * GDN_CHECK_NOT_CHECKED; the caller reads the word when it likes (the
   * call itself never synchronizes). */
  int32_t* check_error_word;
  int32_t check_num_pages;
} gdn_options_t;

/* Head geometry shared by every call, and the call's launch choices. */
typedef struct {
  int32_t num_qk_heads; /* Hqk */
  int32_t num_v_heads;  /* H, also the pool's head count */
  int32_t head_dim_k;   /* K, must be 128 */
  int32_t head_dim_v;   /* V, must be 128 */
  float scale;          /* output scale; <= 0 selects 1/sqrt(K) */
  int32_t state_dtype;  /* GDN_STATE_F32 or GDN_STATE_BF16: element type of the state buffers */
  const gdn_options_t* options; /* host pointer, NULL = every default */
} gdn_dims_t;

/*
 * Per-sequence pool rows of a paged prefill batch, each a device array of
 * [num_seqs] int32 (flashinfer.gdn_paged, GDNPagedPrefillSlots, whose fields
 * the page gives as one int32 entry per sequence; it names state_indices, the
 * other fields are this library's reading of the paged call as a wrapper
 * over the slot arguments):
 *   state_indices         page holding the last prefix token, -1 if no prefix
 *   output_state_indices  last page, -1 for a sequence with no new tokens
 *   checkpoint_cu_starts  indptr[b] + prefix / page_size: where the pages that
 *                         end inside this call start in page_indices
 *   prefix_lens           tokens the sequence held before the call
 *   chunk_starts          exclusive prefix sum of 64-token chunk counts
 *                         (chunks sit at absolute multiples of 64)
 * The struct itself lives in host memory; its pointers are device pointers.
 */
typedef struct {
  int32_t* state_indices;
  int32_t* output_state_indices;
  int32_t* checkpoint_cu_starts;
  int32_t* prefix_lens;
  int32_t* chunk_starts;
} gdn_prefill_slots_t;

/* Per-sequence pool rows of a paged decode batch, [num_seqs] int32 each
 * (flashinfer.gdn_paged, GDNPagedDecodeSlots). */
typedef struct {
  int32_t* initial_state_indices;
  int32_t* output_state_indices;
} gdn_decode_slots_t;

/*
 * gdn_prefill_slots -- pool rows a paged prefill derives from its page table,
 * in one launch and without a host synchronization (flashinfer.gdn_paged,
 * gdn_paged_prefill_slots and "Page table").  The rows depend only on the
 * batch: compute them once per step and pass them to every layer's
 * gdn_prefill_paged, which then skips this launch.
 *   cu_seqlens [num_seqs+1], page_indices [indptr[num_seqs]],
 *   page_indptr [num_seqs+1], last_page_len [num_seqs]: int32 device arrays.
 *   out: five [num_seqs] int32 device arrays, written.
 * Errors: GDN_EINVAL for null pointers, num_seqs < 0, page_size not a positive
 * multiple of 64.
 */
int gdn_prefill_slots(const int32_t* cu_seqlens, const int32_t* page_indices,
                      const int32_t* page_indptr, const int32_t* last_page_len,
                      int32_t num_seqs, int32_t page_size,
                      const gdn_prefill_slots_t* out, hipStream_t stream);

/*
 * gdn_decode_slots -- decode rows (flashinfer.gdn_paged, gdn_paged_decode_slots):
 * a token that opens a new page (last_page_len == 1) reads the previous page
 * and writes the new one; otherwise both rows are the last page.
 * Errors: GDN_EINVAL for null pointers or num_seqs < 0.
 */
int gdn_decode_slots(const int32_t* page_indices, const int32_t* page_indptr,
                     const int32_t* last_page_len, int32_t num_seqs,
                     const gdn_decode_slots_t* out, hipStream_t stream);

/*
 * Workspace bytes gdn_prefill_paged / gdn_prefill need for a batch of
 * `total_tokens` new tokens in `num_seqs` sequences: an upper bound that
 * depends on sizes only and never decreases as either grows, so a workspace
 * sized for the largest call serves every call with at most as many tokens
 * and sequences.  0 on bad dims.
 * Batches whose (sequence, v-head) pairs fill at most the chip's compute
 * units once (B * H <= 256) may run the recurrence sequence-parallel: a long
 * sequence is cut into segments, each segment's transition S -> S M + N is
 * computed in parallel, the maps are composed in order, and the segments
 * rerun from their true start states.  Whether and how finely to cut is
 * decided on the device from the batch's actual lengths (or forced through
 * dims->options); the workspace then also holds three states (H * V * K
 * floats each) per segment, for at most 512 / H + B segments.  The size
 * depends on dims->options (prefill_split_chunks) as the call does.
 */
size_t gdn_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                  const gdn_dims_t* dims);

/*
 * gdn_prefill_paged -- chunked prefill that reads and writes a paged pool
 * (flashinfer.gdn_paged, chunk_gated_delta_rule_paged and "Page table"):
 *  - the initial state is the page holding the last prefix token, or zero
 *    when the prefix is empty;
 *  - the state at every page boundary the new tokens cross goes to the page
 *    ending there, and the final state to the last page;
 *  - pages that end at or before the prefix are never written; a prefix that
 *    ends inside a page continues that page in place;
 *  - prefixes need not be multiples of 64 (the first chunk is padded on the
 *    left); zero-length sequences leave the pool unchanged.
 * Sequence b owns pages page_indices[page_indptr[b] .. page_indptr[b+1]) and
 * holds (pages-1)*page_size + last_page_len[b] tokens after the call; its new
 * tokens are q/k/v rows cu_seqlens[b] .. cu_seqlens[b+1].
 *   slots: NULL, or rows from gdn_prefill_slots for this batch (not checked).
 *   total_tokens = cu_seqlens[num_seqs] (host copy; sizes the launch grids).
 *   workspace: >= gdn_prefill_workspace_size(total_tokens, num_seqs, dims)
 *   bytes of device memory, 256-byte aligned, contents scratch.
 * Errors: GDN_EINVAL (null pointer, negative size, page_size not a positive
 * multiple of 64, pool_row_stride < H*V*K), GDN_EUNSUPPORTED (K or V != 128,
 * H not a multiple of Hqk), GDN_EWORKSPACE, GDN_ELAUNCH.
 */
int gdn_prefill_paged(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const int32_t* cu_seqlens,
                      int32_t num_seqs, int64_t total_tokens, void* state_pool,
                      int64_t pool_row_stride, const int32_t* page_indices,
                      const int32_t* page_indptr, const int32_t* last_page_len,
                      int32_t page_size, const gdn_prefill_slots_t* slots, void* o,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gdn_check_paged -- debug validation of a paged batch, on the device in one
 * launch and without a host synchronization: writes to *error_word a mask of
 * the GDN_CHECK_* bits below (0 = nothing found).  The page says page tables
 * hold real page ids and slots are not validated against them, and that a
 * row one sequence writes must not be touched by another sequence of the
 * call (flashinfer.gdn_paged, "Page table", "Slot arguments"); this call
 * checks what the paged calls take on trust.
 *   cu_seqlens [num_seqs+1] for a prefill batch, NULL for a decode batch.
 *   page_indptr [num_seqs+1] and last_page_len [num_seqs] are read whole,
 *   page_indices for its page_indptr[num_seqs] entries (once page_indptr is
 *   found well formed); num_pages = rows of the pool.
 * The row check covers batches of up to 2048 sequences touching up to 4096
 * pages in all; beyond that it is skipped and GDN_CHECK_NOT_CHECKED is set.
 * Errors: GDN_EINVAL for null pointers, num_seqs < 1, page_size not a
 * positive multiple of 64, num_pages < 1.
 */
enum {
  GDN_CHECK_INDPTR = 1,         /* page_indptr[0] != 0, decreasing, or a sequence with no page */
  GDN_CHECK_LAST_PAGE_LEN = 2,  /* last_page_len outside 1 .. page_size */
  GDN_CHECK_TOKENS = 4,         /* prefill: cu_seqlens[0] != 0, or a sequence with a negative
                                   count or more new tokens than it holds; decode: a sequence
                                   holding no token before the decoded one */
  GDN_CHECK_PAGE_ID = 8,        /* a page id outside 0 .. num_pages - 1 */
  GDN_CHECK_SHARED_ROW = 16,    /* a row one sequence writes is read or written by another */
  GDN_CHECK_NOT_CHECKED = 32    /* batch beyond the row check's size: that check skipped */
};
int gdn_check_paged(const int32_t* cu_seqlens, const int32_t* page_indices,
                    const int32_t* page_indptr, const int32_t* last_page_len, int32_t num_seqs,
                    int32_t page_size, int32_t num_pages, int32_t* error_word,
                    hipStream_t stream);

/*
 * gdn_prefill_paged_noalloc -- gdn_prefill_paged for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments and results, without
 * the workspace.  Its workspace is a fixed scratch array of 256 MiB that the
 * library holds on every device it runs on, from its load until the process
 * ends; the call allocates nothing (its first call on a device only looks up
 * that array's address).  Every call on one device shares that device's
 * scratch and leaves its contents behind (nothing in it needs to start at
 * zero): calls that overlap on one device -- on two streams, or from two
 * threads -- race and give undefined results.  A call whose workspace
 * for its own T and B would exceed 256 MiB fails with GDN_EWORKSPACE before
 * any launch: at 32 v-heads, beyond about 28k new tokens in one sequence,
 * 19k in 8 sequences (batches that may run sequence-parallel also hold
 * segment states) and 43k in 36 sequences.
 * Errors: as gdn_prefill_paged.
 */
int gdn_prefill_paged_noalloc(const gdn_dims_t* dims, const void* q, const void* k,
                              const void* v, const float* g, const float* beta,
                              const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                              void* state_pool, int64_t pool_row_stride,
                              const int32_t* page_indices, const int32_t* page_indptr,
                              const int32_t* last_page_len, int32_t page_size,
                              const gdn_prefill_slots_t* slots, void* o, hipStream_t stream);

/*
 * gdn_decode_paged -- one token per sequence on a paged pool (flashinfer.gdn_paged,
 * gated_delta_rule_decode_paged): last_page_len[b] == 1 reads page n-2 and
 * writes page n-1, otherwise the last page is updated in place.  Every
 * sequence holds at least one token before the decoded one.
 *   q, k [num_seqs, Hqk, K], v [num_seqs, H, V], g, beta [num_seqs, H], o
 *   [num_seqs, H, V].  slots: NULL (rows are derived inside the decode
 *   kernel, no extra launch) or rows from gdn_decode_slots.
 * Errors as gdn_prefill_paged (no workspace is needed).
 */
int gdn_decode_paged(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                     const float* g, const float* beta, int32_t num_seqs, void* state_pool,
                     int64_t pool_row_stride, const int32_t* page_indices,
                     const int32_t* page_indptr, const int32_t* last_page_len,
                     int32_t page_size, const gdn_decode_slots_t* slots, void* o,
                     hipStream_t stream);

/*
 * gdn_prefill -- the slot-argument prefill that the paged call wraps
 * (flashinfer.gdn_paged, "Slot arguments of chunk_gated_delta_rule").
 *   initial_state [rows, H, V, K] or NULL (all sequences start from zero);
 *   state_indices: read row per sequence (-1 = zero state); NULL = row b.
 *   output_final_state: store final states into output_state;
 *   output_state_indices: write row per sequence (-1 = skip); NULL = the read
 *     row (state_indices[b], or b).  Needs output_state and
 *     output_final_state.  A zero-length sequence writes nothing.
 *   state_checkpoints + checkpoint_state_indices + checkpoint_cu_starts +
 *     prefix_lens + checkpoint_every_n_tokens (N): after new token n of
 *     sequence i with (prefix_lens[i] + n) % N == 0, the state goes to row
 *     checkpoint_state_indices[checkpoint_cu_starts[i] + j] (j counts the
 *     call's checkpoints from 0; -1 skips).  Sequence i takes
 *     (prefix_lens[i] + len_i)/N - prefix_lens[i]/N checkpoints.
 *   prefix_lens alone (no checkpoints) only aligns chunks; results match.
 *   index_dtype: GDN_INDEX_INT32 or GDN_INDEX_INT64 for state_indices,
 *     output_state_indices, checkpoint_state_indices, checkpoint_cu_starts and
 *     prefix_lens.  cu_seqlens is always int32.
 *   The three state buffers may be the same memory.
 * Errors: GDN_EINVAL (as above; output_state_indices without output_state or
 * output_final_state; checkpoint rows without N > 0, prefix_lens,
 * checkpoint_cu_starts or state_checkpoints), GDN_EUNSUPPORTED (K or V !=
 * 128), GDN_EWORKSPACE, GDN_ELAUNCH.
 */
int gdn_prefill(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
                const float* g, const float* beta, const int32_t* cu_seqlens,
                int32_t num_seqs, int64_t total_tokens,
                const void* initial_state, int64_t initial_row_stride,
                const void* state_indices,
                void* output_state, int64_t output_row_stride,
                const void* output_state_indices, int32_t output_final_state,
                void* state_checkpoints, int64_t checkpoint_row_stride,
                const void* checkpoint_state_indices, const void* checkpoint_cu_starts,
                const void* prefix_lens, int32_t checkpoint_every_n_tokens,
                int32_t index_dtype, void* o, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * gdn_decode -- single-token step with explicit rows (the decode counterpart
 * of the slot arguments).  initial_state NULL or a read row of -1 starts from
 * zero; initial_state_indices NULL = row b; output_state_indices NULL = the
 * read row; a write row of -1 skips the store.
 */
int gdn_decode(const gdn_dims_t* dims, const void* q, const void* k, const void* v,
               const float* g, const float* beta, int32_t num_seqs,
               const void* initial_state, int64_t initial_row_stride,
               const void* initial_state_indices, void* output_state,
               int64_t output_row_stride, const void* output_state_indices,
               int32_t index_dtype, void* o, hipStream_t stream);

/*
 * gdn_block_table_to_csr -- padded block table -> the CSR page table the
 * paged calls take, on the device, in two launches and without a host
 * synchronization (FlashInfer CSR paging drill, section 2: a sequence of ctx
 * tokens owns ceil(ctx / page_size) pages; indptr is the running sum of those
 * counts with indptr[0] = 0; the indices are the first that many entries of
 * every row, rows in order; the last page holds ctx - (pages - 1) * page_size
 * tokens, 1 .. page_size).
 *   block_tables  [num_seqs, row_stride] int32 device array; only the first
 *                 ceil(ctx_lens[b] / page_size) entries of row b are read.
 *   ctx_lens      [num_seqs] int32 device array, tokens per sequence.
 *   max_blocks    columns a row may use (<= row_stride).
 *   page_indptr   [num_seqs + 1] int32 device array, written.
 *   page_indices  int32 device array with room for num_seqs * max_blocks
 *                 entries; the first page_indptr[num_seqs] are written.
 *   last_page_len [num_seqs] int32 device array, written.
 *   bad_rows      optional [1] int32 device array, written: the number of
 *                 rows the CSR form cannot hold (ctx_lens < 1, or more than
 *                 max_blocks pages).  Such rows get no pages and
 *                 last_page_len 0; a table with bad rows must not be passed to
 *                 the paged calls.
 * Errors: GDN_EINVAL for null pointers, num_seqs < 0, page_size <= 0,
 * max_blocks < 0 or row_stride < max_blocks.
 */
int gdn_block_table_to_csr(const int32_t* block_tables, int64_t row_stride,
                           const int32_t* ctx_lens, int32_t num_seqs, int32_t max_blocks,
                           int32_t page_size, int32_t* page_indptr, int32_t* page_indices,
                           int32_t* last_page_len, int32_t* bad_rows, hipStream_t stream);

/*
 * gdn_csr_to_block_table -- CSR page table -> padded block table and context
 * lengths, on the device, without a host synchronization (FlashInfer CSR
 * paging drill, section 3: page counts are adjacent differences of indptr; a
 * row is the sequence's pages followed by zeros; ctx = (pages - 1) *
 * page_size + last_page_len).
 *   page_indptr [num_seqs + 1], page_indices [page_indptr[num_seqs]],
 *   last_page_len [num_seqs]: int32 device arrays.
 *   block_tables [num_seqs, row_stride] int32 device array; columns
 *                0 .. max_blocks - 1 of every row are written.
 *   ctx_lens     [num_seqs] int32 device array, written.
 *   bad_rows     optional [1] int32 device array, written: the number of
 *                rows with no pages, more than max_blocks pages or
 *                last_page_len outside 1 .. page_size; such rows are written
 *                as all padding with ctx_lens 0, and page_indices is not read
 *                for them.
 * Errors: GDN_EINVAL for null pointers, num_seqs < 0, page_size <= 0,
 * max_blocks < 0 or row_stride < max_blocks.
 */
int gdn_csr_to_block_table(const int32_t* page_indptr, const int32_t* page_indices,
                           const int32_t* last_page_len, int32_t num_seqs, int32_t page_size,
                           int32_t max_blocks, int32_t* block_tables, int64_t row_stride,
                           int32_t* ctx_lens, int32_t* bad_rows, hipStream_t stream);

/*
 * gdn_stream_copy -- copies `bytes` bytes from src to dst (device pointers,
 * 16-byte aligned, not overlapping) on `stream`, with the memory access
 * pattern of the decode kernel (16-byte non-temporal loads and stores, a
 * fixed grid of 8 workgroups per compute unit walking 32 KiB units, each
 * unit's successor loaded before the unit is stored).  Not part of the
 * method: it gives the rate an HBM-bound kernel of this library can reach on
 * the GPU at hand, which the benchmark reports beside the decode's.
 * Errors: GDN_EINVAL for a size that is negative or not a multiple of 16,
 * null, unaligned or overlapping pointers (bytes == 0 does nothing),
 * GDN_ELAUNCH.
 */
int gdn_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream);

/* Message of the last failing call on this thread ("" if none). */
const char* gdn_last_error(void);

/* Library version string. */
const char* gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PAGED_H */
