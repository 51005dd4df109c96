/*
 * pkd.h -- C ABI of libpkd: one batched transformer decode step over a paged
 * KV pool, built for AMD Instinct MI355X (gfx950).
 *
 * Sources for the operations (cited by page title and section):
 *   [GIE]  "GPU inference engine engineering" (coreyjames.ai)
 *   [H100] "Building an LLM runtime from scratch on NVIDIA H100" (svms.in)
 *   [LRS]  "llm-rs: LLM Inference in Rust, from cuTile Tiles to Hand-Written
 *          SIMT Kernels" (mohankku.github.io)
 *   [ENG]  "Engines for the card you have" (coreyjames.ai)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Device memory is owned by the caller.  The library allocates no device
 *    memory in any call; it keeps only small host handles.  A refused call
 *    therefore leaks nothing ([GIE] "Batching without running out of cache":
 *    a failed load frees what it took, memory need is computed without
 *    allocating).
 *  - Every call that launches work takes a stream (a hipStream_t passed as
 *    pkd_stream; NULL is the default stream), enqueues asynchronously and
 *    never synchronises the host, except the admission-time pool calls
 *    kv_pool_create, block_table_set and pkd_pool_check, which say so.  No
 *    hot call allocates ([LRS] section 4, lesson 1: one workspace per request
 *    instead of allocation inside the decode loop).
 *  - Every call returns a pkd_status (0 = PKD_OK).  If `err` is non-NULL it
 *    receives a typed refusal with the numbers involved ([GIE] "Batching
 *    without running out of cache": admission refuses with a typed reason and
 *    the numbers).  Host-visible arguments are validated before anything is
 *    launched; on refusal nothing is launched and nothing is modified.
 *  - Device pointers must be 16-byte aligned unless a call states otherwise.
 *  - Threads and streams: paged_attn_decode and decode_step write the pool
 *    (each row's own key and value, and the sticky error word).  Calls on
 *    different pools may run from several host threads and streams at once;
 *    calls on one pool may overlap only when they touch disjoint sequences
 *    (and no shared page is appended to).  block_table_set and
 *    kv_pool_destroy change a pool's host state and must not overlap any
 *    other call on the same pool; launches that read the tables a
 *    block_table_set replaces must be complete before it is called.
 *  - Determinism: the output of a row depends only on that row's inputs, its
 *    sequence's pages, the weights and the fixed configuration of the pool or
 *    matrix.  It is bit-identical in any batch, at any position in the batch
 *    and across runs ([GIE] "The same bits in any batch").
 */
#ifndef PKD_H
#define PKD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* pkd_stream; /* hipStream_t */

typedef enum {
  PKD_OK = 0,
  PKD_ERR_INVALID_ARG = 1,    /* null or misaligned pointer, bad enum, n < 0 */
  PKD_ERR_UNSUPPORTED = 2,    /* geometry / dtype / family not built */
  PKD_ERR_OUT_OF_MEMORY = 3,  /* caller buffer too small: needed, available in bytes */
  PKD_ERR_BOUNDS = 4,         /* index or count out of range: needed, available */
  PKD_ERR_DUPLICATE_PAGE = 5, /* a page id appears twice in one sequence's table */
  PKD_ERR_DEVICE = 6,         /* HIP runtime error; detail holds its text */
  PKD_ERR_ROW = 7             /* pkd_pool_check: some row had an invalid (seq, pos) or table entry */
} pkd_status;

typedef struct {
  int32_t code;      /* a pkd_status */
  int64_t needed;    /* e.g. bytes needed, pages requested, index given */
  int64_t available; /* e.g. bytes given, pages allowed, valid range end */
  char detail[192];  /* human-readable, NUL-terminated */
} pkd_error;

typedef enum {
  PKD_F32 = 0,
  PKD_BF16 = 1,     /* bfloat16; every rounding to it is round-to-nearest-even */
  PKD_FP8_E4M3 = 2  /* OCP E4M3FN: bias 7, max 448, no infinities, S.1111.111 = NaN */
} pkd_dtype;

typedef enum {
  PKD_FAMILY_GEMV = 0,    /* decode batches: one 64-lane wavefront per 4 weight rows, each lane
                             reading 16-byte vectors (1 KiB runs per wave load), vector ALU,
                             fp32 accumulate */
  PKD_FAMILY_MFMA = 1,    /* tiled matrix-core contraction for large batches: bf16 operands, or
                             fp8 operands decoded exactly to bf16 on chip; products exact and
                             sums with fp32 accumulation */
  PKD_FAMILY_MFMA_FP8 = 2, /* fp8 weights only: the native fp8 matrix-core instruction, twice the
                             matrix-core rate, but each instruction sums its 128 products with
                             ~17 significant bits (measured relative error of a projection
                             ~2e-5 instead of ~1e-7) */
  PKD_FAMILY_GEMV_MFMA = 3 /* GEMV on the matrix cores for decode batches of about 8 to 16:
                             groups of 16 weight rows read straight into registers (one or two
                             groups per wave, by matrix height), the batch as the product's 16
                             columns; bf16 or fp8 weights (fp8 decoded exactly), bf16
                             activations, fp32 accumulation.  Measured on the 7B matrices:
                             faster than PKD_FAMILY_GEMV from batch 8 (146 against 200 us at
                             16), slower below (106 against 94 us at 1). */
} pkd_family;

/* ------------------------------------------------------------------------ */
/* KV pool                                                                   */
/* ------------------------------------------------------------------------ */

/*
 * Geometry of a paged KV pool ([GIE] "Batching without running out of cache":
 * KV memory is a pool of 32-token pages and each sequence has a block table
 * mapping its logical pages to physical ones; [LRS] section 5: attention
 * fetches one block per chunk through the table).  The geometry is fixed at
 * creation, as an engine is committed to one cache layout ([ENG] "The
 * contract travels with the engine").
 */
typedef struct {
  int32_t num_pages;         /* physical pages in the pool, >= 1 */
  int32_t page_tokens;       /* must be 32 */
  int32_t num_kv_heads;      /* >= 1 */
  int32_t head_dim;          /* 64 or 128 */
  int32_t kv_dtype;          /* pkd_dtype of stored K and V */
  float k_scale;             /* fp8: stored code x k_scale = key value; must be 1 otherwise */
  float v_scale;             /* fp8: stored code x v_scale = value;     must be 1 otherwise */
  int32_t max_seqs;          /* sequences with a block table, >= 1 */
  int32_t max_pages_per_seq; /* block-table length, >= 1 */
  int32_t attn_chunk_pages;  /* split-sequence chunk, in pages, >= 1; a row whose context
                                spans more pages is reduced in chunks of this many pages
                                and the chunk results are merged in ascending order
                                ([LRS] section 4, lesson 2).  Fixed per pool, so the
                                split never depends on the batch. */
} pkd_pool_desc;

typedef struct pkd_pool pkd_pool; /* opaque host handle */

/*
 * Memory layout of the pool inside the caller's buffer (byte offsets are
 * reported by pkd_pool_info; every region starts 256-byte aligned):
 *
 *   pages    num_pages x num_kv_heads x 2 blocks; block (page p, kv head g,
 *            kind c, c = 0 for K and 1 for V) starts at
 *            ((p * num_kv_heads + g) * 2 + c) * block_bytes,
 *            block_bytes = 32 * head_dim * sizeof(kv element).
 *   table    int32 [max_seqs][max_pages_per_seq], physical page of each
 *            logical page, -1 where unset.
 *   counts   int32 [max_seqs], pages set for each sequence.
 *   error    uint32 sticky device error word (see pkd_pool_check).
 *
 * Inside a block the 32 x head_dim elements (token t = 0..31 = position mod
 * 32, dimension c) are stored as 16-byte vectors of E = 16 / sizeof(element)
 * elements (E = 4 for f32, 8 for bf16, 16 for fp8), d = head_dim:
 *
 *   K block:  vector ((t / 16) * (d / E) + c / E) * 16 + t % 16,
 *             element c % E.
 *   V block:  write t = 16a + 4b + i (a in 0..1, b in 0..3, i in 0..3):
 *     f32:    vector ((a * (d / 16) + c / 16) * 4 + b) * 16 + c % 16, element i
 *     bf16:   vector ((c / 16) * 4 + b) * 16 + c % 16,                element 4a + i
 *     fp8:    vector ((c / 32) * 4 + b) * 16 + c % 16,
 *             element 8 * ((c / 16) % 2) + 4a + i
 *
 * Both layouts let one 64-lane wavefront fetch a page with fully contiguous
 * 1 KiB loads that land in registers already in the operand order of the
 * gfx950 matrix-core instructions.  A caller that writes history itself (for
 * example a prefill) must follow this layout.
 */
typedef struct {
  size_t total_bytes;
  size_t pages_offset;
  size_t block_bytes;
  size_t table_offset;
  size_t counts_offset;
  size_t error_offset;
  int64_t shared_pages; /* host count: physical pages that two or more sequences' block
                           tables list (a shared prompt prefix).  While it is 0 the
                           attention kernels look for no shared pages to stage, which
                           leaves them more waves per compute unit; results are the
                           same either way. */
} pkd_pool_info;

/* Bytes kv_pool_create needs for `desc`, computed without allocating; 0 if
 * the descriptor is invalid. */
size_t pkd_pool_bytes(const pkd_pool_desc* desc);

/*
 * Lays a pool out in the caller's device buffer `dev_mem` of `bytes` bytes
 * (256-byte aligned): sets every block-table entry to -1, every count to 0
 * and the error word to 0 on `stream`, and synchronises `stream` before
 * returning, so that later calls on any stream see the laid-out pool.  Page
 * contents are left as they are.  The handle keeps a host copy of the block
 * tables (4 bytes per table entry).
 * Errors: PKD_ERR_INVALID_ARG, PKD_ERR_UNSUPPORTED (page_tokens != 32,
 * head_dim not 64/128, scales not 1 for a non-fp8 pool, non-finite or
 * non-positive fp8 scale), PKD_ERR_OUT_OF_MEMORY {needed, available} when
 * `bytes` is too small.  On success *out is a new handle.
 */
pkd_status kv_pool_create(const pkd_pool_desc* desc, void* dev_mem, size_t bytes,
                          pkd_stream stream, pkd_pool** out, pkd_error* err);

/* Frees the host handle only; the device buffer stays the caller's. */
pkd_status kv_pool_destroy(pkd_pool* pool);

pkd_status pkd_pool_info_get(const pkd_pool* pool, pkd_pool_info* info);

/*
 * Admission-time: sets the block tables of sequences first_seq ..
 * first_seq + n_seqs - 1.  pages_host is a host array [n_seqs][max_pages_per_seq]
 * (row i holds the physical pages of sequence first_seq + i in logical order;
 * entries at or past n_pages_host[i] are ignored) and n_pages_host[n_seqs]
 * the page counts.  The whole budget of a sequence (prompt plus answer) is
 * reserved here, up front, so the decode loop never runs out of pages
 * ([GIE] "Batching without running out of cache").  Several sequences may
 * name the same physical page (a shared prompt prefix, [LRS] section 5); the
 * caller must then not append into that page.
 * Errors (nothing is written): PKD_ERR_BOUNDS for a sequence range outside
 * [0, max_seqs) {needed = first_seq + n_seqs, available = max_seqs}, a count
 * above max_pages_per_seq {needed = count, available = max_pages_per_seq} or
 * a page id outside [0, num_pages) {needed = id, available = num_pages};
 * PKD_ERR_DUPLICATE_PAGE for a page listed twice in one sequence.
 * The tables it replaces are taken from the handle's host copy (which keeps
 * the per-page sequence counts behind pkd_pool_info.shared_pages); nothing is
 * read back from the device.  Synchronous: writes the new tables on `stream`
 * and returns after they have reached the device.
 */
pkd_status block_table_set(pkd_pool* pool, int32_t first_seq, int32_t n_seqs,
                           const int32_t* pages_host, const int32_t* n_pages_host,
                           pkd_stream stream, pkd_error* err);

/*
 * Reads and clears the sticky device error word (synchronises `stream`).
 * Returns PKD_ERR_ROW if, since the last check, some launched row had a
 * sequence outside [0, max_seqs), a negative position, a position at or
 * beyond 32 x (pages set for its sequence), or a block-table entry among its
 * pages outside [0, num_pages); such a row's outputs were written as zeros
 * and nothing was appended for it.  The kernels check every table entry and
 * page count they use (the device copies sit in caller memory at published
 * offsets): an entry outside the pool is never dereferenced, and a count is
 * taken as at most max_pages_per_seq.  err->needed holds the bits set
 * (1 = bad sequence, 2 = bad position, 4 = table entry outside the pool).
 */
pkd_status pkd_pool_check(pkd_pool* pool, pkd_stream stream, pkd_error* err);

/* ------------------------------------------------------------------------ */
/* Rows                                                                      */
/* ------------------------------------------------------------------------ */

/*
 * The rows of one step: row r is sequence seq[r] at position pos[r]; its
 * context is positions 0 .. pos[r] (length L = pos[r] + 1, the row's own
 * token included).  Decode rows of many sequences and several rows of one
 * sequence (a slice of a long prompt) may share one step ([GIE] "Batching
 * without running out of cache": every step is a set of rows carrying token,
 * sequence and position; [LRS] section 1: steps mix prefill and decode).
 * seq and pos are device arrays of n int32.
 * flags: 0, or PKD_ROWS_DISTINCT_SEQS when the caller guarantees that no
 * sequence has more than one row in the call (a pure decode batch).  Then the
 * append of each row's key and value runs inside the attention kernel instead
 * of a separate pass before it; results are bit-identical either way.  If the
 * guarantee is broken, a later row of a repeated sequence may miss an earlier
 * row's token (no memory is touched out of bounds).
 */
enum { PKD_ROWS_DISTINCT_SEQS = 1 };

typedef struct {
  const int32_t* seq;
  const int32_t* pos;
  int32_t n;
  int32_t flags;
} pkd_rows;

/* ------------------------------------------------------------------------ */
/* Paged attention decode                                                    */
/* ------------------------------------------------------------------------ */

/* Workspace bytes paged_attn_decode needs for up to max_rows rows. */
size_t pkd_attn_workspace_bytes(const pkd_pool* pool, int32_t n_q_heads, int32_t max_rows);

/*
 * Paged-attention decode ([H100] "Bug #1": online softmax in fp32 over K and V
 * pages staged on chip; [LRS] section 4, lesson 2: split-sequence chunks
 * merged afterwards; [GIE] "The same bits in any batch").
 *
 * q      device [n][n_q_heads][head_dim]; dtype f32 for an f32 pool, bf16
 *        otherwise.  n_q_heads = G x num_kv_heads with 1 <= G <= 16; query
 *        head h reads kv head h / G.
 * k_new, v_new  both NULL, or device [n][num_kv_heads][head_dim] in q's
 *        dtype: the key and value of each row's own token.  Every row's pair
 *        is first written at (seq, pos) -- converted to the pool dtype: bf16
 *        and f32 unchanged, fp8 = E4M3 round-to-nearest-even of value /
 *        scale (fp32 division), saturating at +-448, NaN kept -- and only
 *        then does any row read the pool, so rows of one sequence see each
 *        other's tokens.
 * out    device [n][n_q_heads][head_dim], out_dtype f32 or bf16:
 *        softmax_t(q . K_t / sqrt(head_dim)) applied to V over t = 0..pos.
 * ws     device workspace of at least pkd_attn_workspace_bytes(pool, n_q_heads, n).
 * Invalid rows: see pkd_pool_check.
 * Scheduling (results are bit-identical whichever applies): with a pool
 * whose attn_chunk_pages covers max_pages_per_seq, one wave per (row, kv
 * head); otherwise one wave per (row, page chunk, kv head) and an ordered
 * merge.  On such chunked pools, in calls of at least 128 rows without
 * PKD_ROWS_DISTINCT_SEQS, runs of consecutive rows of one sequence at
 * consecutive positions (a prompt slice, [LRS] section 4, "Prefill: tensor
 * cores, written by hand") are read as shared tiles: rows [t T, t T + T)
 * with T the largest power of two (at most 64) for which T x G <= 64, when
 * they are one such run.  A tile fetches each K/V page once, into LDS, for
 * all its rows and query heads.
 */
pkd_status paged_attn_decode(pkd_pool* pool, const pkd_rows* rows, int32_t n_q_heads,
                             const void* q, const void* k_new, const void* v_new,
                             void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                             pkd_stream stream, pkd_error* err);

/*
 * paged_attn_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, semantics, kernels and results (bit for bit)
 * as paged_attn_decode, without the workspace: the chunk records of chunked
 * pools go to a fixed scratch array of pkd_attn_noalloc_scratch_bytes()
 * (64 MiB) in device memory, which every GPU the library runs on holds from
 * the first such call until the process ends.  The call allocates nothing.
 * A call needing more than the scratch (pkd_attn_workspace_bytes of the same
 * arguments) is refused with PKD_ERR_OUT_OF_MEMORY {needed, available}
 * before anything is launched.  No part of the scratch has to start at zero:
 * every record a call reads is written by the same call.  Every call on one
 * GPU shares that GPU's scratch: calls that overlap on one GPU (other
 * streams, other threads) race and must not be made.
 */
size_t pkd_attn_noalloc_scratch_bytes(void);
pkd_status paged_attn_decode_noalloc(pkd_pool* pool, const pkd_rows* rows, int32_t n_q_heads,
                                     const void* q, const void* k_new, const void* v_new, void* out,
                                     int32_t out_dtype, pkd_stream stream, pkd_error* err);

/* ------------------------------------------------------------------------ */
/* Weight matrix-vector products                                             */
/* ------------------------------------------------------------------------ */

/*
 * A weight matrix, row-major [rows][cols]: output j of a product is
 * sum_k W[j][k] x[k] ([LRS] section 2: decode reads every weight once per
 * step; section 4: one wavefront per output row).
 */
typedef struct {
  const void* data;
  int32_t rows;     /* outputs */
  int32_t cols;     /* inputs, multiple of 64 */
  int32_t dtype;    /* pkd_dtype */
  float scale;      /* fp8: per-tensor scale (code x scale = weight); 1 otherwise */
  int32_t family;   /* pkd_family, fixed per matrix so a row's result never
                       depends on how many rows share the launch */
  int32_t k_splits; /* matrix-core families: 0 or 1 = one pass over K; S > 1 =
                       K cut into S fixed ranges whose fp32 partial sums are
                       added in ascending order (more workgroups for matrices
                       with few output tiles).  Fixed per matrix, like the
                       family, so results stay batch invariant. */
} pkd_matrix;

/*
 * Epilogue applied to each output element acc (fp32):
 *   silu_pair = 0:  y[r][j] = acc[r][j] (+ residual[r][j])
 *   silu_pair = 1:  W stacks [W_gate; W_up] (rows = 2F), and
 *                   y[r][j] = silu(acc[r][j]) * acc[r][F + j], j < F
 *                   ([LRS] section 3: gate and up projections fused with
 *                   their activation); residual must be NULL.
 * Before the silu / residual step, acc (already times the weight scale) is
 *   multiplied by row_scale[r] when row_scale is not NULL (device f32 [n]:
 *   the 1/rms factor of a norm whose gain is folded into W, "llm-rs"
 *   section 4, third lesson: norms folded into the projections), and
 *   rotated in consecutive pairs when rope_cs is not NULL: for columns
 *   j < rope_cols, pair (2i, 2i+1) of each head of rope_head_dim columns
 *   (i = (j mod rope_head_dim) / 2) becomes
 *     (a c - b s, a s + b c),  (c, s) = rope_cs[r][i]  (device f32
 *   [n][rope_head_dim / 2][2], e.g. from rope_table).  rope_head_dim must be
 *   a positive multiple of 4, rope_cols a multiple of it and at most the
 *   output count; rotation and silu_pair exclude each other.
 * out_dtype f32 or bf16.  residual: NULL or device f32 [n][rows].
 * y_bf16: NULL, or a second output that receives y rounded to bf16 (the
 * input of a following bf16 projection).
 */
typedef struct {
  int32_t out_dtype;
  const float* residual;
  int32_t silu_pair;
  void* y_bf16;
  const float* row_scale;
  const float* rope_cs;
  int32_t rope_cols;
  int32_t rope_head_dim;
} pkd_epilogue;

size_t pkd_gemv_workspace_bytes(const pkd_matrix* W, int32_t max_rows);

/*
 * A k_splits value for a matrix-core matrix of rows x cols that will mostly
 * see batches of about typical_rows rows: the S in {1, 2, 3, 4, 6, 8}, with
 * at least 512 columns per split, that minimises the estimated time at that
 * batch (rounds of workgroups over the compute units times the K-work of one
 * workgroup; a larger S must win by 5%).  The caller fixes
 * the result in the pkd_matrix once (results depend on S, never on the batch
 * it later runs).  Returns 1 for the GEMV family or invalid sizes.  Pure host
 * function: no device access.
 */
int32_t pkd_suggest_k_splits(int32_t rows, int32_t cols, int32_t family, int32_t typical_rows);

/*
 * y = epilogue(W x_r) for each of the n_rows rows of x (device [n_rows][cols]).
 *   GEMV family: x is f32 or bf16 and is used exactly; fp32 accumulation.
 *   GEMV_MFMA family: bf16 or fp8 weights, x must be bf16; fp32 accumulation.
 *   MFMA family, bf16 weights: x must be bf16; fp32 accumulation.
 *   MFMA and MFMA_FP8 families, fp8 weights: x (f32 or bf16) is quantised per
 *     row (s = max|x| / 448 in fp32, codes = E4M3 RNE of x / s, saturating),
 *     the contraction runs on the fp8 codes, and acc = s x W.scale x sum.
 *   Matrix-core families need rows % 128 == 0 and cols % 64 == 0 (% 128 for
 *   MFMA_FP8).
 * ws: device workspace of pkd_gemv_workspace_bytes(W, n_rows) bytes (0 for
 * every case except the fp8 MFMA family).
 */
pkd_status gemv_rows(const pkd_matrix* W, const void* x, int32_t x_dtype, int32_t n_rows,
                     void* y, const pkd_epilogue* ep, void* ws, size_t ws_bytes,
                     pkd_stream stream, pkd_error* err);

/*
 * Logits for a candidate list of weight rows only: the output head evaluated
 * for the tokens that may come next rather than for the whole vocabulary
 * ("GPU inference engine engineering", headline figure "Grammar-bounded
 * output" and section "The whole decode loop on the GPU").
 *
 * For each activation row r < n_rows of x (device [n_rows][W->cols], f32 or
 * bf16 per x_dtype) and each c < clamp(n_cand[r], 0, max_cand):
 *   j = cand[r * max_cand + c];
 *   y[r * max_cand + c] = W->scale * sum_k W[j][k] x[r][k]   (0 <= j < rows)
 *                       = NaN                                 (otherwise)
 * Entries y[r][c] at c >= that clamped count are not written.
 *   cand:   device int32 [n_rows][max_cand], weight-row indices; repeats allowed.
 *   n_cand: device int32 [n_rows], entries used per row.
 *   y:      device f32 [n_rows][max_cand].
 * W must be a GEMV or GEMV_MFMA family matrix.  Each y entry is
 * bit-identical to the same entry of gemv_rows(W, x) with an f32 output,
 * whatever the batch, list length or order (same K split, same summation
 * order), so the full head can serve as a cross-check of the gathered one.
 * Bytes read: sum_r clamp(n_cand[r]) rows of W plus x; no workspace.
 * Errors (host-side, before any launch): NULL/misaligned pointers
 * (x and y 16-byte, cand/n_cand 4-byte), max_cand < 1 when n_rows > 0 ->
 * PKD_ERR_INVALID_ARG; a matrix-core family or n_rows > 65535 ->
 * PKD_ERR_UNSUPPORTED.  Asynchronous on `stream`; the caller owns every
 * buffer.
 */
pkd_status gemv_gather_rows(const pkd_matrix* W, const void* x, int32_t x_dtype, int32_t n_rows,
                            const int32_t* cand, const int32_t* n_cand, int32_t max_cand, float* y,
                            pkd_stream stream, pkd_error* err);

/*
 * RMSNorm factor of each row, the part of a norm that remains at step time
 * once its gain is folded into the next projection's weight columns ("llm-rs",
 * section 4, third lesson: norms folded into the projections):
 *   inv_rms[r] = 1 / sqrt(sum_k x[r][k]^2 / cols + eps)
 * computed in fp32 in a fixed order (a row's value never depends on n_rows).
 * x: device f32 [n_rows][cols], cols a positive multiple of 4, 16-byte
 * aligned.  x_bf16: NULL, or device [n_rows][cols] bf16 that receives x
 * rounded to nearest even (16-byte aligned).  inv_rms: device f32 [n_rows].
 * Errors: bad sizes, eps < 0 or not finite, NULL or misaligned pointers ->
 * PKD_ERR_INVALID_ARG / PKD_ERR_UNSUPPORTED, before any launch.
 */
pkd_status rms_norm_factor(const float* x, int32_t n_rows, int32_t cols, float eps, float* inv_rms,
                           void* x_bf16, pkd_stream stream, pkd_error* err);

/*
 * Rotary-position table for the epilogue's rotation (the pages do not
 * describe positional encoding; this is the consecutive-pair form):
 *   cs[r][i] = (cos t, sin t),  t = pos[r] * base^(-2 i / head_dim),
 * for i < head_dim / 2, evaluated in fp64 and stored as f32.
 * pos: device int32 [n_rows]; cs: device f32 [n_rows][head_dim / 2][2].
 * head_dim even and >= 2, base finite and > 0, else PKD_ERR_INVALID_ARG.
 * Checkpoints that rotate the halves (i, i + head_dim / 2) instead can be used
 * by permuting the q and k rows of W_qkv within each head to pair order, which
 * leaves every q . k unchanged.
 */
pkd_status rope_table(const int32_t* pos, int32_t n_rows, int32_t head_dim, float base, float* cs,
                      pkd_stream stream, pkd_error* err);

/* ------------------------------------------------------------------------ */
/* One decode step of one transformer layer                                  */
/* ------------------------------------------------------------------------ */

/*
 * act_dtype is the dtype of q, k, v, the attention output, the FFN
 * activation and of every projection input: f32 (with f32 weights and pool)
 * or bf16.  The residual stream x, h, y is f32.
 */
typedef struct {
  int32_t hidden;     /* D */
  int32_t n_q_heads;  /* H_q */
  int32_t n_kv_heads; /* H_kv, equal to the pool's */
  int32_t head_dim;   /* d, equal to the pool's */
  int32_t ffn;        /* F; 0 = no FFN (y = h) */
  pkd_matrix w_qkv;   /* [(H_q + 2 H_kv) d][D], rows: q heads, then k heads, then v heads */
  pkd_matrix w_o;     /* [D][H_q d] */
  pkd_matrix w_gate_up; /* [2F][D] = [W_gate; W_up] */
  pkd_matrix w_down;  /* [D][F] */
  int32_t act_dtype;
  int32_t flags;      /* PKD_LAYER_NORM | PKD_LAYER_ROPE, or 0 */
  float norm_eps;     /* PKD_LAYER_NORM: the norms' epsilon (>= 0) */
  float rope_base;    /* PKD_LAYER_ROPE: the rotary base (> 0) */
} pkd_layer;

/* PKD_LAYER_NORM: RMSNorm before attention and before the FFN, with their
 * gains already folded into the columns of w_qkv and w_gate_up; the step
 * applies 1/rms(x) to the qkv outputs and 1/rms(h) to both gate/up halves
 * before the silu.  PKD_LAYER_ROPE: q and k heads rotated by the row's
 * position (rope_table's angles) before they are stored or attended. */
enum { PKD_LAYER_NORM = 1, PKD_LAYER_ROPE = 2 };

size_t pkd_step_workspace_bytes(const pkd_layer* layer, const pkd_pool* pool, int32_t max_rows);

/*
 * One decode step for the rows:
 *   qkv = W_qkv x ; append k, v at (seq, pos) ; attn = paged attention of q
 *   h   = x + W_o attn
 *   a   = silu(W_gate h) * (W_up h)          (when ffn > 0)
 *   y   = h + W_down a                       (y = h when ffn = 0)
 * x and y are device f32 [n][hidden].  Every projection input is taken in
 * act_dtype.  With PKD_LAYER_NORM / PKD_LAYER_ROPE (layer->flags):
 *   qkv = (W_qkv x) / rms(x), then q and k rotated by pos ; a = silu(W_gate h
 *   / rms(h)) * (W_up h / rms(h)), with the norm gains folded into W_qkv and
 *   W_gate_up by the caller.  Token embedding is not part of this step.
 */
pkd_status decode_step(const pkd_layer* layer, pkd_pool* pool, const pkd_rows* rows,
                       const float* x, float* y, void* ws, size_t ws_bytes,
                       pkd_stream stream, pkd_error* err);

/* ------------------------------------------------------------------------ */
const char* pkd_status_string(int32_t status);
const char* pkd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PKD_H */
