/*
 * gdn.h -- C ABI of libgdn, the Gated DeltaNet layer core for AMD MI355X
 * (gfx950).
 *
 * The library computes, for a batch of sequences, the four parts of a GDN
 * layer core named by the method statement of this project (Gated DeltaNet):
 *   (a) a width-W depthwise causal conv with SiLU over the q/k/v channels and
 *       the rolling conv window;
 *   (b) the post-conv gating: L2-normalised q and k, decay
 *       g = -exp(A_log) * softplus(a + dt_bias), update strength beta = sigmoid(b);
 *   (c) the gated delta rule per value head,
 *         S_t = e^{g_t} (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *         o_t = scale * S_t^T q_t,
 *       with S a d_k x d_v matrix, token by token or in the chunked WY/UT form;
 *   (d) speculative verify that replays the previous step's accepted
 *       candidate rows from a one-page record ("r9700-stack v0.2.4: one GDN
 *       state page per request", section "What it does").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer is a DEVICE pointer unless its comment says host.  The
 *   caller owns every buffer; libgdn never allocates, frees or synchronises,
 *   and keeps no state between calls.  Kernels run on `stream` (a hipStream_t;
 *   NULL is the default stream).
 * - Channel order of a pre-conv row is [q | k | v], head-major then dim:
 *   C_conv = 2*h_k*d_k + h_v*d_v.  Value head h reads key head h / (h_v/h_k).
 * - Activations (x, conv window, conv weights, a, b) use dims->act_dtype;
 *   states use dims->state_dtype; A_log, dt_bias and every output o are fp32.
 * - A state page holds h_v heads, each a row-major d_k x d_v matrix.
 * - Page indices < 0 mark padding rows: they are skipped and nothing of
 *   theirs is read or written.  Page indices used in one call must be
 *   distinct.  Sequences of length 0 are no-ops.
 * - Host-side argument errors return GDN_ERR_ARG before anything is
 *   launched.  Errors only the device can see (page index >= n_pages, a
 *   malformed cu_seqlens, an acceptance beyond the record, a replayed
 *   step) skip the affected sequence or request and OR a GDN_DEVERR_* bit
 *   into *err when err is not NULL.
 * - conv-window sync words: sequences whose workgroups share conv channels
 *   hand the rolled window to the last workgroup to finish reading it, which
 *   counts arrivals in gdn_conv_pool.sync.  One more word after the
 *   n_pages * h_k arrival counters is the work counter from which the
 *   short-sequence (decode) kernel of gdn_recurrent_seq hands out items.
 *   The words must be zero before the first call and every call leaves them
 *   zero when its kernels complete; a call aborted midway must be followed
 *   by re-zeroing them.
 * - Calls that touch the same pages must be ordered (same stream, or events).
 *   Calls that share a conv pool's sync words must be ordered too, even on
 *   disjoint pages: the decode kernel of gdn_recurrent_seq hands out its
 *   work from the one work counter after the arrival counters, so two such
 *   calls in flight at once would draw from the same counter.
 * - Every compute call can be captured in a HIP graph and replayed: its host
 *   arguments are shapes, strides, host bounds and device pointers; every
 *   value that changes from step to step (lengths, page indices, acceptance
 *   counts, parity) is read on the device; no call issues a memset, a copy or
 *   an allocation, and the sync words return to zero inside the kernels
 *   ("r9700-stack v0.2.4", "A defect found and fixed before the tag": a
 *   result must not depend on whether the step runs in a graph).  The first
 *   short-sequence (decode) call on a device queries its compute-unit count
 *   and the kernel's occupancy (host queries, cached per device); make that
 *   first call outside capture.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

/* status codes returned by every entry point */
#define GDN_OK 0
#define GDN_ERR_ARG 1          /* invalid argument (null pointer, bad dims/stride/size) */
#define GDN_ERR_UNSUPPORTED 2  /* valid but not compiled (head dim, width, dtype combination) */
#define GDN_ERR_LAUNCH 3       /* the HIP launch failed */

/* dtypes */
#define GDN_F32 0
#define GDN_BF16 1

/* speculative page layouts */
#define GDN_SPEC_ONEPAGE 0     /* one state checkpoint + a two-slot record per request */
#define GDN_SPEC_SLOTS 1       /* one state page per candidate (the comparison design) */

/* sticky device error bits OR-ed into *err */
#define GDN_DEVERR_PAGE 1u      /* page index >= n_pages */
#define GDN_DEVERR_BATCH 2u     /* cu_seqlens decreasing or beyond n_rows */
#define GDN_DEVERR_ACCEPTED 4u  /* num_accepted >= rows held by the live record */
#define GDN_DEVERR_PARITY 8u    /* step parity equals the live record's: step already applied */
#define GDN_DEVERR_CACHE 16u    /* prefix-cache entry out of range, or cached row beyond the replay */

typedef struct gdn_dims {
    int32_t h_k, h_v;      /* key heads, value heads; h_v % h_k == 0 */
    int32_t d_k, d_v;      /* head dims; d_k in {32, 64, 128}, d_v % 32 == 0 */
    int32_t conv_w;        /* conv width; 4 is compiled */
    int32_t n_spec;        /* drafts per verify step (candidates per step <= n_spec + 1) */
    int32_t act_dtype;     /* GDN_BF16 or GDN_F32 */
    int32_t state_dtype;   /* GDN_F32 or GDN_BF16 */
    float scale;           /* s in o = s * S^T q */
    float l2_eps;          /* eps in q / sqrt(sum q^2 + eps) */
} gdn_dims;

typedef struct gdn_params {
    const void* conv_w;    /* [C_conv][conv_w], act dtype; tap conv_w-1 meets the newest row */
    const float* a_log;    /* [h_v] */
    const float* dt_bias;  /* [h_v] */
} gdn_params;

/* Ragged batch of sequences packed row by row. */
typedef struct gdn_batch {
    const int32_t* cu_seqlens;  /* [n_seqs+1], cu[0] = 0, non-decreasing, cu[n_seqs] <= n_rows */
    const int32_t* page_idx;    /* [n_seqs], page in both pools; < 0 = padding */
    const uint8_t* has_init;    /* [n_seqs] or NULL (all 1): 0 = start from a zero window and state */
    int32_t n_seqs;
    int32_t max_seqlen;         /* host: upper bound of every length, or 0 if unknown */
    int64_t n_rows;             /* host: rows available in x, a, b and o */
} gdn_batch;

/* Conv windows: page p, row r (oldest first), channel c lives at
 * base + p*page_stride + r*C_conv + c (act dtype).  Rows 0..conv_w-2 hold the
 * window after a sequence call; verify uses rows 0..conv_w-2+n_spec. */
typedef struct gdn_conv_pool {
    void* base;
    int64_t page_stride;   /* elements, >= rows * C_conv */
    int32_t rows;          /* >= conv_w - 1 (verify: >= conv_w - 1 + n_spec) */
    int32_t n_pages;
    uint32_t* sync;        /* [n_pages][h_k] arrival counters + 1 work counter, zero between calls */
} gdn_conv_pool;

/* Recurrent states: page p, head h at base + p*page_stride + h*d_k*d_v
 * (state dtype), row-major d_k x d_v. */
typedef struct gdn_state_pool {
    void* base;
    int64_t page_stride;   /* elements, >= h_v * d_k * d_v */
    int32_t n_pages;
} gdn_state_pool;

/* Byte layout of one speculative page (see gdn_spec_page_layout). */
typedef struct gdn_spec_layout {
    size_t page_bytes;     /* minimum page size (a multiple of 256) */
    size_t header_off;     /* gdn_spec_header */
    size_t state_off;      /* one-page: checkpoint [h_v][d_k][d_v]; slots: [n_spec+1][h_v][d_k][d_v] */
    size_t record_off;     /* one-page only: record slot s, row i at record_off + (s*(n_spec+1)+i)*record_row_bytes */
    size_t record_row_bytes; /* fp32 [C_conv] post-conv q|k|v, then fp32 [h_v] a, then fp32 [h_v] b */
} gdn_spec_layout;

/* Header at the start of every speculative page.  An all-zero header is a
 * fresh page (live slot 0 holding no rows, parity 0): zero it after a
 * prefill or sequence call has written the page's state. */
typedef struct gdn_spec_header {
    uint32_t flag;         /* bit 0 live slot, bit 1 parity of the step that wrote it, bits 8..31 done counter */
    uint32_t n_rows[2];    /* candidate rows held by record slot 0 / 1 (slots layout: slots written) */
    uint32_t accepted;     /* echo of the acceptance the last step replayed */
    uint32_t reserved[60];
} gdn_spec_header;

/* ------------------------------------------------------------ queries */

/* GDN_ABI_VERSION of the loaded library. */
int32_t gdn_abi_version(void);

/* Static text for a status code (never NULL). */
const char* gdn_status_str(int32_t status);

/* Fill *out with the byte layout of a speculative page for `dims` and
 * `layout`.  Host-only.  Returns GDN_ERR_ARG on invalid dims or layout. */
int32_t gdn_spec_page_layout(const gdn_dims* dims, int32_t layout, gdn_spec_layout* out);

/* Workspace bytes gdn_chunked_prefill needs for this batch shape (host-only):
 * (n_seqs + ceil(n_rows / chunk)) chunk slots of h_k key-head records
 * (71 KB each at d = 128) and h_v value-head records (27.25 KB each): about
 * 1.96 MiB per slot at h_k = 16, h_v = 32. */
int32_t gdn_chunked_workspace_bytes(const gdn_dims* dims, int32_t n_seqs, int64_t n_rows,
                                    int32_t chunk, size_t* out_bytes);

/* ---------------------------------------------------- (a) conv update */

/* Causal depthwise conv over a ragged batch (Gated DeltaNet part (a)):
 *   z_t[c] = sum_{j<W} conv_w[c][j] * X_{t-W+1+j}[c],  y = SiLU(z) if activation
 * where rows before the first token come from the page's conv window (zeros if
 * has_init is 0).  Writes y [n_rows][y_stride] (y_dtype, GDN_F32 or GDN_BF16)
 * and rolls the window to the last W-1 rows of (window ++ x).  fp32
 * arithmetic: acc = 0, then one fused multiply-add per tap, oldest first.
 * x: [n_rows][x_stride] act dtype. */
int32_t gdn_conv_update(const gdn_dims* dims, const void* conv_w,
                        const void* x, int64_t x_stride,
                        const gdn_batch* batch, gdn_conv_pool conv,
                        int32_t activation, void* y, int32_t y_dtype, int64_t y_stride,
                        int32_t* err, void* stream);

/* ------------------------------------ (a)+(b)+(c) token-by-token core */

/* The layer core token by token, conv + gating + delta rule fused in one
 * launch (Gated DeltaNet parts (a)-(c); the token-by-token core of
 * "r9700-stack v0.2.3", section "1. Time to first token").  Each sequence
 * continues the state and window of its page (or zeros if has_init is 0);
 * its final state and rolled window are written back.  Decode is T = 1.
 *   x: [n_rows][x_stride] pre-conv rows; a, b: [n_rows][ab_stride] (first
 *   h_v entries used); o: [n_rows][h_v][d_v] fp32. */
int32_t gdn_recurrent_seq(const gdn_dims* dims, const gdn_params* params,
                          const void* x, int64_t x_stride,
                          const void* a, const void* b, int64_t ab_stride,
                          const gdn_batch* batch, gdn_conv_pool conv, gdn_state_pool state,
                          float* o, int32_t* err, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * gdn_recurrent_seq with its sync words kept in the library's own device
 * array of GDN_NOALLOC_SYNC_WORDS 32-bit words (256 KiB, held by every GPU
 * the library runs on until the process ends) instead of conv.sync, which
 * may be NULL here.  The call needs conv.n_pages * h_k + 1 words and
 * returns GDN_ERR_ARG beyond that maximum (at h_k = 16: up to 4,095 pages);
 * it zeroes the words it uses with a fill kernel on `stream` before the
 * layer kernel, so no word of an earlier call is read.  Nothing is
 * allocated, freed or copied.  Every call on one GPU shares the array:
 * calls that may overlap on one GPU (different streams, no ordering) race
 * on it and must be ordered.  Results are those of gdn_recurrent_seq, bit
 * for bit; every other argument, result and error is the same. */
#define GDN_NOALLOC_SYNC_WORDS 65536
int32_t gdn_recurrent_seq_noalloc(const gdn_dims* dims, const gdn_params* params,
                                  const void* x, int64_t x_stride,
                                  const void* a, const void* b, int64_t ab_stride,
                                  const gdn_batch* batch, gdn_conv_pool conv, gdn_state_pool state,
                                  float* o, int32_t* err, void* stream);

/* ------------------------------------------- (c) chunked WY/UT prefill */

/* The same result as gdn_recurrent_seq computed in the chunked WY/UT form
 * (Gated DeltaNet part (c)): per chunk of `chunk` rows, the UT transform
 * T = (I + A)^{-1} of A = tril(diag(beta) K K^T o e^{G_i-G_j}, -1), then
 * W = T diag(beta e^G) K, U = T diag(beta) V and the chunk-state update,
 * with bf16 matrix-core products accumulated in fp32.  chunk == 64 is
 * compiled.  Two launches on `stream`: the first writes every chunk's
 * state-independent operands (q and k rows and k^T, (T - I) diag(beta),
 * the masked decayed Q K^T, gates and norm factors) into the workspace, the
 * second runs each sequence's chunk-to-chunk state chain from them.
 * workspace: caller-owned device memory of at least
 * gdn_chunked_workspace_bytes bytes, 256-byte aligned, else GDN_ERR_ARG; its
 * contents on entry are ignored and on return are scratch.  Calls that share
 * one workspace must be ordered.  batch->max_seqlen, when > 0, must bound
 * every length: a longer sequence is skipped and raises GDN_DEVERR_BATCH.
 * x rows and conv-window rows are read, and o rows written, as 16-byte
 * vectors: x, conv.base and o must be 16-byte aligned and x_stride and
 * conv.page_stride multiples of 16 bytes' worth of elements (8 bf16 or 4
 * fp32), and x_stride and h_v * d_v at most 2^24 elements, else GDN_ERR_ARG. */
int32_t gdn_chunked_prefill(const gdn_dims* dims, const gdn_params* params,
                            const void* x, int64_t x_stride,
                            const void* a, const void* b, int64_t ab_stride,
                            const gdn_batch* batch, gdn_conv_pool conv, gdn_state_pool state,
                            float* o, int32_t chunk, void* workspace, size_t ws_bytes,
                            int32_t* err, void* stream);

/* ------------------------------------------- prefill path selection */

/* Which of the two sequence paths a prefill batch takes ("r9700-stack
 * v0.2.3", section "1. Time to first token": below a measured break-even
 * the layer core runs token by token, above it in the chunked form). */
#define GDN_PATH_TOKEN 0       /* gdn_recurrent_seq */
#define GDN_PATH_CHUNKED 1     /* gdn_chunked_prefill, chunk 64 */
#define GDN_PREFILL_MAX_DEFAULT (-1)

/* The path gdn_prefill takes for this batch shape (host-only, nothing is
 * launched).  Token by token while the longest sequence has at most
 * `token_max` rows, chunked above.  token_max < 0 takes the library's
 * default, the kernel-time break-even measured on MI355X over uniform
 * batches at d_k = d_v = 128: 32 rows for batches of 1-2 sequences, 16 rows
 * for 3-8, 8 rows for more (past that the chunked form is faster at every
 * length and batch size measured, 16 to 8192 rows and 1 to 32 sequences).  A large
 * token_max keeps every batch on the token-by-token path (relative error
 * 1e-4 against the exact recurrence, against 3e-3 for the bf16 matrix-core
 * chunked form); 0 sends every non-empty batch to the chunked path.  The
 * longest length is batch->max_seqlen, or batch->n_rows when that is 0.
 * Head dims the chunked path is not compiled for always take the token path.
 * *path (host) receives GDN_PATH_TOKEN or GDN_PATH_CHUNKED. */
int32_t gdn_prefill_path(const gdn_dims* dims, const gdn_batch* batch, int32_t token_max, int32_t* path);

/* Run the layer core over a prefill batch on the path gdn_prefill_path
 * selects; the result is that of gdn_recurrent_seq or gdn_chunked_prefill
 * (chunk 64) for the same arguments, bit for bit.  Arguments, layouts,
 * ownership and errors are those of the selected entry point (the chunked
 * path's 16-byte alignment rules apply only when it is selected); path
 * (host, may be NULL) receives the path taken. */
int32_t gdn_prefill(const gdn_dims* dims, const gdn_params* params,
                    const void* x, int64_t x_stride,
                    const void* a, const void* b, int64_t ab_stride,
                    const gdn_batch* batch, gdn_conv_pool conv, gdn_state_pool state,
                    float* o, int32_t token_max, void* workspace, size_t ws_bytes,
                    int32_t* path, int32_t* err, void* stream);

/* --------------------------------------------------- (d) spec verify */

/* One speculative verify step over n_req requests ("r9700-stack v0.2.4",
 * section "What it does").  Request r uses page req_page[r] of `pages`
 * (page_bytes apart, laid out per gdn_spec_page_layout) and of the conv pool
 * (rows >= conv_w - 1 + n_spec).  num_accepted[r] is how many drafts of the
 * previous step were accepted (1 + num_accepted[r] rows are committed); it is
 * ignored when the live record holds no rows.  step_parity[r] is 0 or 1 and
 * must differ from the parity stored in the page.
 * ONEPAGE: replay rows 0..num_accepted of the live record into the
 *   checkpoint, store it (rounded to the state dtype) and continue from the
 *   stored value; run the n_cand candidates, write their post-conv q|k|v
 *   and a/b into the other record slot; flip the live slot.
 * SLOTS: start from slot[num_accepted], store the state after candidate i
 *   into slot i.
 * Both designs give bit-identical o and committed states.  n_cand == 0 only
 *   commits (replays) and leaves an empty record.
 * Conv buffer: the window of the step is rows a'..a'+W-2 (a' = the replayed
 * acceptance, 0 for an empty record); afterwards rows are
 * [a'+1 .. a'+W-2, x of the n_cand candidates] (n_cand > 0) or
 * [a' .. a'+W-2] (n_cand == 0).
 *   x: [n_req][n_cand] rows of x_stride; a, b: [n_req][n_cand] rows of
 *   ab_stride; o: [n_req][n_cand][h_v][d_v] fp32. */
int32_t gdn_spec_verify(const gdn_dims* dims, const gdn_params* params, int32_t layout,
                        const void* x, int64_t x_stride,
                        const void* a, const void* b, int64_t ab_stride,
                        int32_t n_req, int32_t n_cand,
                        const int32_t* req_page, const int32_t* num_accepted,
                        const uint8_t* step_parity,
                        void* pages, int64_t page_bytes, int32_t n_pages,
                        gdn_conv_pool conv, float* o, int32_t* err, void* stream);

/* ----------------------------------------- prefix cache beside the record */

/* Cached committed prefixes of speculative requests.  The one-page design of
 * "r9700-stack v0.2.4" (section "What it does") is switched off there when
 * prefix caching is on; here a cache entry coexists with the record: entry e
 * holds a committed state at state.base + e*state.page_stride (state dtype,
 * [h_v][d_k][d_v]) and the conv window that ends with it in rows 0..W-2 of
 * conv page e (act dtype, oldest row first).  conv.sync is not used.
 * Entries written by one call must be distinct. */
typedef struct gdn_prefix_cache {
    const int32_t* entry;  /* [n_req] entry to write, < 0: none */
    const int32_t* row;    /* [n_req] the cached prefix ends at replayed record row `row`, 0..num_accepted */
    gdn_state_pool state;  /* n_pages = entries */
    gdn_conv_pool conv;    /* rows >= W-1, n_pages = entries */
} gdn_prefix_cache;

/* gdn_spec_verify, writing cached prefixes during the same step (no extra
 * launch).  For request r with cache->entry[r] >= 0: when the live record
 * holds rows, the committed stream grows by the replayed rows 0..a' and the
 * entry receives the prefix that ends at replayed row j = cache->row[r]
 * (0 <= j <= a'): the state after row j, rounded to the state dtype exactly
 * as a checkpoint is (j = a' gives the new checkpoint itself; the slot design
 * copies slot j, which holds the same bits), and conv buffer rows j..j+W-2.
 * When the live record holds no rows, the entry receives the checkpoint and
 * conv rows 0..W-2 as they are (row ignored).  An entry >= the cache's
 * entries or a row outside 0..a' refuses the request (GDN_DEVERR_CACHE):
 * nothing of it is written.  Every other argument, result and error is that
 * of gdn_spec_verify; cache == NULL is gdn_spec_verify. */
int32_t gdn_spec_verify_cached(const gdn_dims* dims, const gdn_params* params, int32_t layout,
                               const void* x, int64_t x_stride,
                               const void* a, const void* b, int64_t ab_stride,
                               int32_t n_req, int32_t n_cand,
                               const int32_t* req_page, const int32_t* num_accepted,
                               const uint8_t* step_parity,
                               void* pages, int64_t page_bytes, int32_t n_pages,
                               gdn_conv_pool conv, const gdn_prefix_cache* cache,
                               float* o, int32_t* err, void* stream);

/* Restore cached prefixes into pages: for request r with entry[r] >= 0 and
 * req_page[r] >= 0, the page's state region (the one-page checkpoint, or
 * slot 0 of the slot design) receives entry[r]'s state, its conv rows
 * 0..W-2 the entry's window, and its header is zeroed: the page is fresh, so
 * its next verify step replays nothing and starts from the restored state.
 * cache->entry and cache->row are not read (entry is the argument).  An
 * entry or page out of range skips the request (GDN_DEVERR_CACHE,
 * GDN_DEVERR_PAGE).  Pages of one call must be distinct. */
int32_t gdn_prefix_restore(const gdn_dims* dims, int32_t layout, int32_t n_req,
                           const int32_t* entry, const int32_t* req_page,
                           const gdn_prefix_cache* cache,
                           void* pages, int64_t page_bytes, int32_t n_pages,
                           gdn_conv_pool conv, int32_t* err, void* stream);

/* ------------------------------------------------------- mixed step */

/* The token-by-token part of a mixed step: the arguments of
 * gdn_recurrent_seq (batch is a host pointer), and optionally the
 * speculative pages the sequences go on to verify from.  With spec_pages
 * set, each sequence also leaves the header of its page (page_idx) fresh:
 * all zero, no record rows.  Alias the state pool onto the pages'
 * checkpoints (state.base = spec_pages + state_off, state.page_stride =
 * spec_page_bytes / state element size; gdn_spec_page_layout) and give the
 * sequences a conv pool wide enough for verify: the step then leaves a
 * prefilled request ready for its first verify step, the prefill's state in
 * the checkpoint and its window in conv rows 0..W-2, with nothing copied. */
typedef struct gdn_seq_part {
    const void* x;
    int64_t x_stride;
    const void* a;
    const void* b;
    int64_t ab_stride;
    const gdn_batch* batch;
    gdn_conv_pool conv;
    gdn_state_pool state;
    float* o;
    void* spec_pages;          /* or NULL; 256-byte aligned */
    int64_t spec_page_bytes;   /* multiple of 256 */
    int32_t spec_n_pages;      /* a page index >= spec_n_pages is a device error (GDN_DEVERR_PAGE) */
} gdn_seq_part;

/* The verify part of a mixed step: the arguments of gdn_spec_verify. */
typedef struct gdn_verify_part {
    int32_t layout;
    const void* x;
    int64_t x_stride;
    const void* a;
    const void* b;
    int64_t ab_stride;
    int32_t n_req;
    int32_t n_cand;
    const int32_t* req_page;
    const int32_t* num_accepted;
    const uint8_t* step_parity;
    void* pages;
    int64_t page_bytes;
    int32_t n_pages;
    gdn_conv_pool conv;
    float* o;
} gdn_verify_part;

/* One serving step that mixes token-by-token sequences (prefill or decode
 * rows of a ragged batch) with speculative verify requests
 * ("r9700-stack v0.2.3", section "1. Time to first token": the prefill
 * and verify kernels read their rows where the batch holds them, so such a
 * step gathers nothing first).  The result is that of
 * gdn_recurrent_seq on `seq` followed by gdn_spec_verify on `verify`, bit
 * for bit.  It runs as one launch -- the sequence workgroups first in the
 * grid (longest sequence first), the verify workgroups filling the slots
 * shorter sequences free -- or, for the shapes gdn_mixed_launches names, as
 * those two calls' kernels in stream order.
 * seq and verify are host pointers; either may be NULL or empty (n_seqs or
 * n_req 0).  The two parts must touch distinct pages; their conv pools may
 * be one pool.  Each part is validated as its stand-alone entry point is;
 * err collects the device-side errors of both. */
int32_t gdn_mixed_step(const gdn_dims* dims, const gdn_params* params, const gdn_seq_part* seq,
                       const gdn_verify_part* verify, int32_t* err, void* stream);

#define GDN_MIXED_AUTO 0           /* what gdn_mixed_launches picks */
#define GDN_MIXED_ONE_LAUNCH 1     /* one grid: sequence workgroups, then verify workgroups */
#define GDN_MIXED_TWO_LAUNCHES 2   /* gdn_recurrent_seq's kernel, then gdn_spec_verify's, in stream order */

/* The launch count gdn_mixed_step uses for these parts (host-only, nothing
 * is launched).  *launches (host) receives GDN_MIXED_TWO_LAUNCHES when both
 * parts are non-empty, every sequence has at most 4 rows
 * (1 <= batch->max_seqlen <= 4), no spec_pages are set and d_v is a multiple
 * of 64: gdn_recurrent_seq then runs the sequences on its short-sequence
 * (decode) kernel, whose streaming workgroups beat the one grid's 32-column
 * sequence workgroups by 5-48% on MI355X (uniform batches of 4-32
 * sequences beside 8 or 32 verify requests).  Otherwise
 * GDN_MIXED_ONE_LAUNCH: for longer sequences the one grid measured as fast
 * as two launches or faster (up to 28% with one long sequence among short
 * ones).  seq and verify may be NULL. */
int32_t gdn_mixed_launches(const gdn_dims* dims, const gdn_seq_part* seq, const gdn_verify_part* verify,
                           int32_t* launches);

/* gdn_mixed_step with the launch count given: GDN_MIXED_AUTO,
 * GDN_MIXED_ONE_LAUNCH or GDN_MIXED_TWO_LAUNCHES (anything else is
 * GDN_ERR_ARG).  Every choice gives the same results bit for bit; with two
 * launches the sequences take gdn_recurrent_seq's kernel for their shape
 * (its 32-column kernel when spec_pages are set, which the short-sequence
 * kernel does not write), so the first such call on a device makes the
 * host queries described for gdn_recurrent_seq. */
int32_t gdn_mixed_step_launches(const gdn_dims* dims, const gdn_params* params, const gdn_seq_part* seq,
                                const gdn_verify_part* verify, int32_t launches, int32_t* err, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
