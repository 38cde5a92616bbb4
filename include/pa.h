/*
 * pa.h -- C ABI of the paged K/V split-K decode attention library for
 * MI355X (gfx950), libpa_walk.so.
 *
 * The method (Luce-Org/lucebox pull 555, "feat(qwen35): add paged-attention
 * monolithic decode-only AR foundation", Summary): decode attention with head
 * size 256 and grouped queries -- 24 query heads over 4 KV heads, so one KV
 * head serves 6 query heads -- for 1 to 4 new query tokens per sequence
 * (and, as achyudh/llama.cpp pull 2 extends its decode kernel to verify
 * batches of up to 8 query tokens, for 5 to 8 as well; pa_prefill takes
 * more), with K and V stored as F16, BF16, Q8_0 or Q4_0 rows in fixed-size pages that a
 * per-sequence block table scatters through one pool.  Each sequence's
 * context is split into chunks; every chunk produces a normalised partial
 * output and its log-sum-exp, and a stable merge combines them.
 *
 * Conventions for every call:
 *  - the return value is a pa_status: PA_OK (0) or a negative error code;
 *    no C++ exception crosses the ABI;
 *  - errors the host can detect are returned before anything is enqueued,
 *    so a failed call has no effect on the device or on the pool
 *    (lucebox pull 555, Scope: unsupported combinations fail explicitly);
 *  - device work is enqueued on the given HIP stream and the call returns
 *    without waiting for it, unless the description says otherwise;
 *  - pointers documented as "device" must point to device memory of the
 *    pool's / stream's device; "host" pointers are read before the call
 *    returns and may be reused afterwards;
 *  - a pa_pool is safe to use from several host threads (one mutex per
 *    pool); device work on different streams is ordered only as stated.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */

typedef int32_t pa_status;

#define PA_OK               0
#define PA_ERR_INVALID     (-1) /* an argument is out of range or inconsistent   */
#define PA_ERR_NOMEM       (-2) /* not enough free pool blocks / device memory     */
#define PA_ERR_STALE       (-3) /* a handle is stale, already free or repeated     */
#define PA_ERR_UNSUPPORTED (-4) /* a type, page size or shape the library lacks    */
#define PA_ERR_HIP         (-5) /* a HIP runtime call failed                       */
#define PA_ERR_NOT_FOUND   (-6) /* a K/V pointer is not the base of a live pool    */

/* Static text for a status code. */
const char *pa_status_string(pa_status s);

/* Library version, "major.minor.patch".  The minor number changes when a
 * struct of this header grows or calls are added: 0.2 added
 * pa_decode_ext.seq_lens_host, pa_split_plan and pa_read_bandwidth_probe;
 * 0.3 added pa_split_workgroups_per_cu, pa_read_bandwidth_probe_ex and
 * pa_decode_scratch and attaches pa_decode_ext.split_events to the split
 * kernel's dispatch. */
#define PA_VERSION_STRING "0.3.0"
const char *pa_version(void);

/* ------------------------------------------------------------------ types */

/* K/V row encodings.  A row is one KV head's 256 values at one position.
 *  PA_F16 / PA_BF16: 256 little-endian 2-byte values, 512 bytes
 *    (F16: lucebox pull 555, Summary; bf16 K/V: ashhart/TensorFold issue 1156,
 *    "CUDA: Qwen3.5/3.6 attention caches on the core KV pool", Summary).
 *  PA_Q8_0: 8 blocks of 34 bytes: fp16 scale d, then 32 int8 codes c;
 *    value = c*d (block size: achyudh/llama.cpp pull 2, "hip: add RDNA2 gfx1030
 *    paged attention fallback for adaptive KV streaming", commit on the LDS
 *    reads of K/V dequantization).  272 bytes.
 *  PA_Q4_0: 8 blocks of 18 bytes: fp16 scale d, then 16 bytes whose byte j
 *    holds code c_j in its low nibble and c_{j+16} in its high nibble;
 *    value = (c-8)*d (size: lucebox pull 555, K/V capacity table; scale
 *    position: llama.cpp pull 2, same commit).  144 bytes.
 * A kv_type argument packs the K encoding in bits 0-7 and the V encoding in
 * bits 8-15; a V field of 0 means "same as K".  Every pair is decoded: K and
 * V pools may hold different encodings (lucebox pull 555, Validation: all
 * nine F16/Q8_0/Q4_0 K x V combinations; llama.cpp pull 2 defaults to Q8_0
 * K with Q4_0 V). */
enum { PA_F16 = 1, PA_BF16 = 2, PA_Q8_0 = 3, PA_Q4_0 = 4 };

/* float32 values: a source type of pa_append_kv_device, not a pool encoding. */
#define PA_F32 5
#define PA_KV_TYPE(k, v) ((int32_t)((k) | ((v) << 8)))

#define PA_HEAD_DIM   256
#define PA_N_Q_HEADS  24
#define PA_N_KV_HEADS 4
#define PA_MAX_QTOK   8
#define PA_MAX_PREFILL_TOKENS 65536

/* Bytes of one row of encoding t (0 for an unknown t). */
size_t pa_row_bytes(int32_t t);

/* -------------------------------------------------------------- the pool */

/* Pool layout in device memory (K and V pools alike, each with its own row
 * size): [n_blocks][4 KV heads][page_size][row_bytes] -- inside a page, one
 * KV head's rows are contiguous.  A block-table entry is a page index.
 * The layout inside a page is this library's choice; the pages say only that
 * K and V are pools of fixed-size pages (llama.cpp pull 2, page-table commit). */
typedef struct pa_pool pa_pool;

/* A block handle: (generation << 32) | page index. */
typedef uint64_t pa_block;

#define PA_POOL_HOST_ONLY 1u /* allocator only: no device memory, no decode */

typedef struct pa_pool_desc {
    int32_t  n_blocks;           /* pages in the pool, >= 1                                  */
    int32_t  page_size;          /* positions per page: a multiple of 16 in [16, 512]        */
    int32_t  n_kv_heads;         /* must be 4                                                */
    int32_t  head_dim;           /* must be 256                                              */
    int32_t  kv_type;            /* PA_KV_TYPE(k, v)                                         */
    int32_t  device;             /* HIP device ordinal of the pool                           */
    int32_t  max_seqs;           /* n_seq bound for pa_decode without a caller workspace;
                                    0 => 512                                                 */
    int32_t  max_blocks_per_seq; /* block-table row length pa_decode assumes when it is
                                    given no pa_decode_ext; 0 => n_blocks                    */
    int32_t  max_append_rows;    /* rows per staging batch of pa_append_kv; 0 => 1024       */
    uint32_t flags;              /* PA_POOL_HOST_ONLY or 0                                   */
    void    *k_pool;             /* device memory of the K pool, or NULL: the library
                                    allocates it (and frees it in pa_pool_destroy).  A
                                    caller-given pool stays caller-owned, must be 16-byte
                                    aligned and hold n_blocks pages                          */
    void    *v_pool;             /* likewise for V                                           */
} pa_pool_desc;

typedef struct pa_pool_info {
    void    *k_pool, *v_pool;       /* device base pointers (NULL for a host-only pool)       */
    void    *workspace;             /* the pool's own decode workspace (device), or NULL       */
    size_t   workspace_bytes;
    size_t   k_row_bytes, v_row_bytes;
    size_t   k_page_bytes, v_page_bytes; /* bytes of one page, all 4 KV heads               */
    int32_t  n_blocks, n_free, page_size, kv_type, max_blocks_per_seq, max_seqs, device;
} pa_pool_info;

/* Creates a pool and its block allocator; all blocks start free.  With NULL
 * k_pool / v_pool the library allocates them (hipMalloc, not zeroed).  Unless
 * the pool is host-only it also allocates a decode workspace sized for
 * max_seqs sequences of up to 8 query tokens, pinned and device staging for
 * pa_append_kv, and registers k_pool so that pa_decode can find the pool from
 * the pointer.  Errors: PA_ERR_INVALID (null out/desc, n_blocks < 1, bad
 * head count / head_dim, a K/V pointer already registered), PA_ERR_UNSUPPORTED
 * (page size, kv_type), PA_ERR_HIP / PA_ERR_NOMEM (device allocation); on
 * error nothing is allocated and *out is untouched. */
pa_status pa_pool_create(const pa_pool_desc *desc, pa_pool **out);

/* Waits for the pool's staging copies, frees what the library allocated and
 * unregisters the pool.  Caller-owned K/V memory is not freed.  NULL is a
 * no-op.  The caller must not destroy a pool that enqueued decode work still
 * reads. */
pa_status pa_pool_destroy(pa_pool *pool);

pa_status pa_pool_get_info(const pa_pool *pool, pa_pool_info *info);

/* Exact transactional allocation (lucebox pull 555, Summary: exact fixed-block
 * allocator, transactional allocation).  Allocates n blocks, all or none,
 * always the n lowest free page indices in increasing order (pages come from
 * the bottom of the pool, as TensorFold issue 1156, Design / Host, takes K/V
 * pages).  handles[i] (host, may be NULL) receives the handle and indices[i]
 * (host, may be NULL) the page index to put in block tables.  n == 0 is a
 * no-op.  Errors: PA_ERR_INVALID (n < 0, n > 0 with both outputs NULL),
 * PA_ERR_NOMEM (fewer than n free; nothing changes).  Host only. */
pa_status pa_alloc_blocks(pa_pool *pool, int32_t n, pa_block *handles, int32_t *indices);

/* Frees n blocks, all or none (lucebox pull 555, Summary: stale-handle
 * detection, immediate release).  Every handle is checked before anything is
 * released: a page index out of range gives PA_ERR_INVALID; a generation that
 * is not the page's current one, a page that is not allocated, or the same
 * page twice in the call gives PA_ERR_STALE; either way nothing is freed.
 * On success each page's generation advances (so every earlier handle of it
 * turns stale) and the pages are free at once in host bookkeeping.  Release
 * is not ordered with device work: blocks that work enqueued on a stream
 * still reads may be reallocated and then rewritten by pa_append_kv on the
 * same stream safely (stream order), but not from another stream until that
 * work has finished (ashhart/TensorFold issue 1156, Activity, returns pages
 * only once the stream has drained).  Host only. */
pa_status pa_free_blocks(pa_pool *pool, int32_t n, const pa_block *handles);

/* Writes n_rows new K/V rows into pages (JustVugg/colibri pull 372, "cuda: keep
 * paged ragged KV resident across decode steps", Summary: only the newly
 * appended rows are uploaded, in one packed transfer, and a scatter kernel
 * puts them in place).  Row i goes to page dst_block[i], slot dst_slot[i], for
 * all 4 KV heads.  k_rows / v_rows (host) are [n_rows][4][row_bytes], already
 * encoded in the pool's K / V encodings.  dst_block / dst_slot are host
 * arrays.  The call copies indices and rows into pinned staging and enqueues
 * one host-to-device copy per staging batch (max_append_rows rows) on the
 * pool's own copy stream, so that the transfer overlaps work already on
 * `stream`.  It then makes `stream` wait for the copy, enqueues one scatter
 * kernel per batch on `stream`, and returns.  The host waits only when a
 * staging slot is still in use by an earlier batch.  It is not for graph
 * capture: host copies and waits happen in the call.  A caller appending
 * position L of a sequence passes the page holding L and slot L % page_size:
 * the new row's position is the committed length (lucebox pull 555, Summary,
 * first-token bookkeeping fix).  Two rows with the same destination leave
 * the later one.  Errors: PA_ERR_INVALID (n_rows < 0, null arrays with
 * n_rows > 0, a page index outside the pool or not allocated, a slot outside
 * [0, page_size)), PA_ERR_HIP; nothing is enqueued on error. */
pa_status pa_append_kv(pa_pool *pool, int32_t n_rows, const int32_t *dst_block,
                       const int32_t *dst_slot, const void *k_rows, const void *v_rows,
                       hipStream_t stream);

/* Device-side append with fused encoding (colibri pull 372, Summary: only
 * the new rows move and a scatter kernel places them; here they are already
 * on the device, as a K/V projection leaves them, and the kernel encodes
 * them on the way, with no host staging and no separate pass over HBM).
 *
 * k_src, v_src  device [n_rows][4][256] values of src_type: PA_F32, PA_BF16
 *               or PA_F16 (16-byte aligned).  They are encoded into the
 *               pool's K and V encodings:
 *                 F16 / BF16: the nearest value, ties to even;
 *                 Q8_0 / Q4_0, per block of 32 (the Q8_0 and Q4_0 workload
 *                 definitions: scale max|x|/127 resp. max|x|/8): the scale is
 *                 max|x|/127 (/8) computed in float32 and stored as the
 *                 nearest fp16; codes are round(x * r), r = 1/scale as
 *                 stored, in float32, halves away from zero, Q8_0 clipped to
 *                 [-127, 127], Q4_0 stored as code + 8 clipped to [0, 15] (a
 *                 block's positive extreme, 8 steps, is stored as 7); a block
 *                 of zeros stores scale 0.  Values must be finite.
 * dst_block,
 * dst_slot      device int32 [n_rows]: row i goes to page dst_block[i], slot
 *               dst_slot[i], for all 4 KV heads (the page holding position L
 *               and slot L % page_size for a sequence of committed length L).
 *               A destination outside [0, n_blocks) x [0, page_size) is
 *               skipped and PA_DEVERR_APPEND is ORed into the error word;
 *               whether a page is allocated is not known on the device and
 *               is the caller's to ensure.  Two rows with the same
 *               destination leave unspecified bytes there.
 * err_word      device int32, or NULL for the error word of the pool's own
 *               workspace (read with pa_get_device_error(pool, NULL, ...)).
 * stream        one kernel is enqueued; nothing is staged on the host.
 * Errors: PA_ERR_INVALID (null pool or arrays with n_rows > 0, n_rows < 0,
 * another src_type, misalignment, a host-only pool), PA_ERR_HIP. */
pa_status pa_append_kv_device(pa_pool *pool, int32_t n_rows, const int32_t *dst_block,
                              const int32_t *dst_slot, const void *k_src, const void *v_src,
                              int32_t src_type, int32_t *err_word, hipStream_t stream);

/* ------------------------------------------------------------------ decode */

/* pa_decode_ext.flags: run the fp32 vector-ALU path instead of the matrix-core
 * path (same plan and merge; a second implementation for cross-checks). */
#define PA_DECODE_VECTOR_REFERENCE 1u

/* Device-side error bits, ORed into the workspace's error word. */
#define PA_DEVERR_TABLE  1 /* a block-table entry outside [0, n_pool_blocks)         */
#define PA_DEVERR_LENGTH 2 /* a seq_len < 0, or beyond the table row / contiguous rows */
#define PA_DEVERR_APPEND 4 /* pa_append_kv_device: a destination outside the pool     */

typedef struct pa_decode_ext {
    int32_t  bt_stride;      /* int32 entries per block-table row; in contiguous mode the
                                rows per sequence are bt_stride * page_size              */
    int32_t  n_pool_blocks;  /* pages in the pool (bounds for table entries)            */
    float    scale;          /* softmax scale; 0 => 1/sqrt(256) = 1/16                   */
    uint32_t flags;          /* 0, or PA_DECODE_VECTOR_REFERENCE                         */
    float   *lse_out;        /* optional device [n_seq][n_qtok][24] float: natural-log
                                log-sum-exp of each row's scaled, masked logits; -inf
                                for a row with no visible key                           */
    void    *workspace;      /* device scratch of at least pa_decode_workspace_size()
                                bytes, 256-byte aligned, or NULL for the pool's own
                                workspace.  Its first 4 bytes are the device error
                                word: zero them before the first use (e.g. hipMemset) */
    size_t   workspace_bytes;
    void    *split_events[2];/* optional hipEvent_t pair (created with timing) attached
                                to the split kernel's dispatch on `stream`: [0] records
                                when it starts executing, [1] when it has completed, so
                                hipEventElapsedTime gives the kernel's run time
                                (profiling).  Either may be NULL.                       */
    const int32_t *seq_lens_host; /* optional HOST copy of seq_lens ([n_seq] int32), or
                                NULL.  With it (and n_seq <= PA_HOST_PLAN_MAX_SEQS) the
                                split-K plan -- chunk length and each sequence's first
                                work item -- is computed on the host, with the same
                                integer arithmetic as the device plan, and travels with
                                the launch: the kernels then never read the device
                                seq_lens, and the caller guarantees that it holds the
                                same values.  Results are bitwise identical to the
                                device-planned call.  Larger batches ignore it.        */
} pa_decode_ext;

/* Largest batch whose plan pa_decode_ext.seq_lens_host can carry. */
#define PA_HOST_PLAN_MAX_SEQS 256

/* The split-K partition of a one-token decode call (occupancy-aware,
 * ragged-length-aware context parallelism: lucebox pull 555, Summary;
 * achyudh/llama.cpp pull 2, split-K decode commit), computed on the host with
 * the same integer arithmetic pa_decode uses; for inspection and tests, no
 * device needed.
 *
 * seq_lens_host  host int32 [n_seq] (0 <= n_seq <= PA_HOST_PLAN_MAX_SEQS);
 *                a length < 0 or > cap counts as one empty chunk.
 * cap            rows per sequence (bt_stride * page_size).
 * n_cu, wgs_per_cu  compute units and resident split workgroups per compute
 *                unit (pa_decode takes both from the device; the second is what
 *                pa_split_workgroups_per_cu reports: 256 and 2 for a one-token
 *                Q4_0 call on MI355X).
 * Writes *chunk (positions per chunk, a multiple of 128), *n_items (work
 * items = chunks x 4 KV heads) and, if first != NULL, first[s] = index of
 * sequence s's first chunk for s = 0..n_seq (first[n_seq] = all chunks).
 * Errors: PA_ERR_INVALID (null chunk / n_items, or seq_lens_host with
 * n_seq > 0; n_seq, cap, n_cu or wgs_per_cu out of range); nothing is
 * written then. */
pa_status pa_split_plan(const int32_t *seq_lens_host, int32_t n_seq, int32_t cap, int32_t n_cu,
                        int32_t wgs_per_cu, int32_t *chunk, int32_t *n_items, int32_t *first);

/* Resident split workgroups per compute unit that pa_decode / pa_prefill
 * plan with for `kv_type`, `n_qtok` query tokens (1..PA_MAX_QTOK) and `flags`
 * (pa_decode_ext.flags) on the current device: the runtime's occupancy query
 * for the kernel the call launches.  On the matrix-core path a decode call
 * of 6..8 tokens runs as two token groups of at most four and a prefill in
 * groups of four (pass 4 for it); the vector path runs a decode whole and a
 * prefill in groups of eight.  Pass it
 * to pa_split_plan to reproduce a call's partition.
 * Errors: PA_ERR_INVALID (null wgs, a bad kv_type, n_qtok or flags);
 * PA_ERR_HIP (no usable device). */
pa_status pa_split_workgroups_per_cu(int32_t kv_type, int32_t n_qtok, uint32_t flags, int32_t *wgs);

/* One decode step (lucebox pull 555, Summary; achyudh/llama.cpp pull 2,
 * split-K decode and page-table commits).
 *
 * q        device float [n_seq][n_qtok][24][256]: the new tokens' queries.
 * k_pool,
 * v_pool   device pools of the layout above, or, when block_table is NULL,
 *          contiguous storage [n_seq][4][bt_stride*page_size][row_bytes]
 *          (the no-table case of one row-address helper: ashhart/TensorFold
 *          issue 1156, Design / Kernels).
 * block_table device int32 [n_seq][bt_stride]; entry p of row s is the pool
 *          page of the sequence's positions [p*page_size, (p+1)*page_size).
 *          Entries past ceil(seq_len/page_size) are never read.
 * seq_lens device int32 [n_seq]: stored rows of each sequence, including the
 *          n_qtok new tokens.  New token t sits at position
 *          seq_len - n_qtok + t and attends to positions 0..seq_len-n_qtok+t.
 * n_seq    >= 0 (0 is a no-op).   n_qtok  1..8 (PA_MAX_QTOK).
 * kv_type  PA_KV_TYPE(k, v), matching the pool.   page_size: as the pool.
 * out      device float [n_seq][n_qtok][24][256]; query head h reads KV head
 *          h / 6.  A row with no visible key is 0.  All rows of a sequence
 *          whose length or table entries are out of range are NaN and the
 *          workspace error word gets PA_DEVERR_* bits; nothing outside the
 *          pool or table row is ever read (lucebox pull 555, Validation:
 *          corrupt block-table bounds guards).
 * stream   HIP stream for the kernels.
 * ext      NULL: k_pool must be the K base of a live pool (pa_pool_create);
 *          bt_stride is its max_blocks_per_seq, the scale 1/16, the pool's
 *          own workspace is used (so calls sharing a pool must not overlap on
 *          different streams) and n_seq must not exceed its max_seqs.
 *          Non-NULL: every field as documented; k_pool need not be a pool.
 *
 * Two kernels run: a split kernel over (sequence, KV head, context chunk)
 * work items, whose count and chunk sizes depend only on seq_lens, n_qtok and
 * the device's compute-unit count (so paged and contiguous storage give
 * bitwise-equal outputs), and a merge kernel for sequences split in several
 * chunks.  A call enqueues only these kernel launches on `stream` (no
 * allocation, copy or memset), so it may be captured in a HIP graph.  With
 * seq_lens_host the plan is fixed at capture and a replay must see the same
 * lengths; without it the kernels read seq_lens when they run, so one
 * capture serves every step of the same n_seq whose lengths fit the table.
 * Calls with separate workspaces may run on several streams at once.  Errors: PA_ERR_INVALID (null pointers, n_qtok outside 1..8,
 * misaligned K/V (16 bytes) or q/out (16 bytes), workspace too small,
 * page_size or kv_type different from the pool's), PA_ERR_UNSUPPORTED (a
 * split or merge grid past 2^32 - 1 work items), PA_ERR_NOT_FOUND (ext NULL
 * and k_pool not a pool), PA_ERR_HIP.
 * Numeric range of the matrix-core path (the default): products take f16
 * operands (bf16 for BF16 K or V), split into hi + lo parts.  Two limits
 * follow.  (1) Each dequantised Q8_0 / Q4_0 V value |code x d| must be at
 * most 65504, the f16 range: Q8_0 scales up to 515 and Q4_0 scales up to
 * 8188 always are, and rows encoded from data within the f16 range (scale
 * max|x| / 127 or / 8) never exceed it.  (2) For F16 / Q8_0 / Q4_0 K, each
 * |q x scale x log2(e)| must be at most 65504.  Past either limit the query
 * rows that see such a value come out non-finite; other rows are
 * unaffected.  The vector path (PA_DECODE_VECTOR_REFERENCE, fp32 throughout)
 * has neither limit. */
pa_status pa_decode(const float *q, const void *k_pool, const void *v_pool,
                    const int32_t *block_table, const int32_t *seq_lens,
                    int32_t n_seq, int32_t n_qtok, int32_t kv_type, int32_t page_size,
                    float *out, hipStream_t stream, const pa_decode_ext *ext);

/* pa_decode for callers that cannot allocate device memory or pass a
 * workspace (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same call, with the chunk partials and plan header
 * in a static device buffer of PA_SCRATCH_BYTES that the library holds on each
 * device it runs on until the process ends.  It allocates nothing.
 * ext           required (bt_stride, n_pool_blocks, scale, lse_out, flags,
 *               split_events, seq_lens_host as for pa_decode); ext->workspace
 *               must be NULL and ext->workspace_bytes 0.
 * Every call on a device shares that device's buffer: calls that overlap on
 * one device (on different streams, or from different threads) race.  The
 * buffer's error word is cleared at the start of each call, on `stream`;
 * read it with pa_get_device_error(NULL, NULL, stream, ...).
 * Errors: as pa_decode; PA_ERR_INVALID without ext or with a workspace in
 * it; PA_ERR_UNSUPPORTED when pa_decode_workspace_size(n_seq, n_qtok) on the
 * device exceeds PA_SCRATCH_BYTES (on 256 compute units: up to 2463
 * sequences of one token, 423 of four, 83 of eight). */
#define PA_SCRATCH_BYTES (64u << 20)
pa_status pa_decode_scratch(const float *q, const void *k_pool, const void *v_pool,
                            const int32_t *block_table, const int32_t *seq_lens,
                            int32_t n_seq, int32_t n_qtok, int32_t kv_type, int32_t page_size,
                            float *out, hipStream_t stream, const pa_decode_ext *ext);

/* Bytes of decode workspace for n_seq sequences of n_qtok (1..8) tokens on
 * `device` (reserved up front, as llama.cpp pull 2 does for its split
 * partials in the commit that moved them out of run-time pool allocations).
 * A workspace of this size also serves every call of n_seq or fewer
 * sequences with n_qtok or fewer tokens. */
pa_status pa_decode_workspace_size(int32_t n_seq, int32_t n_qtok, int32_t device, size_t *bytes);

/* Paged chunked prefill: pa_decode for n_qtok = 1..PA_MAX_PREFILL_TOKENS new
 * tokens per sequence (achyudh/llama.cpp pull 2: batches of more query tokens
 * attend paged K/V chunk by chunk, each chunk writing its log-sum-exp, and the
 * normalised parts are merged in f32; batches the large-tile kernel does not
 * take run on the decode kernel's row tiles).  Arguments, layouts, causality
 * (new token t at position seq_len - n_qtok + t sees positions up to it),
 * masking, errors and the ext struct are those of pa_decode; q, out and
 * lse_out hold n_qtok tokens per sequence, and the K/V rows of all n_qtok new
 * tokens must already be in the pages (pa_append_kv / pa_append_kv_device).
 *
 * The tokens are taken in groups of 4 on the matrix-core path (24 query rows
 * of a KV head per workgroup; 8 on the vector path).  Work items are (sequence, KV head, context chunk, token
 * group), the groups of one chunk run side by side so its K/V bytes are
 * shared through the caches, and a group skips the keys past its last token.
 * Chunk partials of every group are merged as in pa_decode.  The workspace
 * (ext->workspace, or the pool's own when it is large enough) must hold
 * pa_prefill_workspace_size() bytes.  Errors as pa_decode; n_qtok outside
 * 1..PA_MAX_PREFILL_TOKENS gives PA_ERR_INVALID. */
pa_status pa_prefill(const float *q, const void *k_pool, const void *v_pool,
                     const int32_t *block_table, const int32_t *seq_lens,
                     int32_t n_seq, int32_t n_qtok, int32_t kv_type, int32_t page_size,
                     float *out, hipStream_t stream, const pa_decode_ext *ext);

/* Bytes of workspace pa_prefill needs for n_seq sequences of n_qtok tokens on
 * `device`. */
pa_status pa_prefill_workspace_size(int32_t n_seq, int32_t n_qtok, int32_t device, size_t *bytes);

/* Reads the error word of a workspace after the work on `stream` finishes
 * (this call waits for the stream) and, if clear != 0, zeroes it (enqueued on
 * `stream`).  Pass NULL to read the pool's own workspace through `pool`;
 * pool and workspace both NULL read the buffer of pa_decode_scratch on the
 * current device. */
pa_status pa_get_device_error(pa_pool *pool, void *workspace, hipStream_t stream,
                              int32_t clear, int32_t *err);

/* Measurement helper: reads `bytes` (a multiple of 16) of device memory at
 * `src` (16-byte aligned) once with 16-byte loads and folds them into one
 * word per wave written to `sink` (device, at least
 * 4 x wgs_per_cu x compute-unit-count words).  Time it to get the HBM read
 * rate that a pure stream of 16-byte loads reaches on this device, the
 * practical ceiling for the K/V stream of pa_decode (the bound the decode
 * roofline refers to: lucebox pull 555 and achyudh/llama.cpp pull 2 report
 * their decode throughput as a share of the card's bandwidth).  Enqueued on
 * `stream`.
 * wgs_per_cu      256-thread workgroups per compute unit (1..32).
 * loads_in_flight 16-byte loads issued back to back per lane (1, 2, 4, 8, 16).
 * flags           PA_PROBE_SLICE: each workgroup streams one contiguous share
 *                 of the buffer (as a split-K work item streams its chunk)
 *                 instead of a grid-stride loop over the whole of it;
 *                 PA_PROBE_LDS: the loads write LDS directly
 *                 (global_load_lds_dwordx4) instead of registers.
 * pa_read_bandwidth_probe is this call with the configuration that measured
 * fastest on MI355X (PA_PROBE_DEFAULT_*).
 * Errors: PA_ERR_INVALID (null or misaligned pointers, bytes 0 or not a
 * multiple of 16, sink too small, a parameter out of range), PA_ERR_HIP. */
#define PA_PROBE_SLICE 1u
#define PA_PROBE_LDS   2u
#define PA_PROBE_DEFAULT_WGS    8
#define PA_PROBE_DEFAULT_LOADS  1
#define PA_PROBE_DEFAULT_FLAGS  0u
pa_status pa_read_bandwidth_probe_ex(const void *src, size_t bytes, uint32_t *sink, size_t sink_words,
                                     int32_t wgs_per_cu, int32_t loads_in_flight, uint32_t flags,
                                     hipStream_t stream);
pa_status pa_read_bandwidth_probe(const void *src, size_t bytes, uint32_t *sink, size_t sink_words,
                                  hipStream_t stream);

/* Test hook: copies the logical rows [0, seq_len) of sequence `seq` of one
 * pool (K or V, row size row_bytes) through its block-table row into dst
 * (device, [4][seq_len][row_bytes]), using the same row-address helper as the
 * decode kernels.  block_table NULL selects contiguous storage as in
 * pa_decode.  Out-of-range table entries leave the affected rows of dst
 * 0xFF-filled and set PA_DEVERR_TABLE in *err_word (device int32, may be
 * NULL). */
pa_status pa_debug_gather(const void *pool, int32_t row_bytes, const int32_t *block_table,
                          int32_t bt_stride, int32_t n_pool_blocks, int32_t seq, int32_t seq_len,
                          int32_t page_size, void *dst, int32_t *err_word, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
