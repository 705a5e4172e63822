/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-attention decode library (libpa.so).
 *
 * One call, pa_decode(), evaluates one decode step of attention for a batch of
 * sequences whose keys and values live in a paged cache:
 *
 *   out[b][h][:] = sum_t softmax_t( scale * q[b][h] . K[t][g] ) * V[t][g][:]
 *
 * over the context_lengths[b] cached tokens t of sequence b, with query head h
 * reading KV head g = h / (query_heads / kv_heads).  The definition is the one of
 * the "Paged Attention" section of "[TIL] Optimizing paged attention"
 * (retepy.com); the score is multiplied by `scale` as in that page's Baseline
 * kernel, and query heads map to KV heads in contiguous groups as there.
 *
 * Cache layout ("Data Layout" section of the same page): key_cache and
 * value_cache are pools of physical pages, each [page_size][kv_heads][head_dim]
 * fp16, pages contiguous: element (page p, slot s, kv head g, dim d) is at
 * ((p * page_size + s) * kv_heads + g) * head_dim + d.  Token t of sequence b is
 * in slot t % page_size of physical page block_tables[b][t / page_size].
 *
 * Long contexts are split into partitions of partition_size tokens whose
 * (max, sum, unnormalised output) triples are combined afterwards, as the
 * "V4 (Context-axis parallelism)" section of the same page does with its split
 * and merge kernels; a sequence that fits one partition is finished in a single
 * pass without the workspace (the single-tile path of the
 * "paged_attention_v2_pytorch.py" commit page).
 *
 * Ownership and threading: the caller owns every device buffer, the workspace
 * and the stream; the library owns only the host-side handle.  pa_decode()
 * allocates nothing, copies nothing to or from the host and does not
 * synchronise: it enqueues one or two kernels on `stream` and returns.  Buffers
 * must stay valid until the stream has passed the call.  A handle is immutable
 * after pa_create() and may be used from several threads at once; concurrent
 * calls need distinct workspaces.
 *
 * Errors: every function returns a pa_status.  Argument checks run on the host
 * before any HIP call; device array contents (table entries, lengths) are
 * preconditions the library does not check (see pa_decode).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
    PA_OK = 0,
    PA_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, query_heads % kv_heads != 0,
                                    partition_size not a multiple of page_size, ...            */
    PA_ERR_UNSUPPORTED = 2,      /* a shape this build has no kernel for (head_dim, page_size,
                                    partition too long)                                         */
    PA_ERR_MISALIGNED = 3,       /* query / key_cache / value_cache / out / workspace not 16-byte
                                    aligned                                                     */
    PA_ERR_WORKSPACE = 4,        /* workspace missing or smaller than pa_workspace_size()        */
    PA_ERR_HIP = 5,              /* the HIP runtime reported an error on launch                  */
    PA_ERR_NO_MEMORY = 6,        /* host allocation of the handle failed                         */
    PA_ERR_SCRATCH = 7           /* pa_decode_noalloc: the problem needs more workspace than the
                                    library's scratch array holds (PA_NOALLOC_SCRATCH_BYTES)      */
} pa_status;

/* Bytes of the device scratch array pa_decode_noalloc() uses in place of a workspace (one
 * array per GPU, held until the process ends).  Its last 64 KiB hold the arrival counters
 * of PA_FLAG_SINGLE_LAUNCH calls; a problem's workspace must fit in the rest. */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Flags for pa_problem.flags */
#define PA_FLAG_FORCE_SPLIT  0x1u /* route every sequence through partition triples + merge */
#define PA_FLAG_FORCE_SINGLE 0x2u /* one partition per sequence (partition = max context)     */
/* Partitions of exactly partition_size tokens, counted from token 0 (the PARTITION_SIZE
 * scheme of the "paged_attention_v2_pytorch.py" commit page), even when the default split
 * would keep every partial within partition_size (see pa_problem.partition_size). */
#define PA_FLAG_FIXED_PARTITIONS 0x10u
/* Record block-table entries outside the pool.  Every call treats a table entry that a
 * context dereferences but that lies outside [0, num_physical_pages) as a page of zero
 * keys and values: it is never read, so it cannot fault.  (The first page's "Baseline"
 * section shows unused table slots as placeholders and never describes an entry that
 * names no page.)  With this flag, pa_decode() also records each such entry: the
 * workspace then begins with a bitmap of batch * max_pages_per_sequence bits in
 * little-endian uint32 words, with bit i of word w for table entry 32 w + i (row-major,
 * entry b * max_pages_per_sequence + logical page).  The call clears the bitmap, then
 * sets the bit of every dereferenced entry outside the pool.  The caller reads the
 * words after the stream passes the call.  pa_workspace_size() includes them, rounded up
 * to 256 bytes. */
#define PA_FLAG_DEBUG_BOUNDS 0x4u
/* One kernel launch per call on the default route: the workgroups that share a context
 * split merge it themselves at the end of the decode kernel (the last to arrive on a
 * counter merges; long splits in two levels of at most 16 pieces each) instead of a
 * second merge kernel, the split and merge of the first page's "V4 (Context-axis
 * parallelism)" section in one launch.  Only without a partition size or the route flags
 * above.  The workspace then ends with arrival counters that must be zero before the
 * first call: zero the whole workspace once after allocating it (e.g. hipMemset), and
 * again after using it for any other problem or route.  Every call leaves its counters
 * at zero.  (pa_decode_noalloc keeps its own counters, zero from the start.)  A crossing
 * band is merged in groups of 16 pieces, 16 groups at most: on a GPU with more than 256
 * compute units the call fails with PA_ERR_HIP before enqueuing anything.  Measured
 * slower than the two launches on the serving-shaped and long-context workloads: the
 * device-scope arrivals cost more than the second launch. */
#define PA_FLAG_SINGLE_LAUNCH 0x8u

typedef struct pa_problem {
    int32_t batch;                  /* number of sequences, >= 1                                  */
    int32_t query_heads;            /* query heads per sequence, multiple of kv_heads             */
    int32_t kv_heads;               /* KV heads, >= 1                                             */
    int32_t head_dim;               /* 64 or 128                                                  */
    int32_t page_size;              /* tokens per page: power of two, 8 .. 256                    */
    int32_t max_pages_per_sequence; /* row stride of block_tables                                 */
    int32_t num_physical_pages;     /* pages in each of key_cache / value_cache (pa_append writes
                                       only below it)                                             */
    int32_t partition_size;         /* 0: the library splits the work (default; when the bound
                                       below keeps every context short, each sequence is one
                                       partition and no workspace is needed).  > 0: no
                                       partial (max, sum, acc) triple covers more than this many
                                       tokens of a context; a multiple of page_size, at most 512
                                       pages.  The default split runs when the problem's sizes
                                       guarantee that on the device (every workgroup's share is
                                       at most partition_size tokens per stream); otherwise, or
                                       with PA_FLAG_FIXED_PARTITIONS or a FORCE flag, fixed
                                       partitions of exactly this many tokens                     */
    int32_t max_context_length;     /* bound on every context_lengths[b]; sizes the grid and the
                                       workspace; 0 -> max_pages_per_sequence * page_size          */
    uint32_t flags;                 /* PA_FLAG_*                                                  */
} pa_problem;

typedef struct pa_handle pa_handle; /* opaque, host memory only */

/* Validate *problem and create a handle holding a copy of it plus the launch plan.
 * The problem struct is the shape description of the launchers in the first page's
 * "Baseline" to "V4" sections (batch, query and KV heads, head_dim, page_size, table row
 * stride), plus the pool size, the split and the flags.  Host only: no HIP call.  On
 * error *out is set to NULL. */
pa_status pa_create(const pa_problem *problem, pa_handle **out);

/* Bytes of device workspace pa_decode() needs for this problem.  The workspace holds the
 * partial (max, sum, output) triples of a split context, as in the split kernel of the
 * first page's "V4 (Context-axis parallelism)" section, whose launcher leaves workspace
 * ownership to its caller; with PA_FLAG_DEBUG_BOUNDS the bad-entry bitmap comes first.
 * 0 when no sequence can need more than one partition and the flag is not set.  Host
 * only. */
pa_status pa_workspace_size(const pa_handle *handle, size_t *bytes);

/* Enqueue one decode step on `stream`.
 *   query           fp16 [batch][query_heads][head_dim], 16-byte aligned
 *   key_cache       fp16 [pages][page_size][kv_heads][head_dim], 16-byte aligned
 *   value_cache     fp16, same layout as key_cache
 *   block_tables    int32 [batch][max_pages_per_sequence]
 *   context_lengths int32 [batch]
 *   scale           multiplies q . k (pass 1/sqrt(head_dim) for the usual scaling)
 *   out             fp32 [batch][query_heads][head_dim], 16-byte aligned; every element is
 *                   written (a sequence with context length 0 gets zeros)
 *   workspace       device scratch of at least pa_workspace_size() bytes, 16-byte aligned
 *                   (may be NULL when that size is 0); contents undefined afterwards
 * Precondition (not checked): 0 <= context_lengths[b] <= max_context_length.  Table
 * entries i < ceil(context_lengths[b] / page_size) should lie in [0, num_physical_pages):
 * one that does not reads as a page of zeros (see PA_FLAG_DEBUG_BOUNDS).  Table slots past
 * that are never read.  Pointers are device pointers (or host-mapped memory the GPU can
 * read).  The step is the "Paged Attention" definition above, evaluated as the first
 * page's Baseline recurrence with the "V4" split and merge (and the commit page's
 * single-tile path for contexts that need no merge). */
pa_status pa_decode(const pa_handle *handle, const void *query, const void *key_cache,
                    const void *value_cache, const int32_t *block_tables,
                    const int32_t *context_lengths, float scale, float *out, void *workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* pa_decode() for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It takes pa_decode()'s
 * arguments except the workspace, and uses instead a device array inside the library of
 * PA_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, which each GPU holds until the process ends.
 * The first call on a device (with that device current) looks up the array's address and
 * the device's compute-unit count and caches both; no call allocates (no hipMalloc,
 * hipFree or allocating library routine), copies to or from the host or synchronises.
 * Returns PA_ERR_SCRATCH, before enqueuing anything, when the problem needs more workspace
 * than the array holds (e.g. fixed partitions over a large batch; the default route of
 * every supported shape fits on a GPU of up to 320 compute units), and
 * PA_ERR_INVALID_ARGUMENT for a problem with PA_FLAG_DEBUG_BOUNDS (its bitmap needs a
 * workspace the caller can read).
 * All calls on one GPU share its array, and the array keeps the last call's contents: two
 * calls that may run at the same time on one GPU (two streams, two threads without
 * ordering) race and corrupt each other's results.  Order them on one stream. */
pa_status pa_decode_noalloc(const pa_handle *handle, const void *query, const void *key_cache,
                            const void *value_cache, const int32_t *block_tables,
                            const int32_t *context_lengths, float scale, float *out,
                            hipStream_t stream);

/* Enqueue the step before a decode: store one new token's key and value rows per
 * sequence in the paged cache.  The cache exists so that earlier tokens' keys and values
 * are reused rather than recomputed ("Paged Attention" section of the page named above);
 * under its "Data Layout" section the token at position pos of sequence b belongs in slot
 * pos % page_size of physical page block_tables[b][pos / page_size].
 *   new_key, new_value  fp16 [batch][kv_heads][head_dim], 16-byte aligned
 *   key_cache, value_cache  the caches pa_decode() reads (same layout), 16-byte aligned;
 *                   written in place, one row per (sequence, KV head)
 *   block_tables    int32 [batch][max_pages_per_sequence]
 *   positions       int32 [batch]: the new token's position (the context length before
 *                   the step); a negative position stores nothing for that sequence
 * A position at or past max_pages_per_sequence * page_size, or a table entry outside
 * [0, num_physical_pages), names no slot: that sequence is skipped and no byte outside the
 * pool is written.  Two sequences must not name the same slot (the stores would race).
 * Uses the batch, kv_heads, head_dim, page_size, max_pages_per_sequence and
 * num_physical_pages of the handle's problem; needs no workspace; allocates nothing and
 * does not synchronise.  A following pa_decode() on the same stream with
 * context_lengths[b] = positions[b] + 1 attends over the new token. */
pa_status pa_append(const pa_handle *handle, const void *new_key, const void *new_value,
                    void *key_cache, void *value_cache, const int32_t *block_tables,
                    const int32_t *positions, hipStream_t stream);

/* Free the handle (host memory only; the library holds nothing else per handle, as the
 * first page's launchers hold nothing between calls).  NULL is accepted. */
pa_status pa_destroy(pa_handle *handle);

/* Static, NUL-terminated name of a status code (a host-side convenience with no
 * counterpart on the pages). */
const char *pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
