// pa_api.cpp -- the C ABI of libpa.so: argument validation, launch planning and
// dispatch.  Everything before pa::launch() is plain host code with no HIP call, so the
// error paths can be exercised on a machine without a GPU.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "pa.h"
#include "pa_internal.h"

struct pa_handle {
    pa::Plan plan;
};

namespace pa {

static bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

static int gcd(int a, int b) {
    while (b) {
        const int t = a % b;
        a = b;
        b = t;
    }
    return a;
}

// Waves per balanced workgroup (12: three per SIMD, which the kernels' register use
// allows; more waves, each with one tile in flight, keep more of the memory system busy).
// Balanced route: below this many bands in the batch, fewer streams are read side by side.
static constexpr long long kFewBands = 32;

static int balanced_waves(int /*streams*/) {
#ifdef PA_BAL_WAVES
    if (PA_BAL_WAVES == 8 || PA_BAL_WAVES == 12 || PA_BAL_WAVES == 16) return PA_BAL_WAVES;
#endif
    return 12;
}

static int ilog2(int x) {
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

int build_plan(const pa_problem* in, Plan* pl) {
    if (!in || !pl) return PA_ERR_INVALID_ARGUMENT;
    pa_problem p = *in;
    if (p.batch < 1 || p.query_heads < 1 || p.kv_heads < 1 || p.head_dim < 1 || p.page_size < 1 ||
        p.max_pages_per_sequence < 1 || p.num_physical_pages < 1 || p.partition_size < 0 ||
        p.max_context_length < 0)
        return PA_ERR_INVALID_ARGUMENT;
    if (p.query_heads % p.kv_heads) return PA_ERR_INVALID_ARGUMENT;
    const uint32_t known = PA_FLAG_FORCE_SPLIT | PA_FLAG_FORCE_SINGLE | PA_FLAG_DEBUG_BOUNDS |
                           PA_FLAG_SINGLE_LAUNCH | PA_FLAG_FIXED_PARTITIONS;
    if (p.flags & ~known) return PA_ERR_INVALID_ARGUMENT;
    if ((p.flags & PA_FLAG_FORCE_SPLIT) && (p.flags & PA_FLAG_FORCE_SINGLE))
        return PA_ERR_INVALID_ARGUMENT;
    if (p.head_dim != 64 && p.head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!is_pow2(p.page_size) || p.page_size < 8 || p.page_size > 256) return PA_ERR_UNSUPPORTED;

    const long long table_tokens = (long long)p.max_pages_per_sequence * p.page_size;
    if (table_tokens > INT32_MAX) return PA_ERR_UNSUPPORTED;
    if (p.max_context_length == 0) p.max_context_length = (int32_t)table_tokens;
    if (p.max_context_length > table_tokens) return PA_ERR_INVALID_ARGUMENT;

    Plan out{};
    out.group = p.query_heads / p.kv_heads;
    out.heads_per_wg = 1;
    for (int hp = kMaxHeadsPerWave; hp >= 1; --hp)
        if (out.group % hp == 0) { out.heads_per_wg = hp; break; }
    out.n_chunks = out.group / out.heads_per_wg;
    out.ps_log2 = ilog2(p.page_size);
    // No partition size and no flag: the library splits the work itself (balanced
    // route).  A route flag asks for fixed partitions.  A partition size bounds the tokens
    // any partial (max, sum, acc) triple covers: the balanced route runs when the
    // problem's sizes guarantee its partials stay within it (decided per call, from the
    // device's compute units; see balanced_partials_fit), else fixed partitions of exactly
    // that size.  The balanced route's tile indices are 32-bit: all (sequence, KV head,
    // chunk) streams together hold fewer than 2^31 tiles of 16 tokens.
    const long long max_tiles = (long long)p.batch * p.kv_heads * out.n_chunks * ((p.max_context_length + 15LL) / 16);
    const uint32_t route_flags = p.flags & (PA_FLAG_FORCE_SPLIT | PA_FLAG_FORCE_SINGLE | PA_FLAG_FIXED_PARTITIONS);
    const bool balanced_capable = route_flags == 0 && p.batch <= kMaxBalancedBatch && max_tiles <= INT32_MAX;
    out.balanced = balanced_capable && p.partition_size == 0;
    out.partition_balanced = balanced_capable && p.partition_size > 0;
    out.debug_bounds = (p.flags & PA_FLAG_DEBUG_BOUNDS) != 0;
    out.single_launch = (p.flags & PA_FLAG_SINGLE_LAUNCH) != 0;
    // one launch needs the default route: no partition size, no route flag
    if (out.single_launch && (p.partition_size != 0 || route_flags != 0)) return PA_ERR_INVALID_ARGUMENT;
    if (out.single_launch && !out.balanced) return PA_ERR_UNSUPPORTED;
    // the bitmap has one bit per table entry
    if (out.debug_bounds && (long long)p.batch * p.max_pages_per_sequence > (1LL << 40))
        return PA_ERR_UNSUPPORTED;

    int partition = p.partition_size;
    if (p.flags & PA_FLAG_FORCE_SINGLE) {
        long long t = ((long long)p.max_context_length + p.page_size - 1) / p.page_size * p.page_size;
        partition = (int)(t < p.page_size ? p.page_size : t);
    } else if (partition == 0) {
        partition = kDefaultPartition < p.page_size ? p.page_size : kDefaultPartition;
    }
    if (partition % p.page_size) return PA_ERR_INVALID_ARGUMENT;
    if (!out.balanced && partition / p.page_size > kMaxPartitionPages) return PA_ERR_UNSUPPORTED;
    p.partition_size = out.balanced ? 0 : partition;
    // the fixed route's limits hold whenever it may run (a partition size may still take it)
    out.prob = p;
    out.partition = partition;
    long long nparts = ((long long)p.max_context_length + partition - 1) / partition;
    out.n_part_max = (int)(nparts < 1 ? 1 : nparts);
    out.force_split = (p.flags & PA_FLAG_FORCE_SPLIT) != 0;
    // the merge reads one output row's partition triples through a buffer resource with a
    // 32-bit range
    if (!out.balanced && (long long)out.n_part_max * p.head_dim * 4 > INT32_MAX) return PA_ERR_UNSUPPORTED;

    const long long grid = (long long)p.batch * p.kv_heads * out.n_chunks * out.n_part_max;
    const long long mgrid = (long long)p.batch * p.query_heads;
    if (mgrid > INT32_MAX || (!out.balanced && grid > INT32_MAX)) return PA_ERR_UNSUPPORTED;
    out.decode_grid = grid;
    out.merge_grid = mgrid;
    if (balanced_capable) {
        const int streams = p.kv_heads * out.n_chunks;
        out.bal_waves = balanced_waves(streams);
        out.spw = gcd(streams, out.bal_waves);
        // With few bands in the whole batch (one long sequence, a handful of sequences),
        // each band spans many workgroups and leaves one piece of spw x heads_per_wg rows
        // in each: the merge then weighs most, and reading half as many streams side by
        // side halves its rows.  With many bands, more bands per sequence cost the decode
        // kernel more segments per wave than the merge saves.
        if ((long long)p.batch * (streams / out.spw) < kFewBands && out.spw % 2 == 0) out.spw /= 2;
        out.waves_per_stream = out.bal_waves / out.spw;
        out.bands = streams / out.spw;
        out.rows_per_wg = (size_t)2 * out.spw * out.heads_per_wg;
        // units (band, 16-token tile) of the whole batch at most, from the host's bound
        out.balanced_units_max = (long long)out.bands * p.batch * ((p.max_context_length + 15LL) / 16);
        // Short contexts (the host's bound): every sequence is one partition of the fixed
        // route -- a workgroup per (sequence, KV head, head chunk) reads its own length,
        // takes all the sequence's tiles and writes its rows: no split to compute, no
        // merge, no workspace (p2's single-tile fast path for every sequence).  Taken when
        // the longest sequence needs at most kSingleMaxTilesPerWave tiles per wave of its
        // workgroup and the grid has kSingleMinGrid workgroups, or when every band is short
        // (the even split would then leave most compute units idle and split every band
        // over many workgroups).  Measured against the even split, alternating in one
        // process: 1.5-35% less on 11 shapes of 8 to 512 sequences up to 1024 tokens at up
        // to 8 tiles per wave; 2-40% more at 16 or more tiles per wave (batch64 58.4 against
        // 65.3 us) and on a 32-workgroup grid; tiny 6.8 -> 5.0 us.
        const long long band_tiles = (p.max_context_length + 15LL) / 16 * out.spw;
        const long long grid_single = (long long)p.batch * p.kv_heads * out.n_chunks;
        const long long waves_single = grid_single <= kPlanComputeUnits ? kFixedWavesWide : kFixedWaves;
        const long long per_wave = ((p.max_context_length + 15LL) / 16 + waves_single - 1) / waves_single;
        const bool single_fits = per_wave <= kSingleMaxTilesPerWave && grid_single >= kSingleMinGrid;
        if (out.balanced && (band_tiles <= kShortBandTiles || single_fits)) {
            const long long t = ((long long)p.max_context_length + p.page_size - 1) / p.page_size * p.page_size;
            const int whole = (int)(t < p.page_size ? p.page_size : t);
            if (whole / p.page_size <= kMaxPartitionPages) {
                out.balanced = false;
                out.short_single = true;
                out.single_launch = false;   // one kernel already
                out.partition = whole;
                out.n_part_max = 1;
                out.prob.partition_size = whole;
                out.decode_grid = (long long)p.batch * p.kv_heads * out.n_chunks;
            }
        }
    }
    out.need_merge = out.balanced || out.force_split || out.n_part_max > 1;
    out.ws_bytes = workspace_layout(out, kMaxBalancedWG).bytes;
    if (out.partition_balanced) {
        const size_t b = workspace_layout(as_balanced(out), kMaxBalancedWG).bytes;
        if (b > out.ws_bytes) out.ws_bytes = b;
    }
    *pl = out;
    return PA_OK;
}

Plan as_balanced(const Plan& pl) {
    Plan r = pl;
    r.balanced = true;
    r.short_single = false;
    r.need_merge = true;
    return r;
}

bool balanced_partials_fit(const Plan& pl, int cus) {
    if (!pl.partition_balanced || cus <= 0) return false;
    // A workgroup's range holds at most ceil(units / grid) units, so no partial covers more
    // than 16 times that many tokens of a stream.
    const long long per_wg = (pl.balanced_units_max + cus - 1) / cus;
    return 16 * per_wg <= pl.prob.partition_size;
}

WsLayout workspace_layout(const Plan& pl, int wg_slots) {
    WsLayout l{0, 0, 0, 0, 0, 0, wg_slots};
    if (pl.debug_bounds) {
        l.bitmap_words = ((size_t)pl.prob.batch * (size_t)pl.prob.max_pages_per_sequence + 31) / 32;
        l.acc_offset = (l.bitmap_words * 4 + 255) / 256 * 256;
    }
    if (!pl.need_merge) {
        l.ml_offset = l.desc_offset = l.cnt_offset = l.bytes = l.acc_offset;
        return l;
    }
    size_t rows;
    if (pl.balanced) {
        // Rows of D floats (plus a (max, sum) pair each): per workgroup, two sides x spw
        // streams x heads_per_wg heads of piece triples; then two 16-byte merge records
        // per workgroup.
        rows = (size_t)wg_slots * pl.rows_per_wg;
    } else {
        // one triple per (sequence, query head, partition)
        rows = (size_t)pl.prob.batch * pl.prob.query_heads * (size_t)pl.n_part_max;
    }
    l.ml_offset = l.acc_offset + rows * (size_t)pl.prob.head_dim * sizeof(float);
    l.desc_offset = l.ml_offset + rows * 2 * sizeof(float);
    l.cnt_offset = l.desc_offset + (pl.balanced ? (size_t)wg_slots * 2 * 16 : 0);
    l.bytes = l.cnt_offset + (pl.single_launch ? (size_t)wg_slots * 3 * sizeof(int) : 0);
    l.wg_slots = wg_slots;
    return l;
}

}  // namespace pa

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A float that is neither infinite nor NaN, tested on its bits (the library is built with
// no-NaN arithmetic semantics, under which a library isfinite() may be folded away).
static bool finite_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    return (u & 0x7f800000u) != 0x7f800000u;
}

// The checks pa_decode() and pa_decode_noalloc() share (host only).
static pa_status check_decode_args(const pa_handle* handle, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lengths, float scale, const float* out) {
    if (!handle || !query || !key_cache || !value_cache || !block_tables || !context_lengths || !out)
        return PA_ERR_INVALID_ARGUMENT;
    if (!finite_bits(scale)) return PA_ERR_INVALID_ARGUMENT;
    if (!aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) || !aligned16(out))
        return PA_ERR_MISALIGNED;
    return PA_OK;
}

extern "C" {

pa_status pa_create(const pa_problem* problem, pa_handle** out) {
    if (!out) return PA_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    pa::Plan plan;
    int st = pa::build_plan(problem, &plan);
    if (st != PA_OK) return (pa_status)st;
    pa_handle* h = new (std::nothrow) pa_handle;
    if (!h) return PA_ERR_NO_MEMORY;
    h->plan = plan;
    *out = h;
    return PA_OK;
}

pa_status pa_workspace_size(const pa_handle* handle, size_t* bytes) {
    if (!handle || !bytes) return PA_ERR_INVALID_ARGUMENT;
    *bytes = handle->plan.ws_bytes;
    return PA_OK;
}

pa_status pa_decode(const pa_handle* handle, const void* query, const void* key_cache,
                    const void* value_cache, const int32_t* block_tables,
                    const int32_t* context_lengths, float scale, float* out, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
    const pa_status st = check_decode_args(handle, query, key_cache, value_cache, block_tables,
                                           context_lengths, scale, out);
    if (st != PA_OK) return st;
    const pa::Plan& pl = handle->plan;
    if (pl.ws_bytes) {
        if (!workspace || workspace_bytes < pl.ws_bytes) return PA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PA_ERR_MISALIGNED;
    }
    // a partition size that the balanced route's partials respect on this device takes it
    const pa::Plan run = pa::balanced_partials_fit(pl, pa::device_compute_units()) ? pa::as_balanced(pl) : pl;
    hipError_t err = pa::launch(run, query, key_cache, value_cache, block_tables, context_lengths,
                                scale, out, workspace, pa::workspace_layout(run, pa::kMaxBalancedWG),
                                stream);
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_decode_noalloc(const pa_handle* handle, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lengths, float scale, float* out,
                            hipStream_t stream) {
    const pa_status st = check_decode_args(handle, query, key_cache, value_cache, block_tables,
                                           context_lengths, scale, out);
    if (st != PA_OK) return st;
    const pa::Plan& plan = handle->plan;
    if (plan.debug_bounds) return PA_ERR_INVALID_ARGUMENT;   // its bitmap needs a caller workspace
    const int cus = plan.partition_balanced ? pa::device_compute_units() : 0;
    const pa::Plan pl = pa::balanced_partials_fit(plan, cus) ? pa::as_balanced(plan) : plan;
    void* scratch = nullptr;
    pa::WsLayout layout{0, 0, 0, 0, 0, 0, 0};
    if (pl.need_merge) {
        // the balanced route's rows are indexed by workgroup: sized for this device's grid
        const int slots = pl.balanced ? pa::device_compute_units() : 0;
        if (pl.balanced && slots <= 0) return PA_ERR_HIP;
        layout = pa::workspace_layout(pl, slots);
        // the scratch's tail holds the single-launch counters, which no layout may reach
        const size_t usable = pa::kNoallocScratchBytes - pa::kNoallocCounterBytes;
        if (layout.cnt_offset > usable) return PA_ERR_SCRATCH;
        if ((size_t)slots * 3 * sizeof(int) > pa::kNoallocCounterBytes) return PA_ERR_SCRATCH;
        if (pl.single_launch) {
            layout.cnt_offset = usable;
            layout.bytes = pa::kNoallocScratchBytes;
        }
        size_t cap = 0;
        if (!pa::noalloc_scratch(&scratch, &cap)) return PA_ERR_HIP;
        if (layout.bytes > cap) return PA_ERR_SCRATCH;
    }
    hipError_t err = pa::launch(pl, query, key_cache, value_cache, block_tables, context_lengths,
                                scale, out, scratch, layout, stream);
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_append(const pa_handle* handle, const void* new_key, const void* new_value,
                    void* key_cache, void* value_cache, const int32_t* block_tables,
                    const int32_t* positions, hipStream_t stream) {
    if (!handle || !new_key || !new_value || !key_cache || !value_cache || !block_tables ||
        !positions)
        return PA_ERR_INVALID_ARGUMENT;
    if (!aligned16(new_key) || !aligned16(new_value) || !aligned16(key_cache) ||
        !aligned16(value_cache))
        return PA_ERR_MISALIGNED;
    const pa::Plan& pl = handle->plan;
    // grid: one workgroup column per sequence (x), the sequence's row chunks along y
    const long long row_chunks = (long long)pl.prob.kv_heads * (pl.prob.head_dim / 8);
    const long long threads = pa::append_threads(row_chunks);
    // a page's bytes address one buffer resource (32-bit range)
    if (row_chunks * 16 * pl.prob.page_size > INT32_MAX ||
        (row_chunks + threads - 1) / threads > 65535 ||
        (long long)pl.prob.batch * threads > UINT32_MAX)
        return PA_ERR_UNSUPPORTED;
    hipError_t err = pa::launch_append(pl, new_key, new_value, key_cache, value_cache,
                                       block_tables, positions, stream);
    return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_destroy(pa_handle* handle) {
    delete handle;
    return PA_OK;
}

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "PA_OK";
        case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
        case PA_ERR_MISALIGNED: return "PA_ERR_MISALIGNED";
        case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
        case PA_ERR_HIP: return "PA_ERR_HIP";
        case PA_ERR_NO_MEMORY: return "PA_ERR_NO_MEMORY";
        case PA_ERR_SCRATCH: return "PA_ERR_SCRATCH";
        default: return "PA_ERR_UNKNOWN";
    }
}

}  // extern "C"
