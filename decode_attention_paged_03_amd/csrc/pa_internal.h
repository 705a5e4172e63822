// pa_internal.h -- launch plan shared by the host API (pa_api.cpp) and the kernels
// (pa_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "pa.h"

namespace pa {

// Largest number of pages one fixed partition may span; the partition's block-table
// slice is staged in LDS.
constexpr int kMaxPartitionPages = 512;
// Tokens per partition when PA_FLAG_FORCE_SPLIT is given without a partition size.
constexpr int kDefaultPartition = 1024;
// Balanced route: at most this many sequences (their lengths and tile prefix sums are
// held in LDS) and at most this many workgroups, one per compute unit (sizes the
// workspace on the host, without asking the device).
constexpr int kMaxBalancedBatch = 2048;
constexpr int kMaxBalancedWG = 1024;
// pa_decode_noalloc: bytes of the library's own device scratch array (per GPU).  Enough for
// the balanced route of every supported shape on a part with up to 320 compute units
// (2 sides x 12 streams x 8 heads of 520-byte rows per workgroup, plus its records), and for
// fixed partitions up to that size.
constexpr size_t kNoallocScratchBytes = (size_t)PA_NOALLOC_SCRATCH_BYTES;
// The scratch's last bytes: single-launch arrival counters (3 ints per workgroup), zero from
// load time on because no other layout reaches them and every call leaves them at zero.
constexpr size_t kNoallocCounterBytes = 64 * 1024;
// Query heads one wave scores at once (MFMA rows are 16; LDS partial slots are sized
// for this many heads).
constexpr int kMaxHeadsPerWave = 8;
// Short contexts: every sequence is one partition of the fixed route (no merge, no
// workspace) when the host's bound keeps the longest sequence within
// kSingleMaxTilesPerWave tiles per wave of its workgroup and there are at least
// kSingleMinGrid workgroups, or when no band of the balanced route could hold more than
// kShortBandTiles stream tiles.
constexpr int kShortBandTiles = 24;
constexpr int kSingleMaxTilesPerWave = 8;
constexpr int kSingleMinGrid = 64;
// Waves per fixed-route workgroup: kFixedWavesWide when the grid is no larger than the
// compute units, else kFixedWaves.
constexpr int kFixedWaves = 4;
constexpr int kFixedWavesWide = 8;
// The plan is made at pa_create, which makes no HIP call: its route choice assumes the
// compute units of an MI355X.  (Each call still sizes its grids from the device.)
constexpr int kPlanComputeUnits = 256;

struct Plan {
    pa_problem prob;        // validated copy, defaults resolved
    int group;              // query heads per KV head
    int heads_per_wg;       // query heads one workgroup serves (divides group, <= 8)
    int n_chunks;           // group / heads_per_wg
    bool balanced;          // route: even split of all token tiles over a resident grid
    bool short_single;      // short contexts (the host's bound): the fixed route with one
                            // partition per sequence, no merge and no workspace
    bool partition_balanced;  // a partition size was given and the balanced route may run
                              // (when its partials fit it: balanced_partials_fit)
    long long balanced_units_max;  // balanced route: bound on the batch's (band, tile) units
    int bal_waves;          // balanced route: waves per workgroup (8, 12 or 16)
    int spw;                // balanced route: streams a workgroup reads side by side
    int waves_per_stream;   // balanced route: bal_waves / spw
    int bands;              // balanced route: (streams per sequence) / spw
    // fixed-partition route
    int partition;          // tokens per partition (multiple of page_size)
    int n_part_max;         // ceil(max_context_length / partition), >= 1
    bool force_split;       // every sequence writes partition triples and is merged
    // both
    int ps_log2;            // log2(page_size)
    bool need_merge;        // a merge kernel is launched
    bool debug_bounds;      // PA_FLAG_DEBUG_BOUNDS: record table entries outside the pool
    bool single_launch;     // PA_FLAG_SINGLE_LAUNCH: the decode kernel merges crossing bands
    size_t rows_per_wg;     // balanced route: partial rows per workgroup (2 sides x spw x heads)
    size_t ws_bytes;        // workspace bytes pa_workspace_size() reports (0 when need_merge is
                            // false): the layout for kMaxBalancedWG workgroups
    long long decode_grid;  // workgroups of the fixed-partition decode kernel
    long long merge_grid;   // workgroups of the fixed-partition merge kernel
};

// Where the parts of the workspace start.  The balanced route's partial rows are indexed
// by workgroup, so its layout depends on how many workgroups it is sized for: the
// caller-provided workspace is sized for kMaxBalancedWG (no device query on the host), the
// library's own scratch (pa_decode_noalloc) for the device's compute units.
struct WsLayout {
    size_t bitmap_words;    // PA_FLAG_DEBUG_BOUNDS: uint32 words of the bad-entry bitmap at
                            // offset 0 (0 without the flag)
    size_t acc_offset;      // byte offset of the partial rows (the bitmap rounded to 256 B)
    size_t ml_offset;       // byte offset of the (max, sum) pairs
    size_t desc_offset;     // balanced route: byte offset of the per-workgroup merge records
    size_t cnt_offset;      // single launch: byte offset of the arrival counters (3 per workgroup)
    size_t bytes;           // total (0 when no merge is launched and no bitmap is kept)
    int wg_slots;           // balanced route: workgroups the partial rows are sized for
};
WsLayout workspace_layout(const Plan& plan, int wg_slots);

// The plan with the balanced route chosen (a partition-size plan whose partials fit).
Plan as_balanced(const Plan& plan);
// Whether, on a device with `cus` compute units, every partial of the balanced route covers
// at most the problem's partition size (then that route honours it and runs).
bool balanced_partials_fit(const Plan& plan, int cus);

// Host-only validation + planning; returns a pa_status.
int build_plan(const pa_problem* p, Plan* out);

// Compute units of the current device (capped at kMaxBalancedWG), queried once per device
// and cached; 0 when the HIP runtime reports an error.
int device_compute_units();

// Enqueue the decode (and, if planned, merge) kernels.  Pointers already validated; the
// workspace holds at least layout.bytes bytes laid out as `layout`, and the balanced route's
// grid (the device's compute units) is at most the workgroups the layout is sized for.
hipError_t launch(const Plan& plan, const void* q, const void* k, const void* v,
                  const int32_t* block_tables, const int32_t* ctx, float scale, float* out,
                  void* workspace, const WsLayout& layout, hipStream_t stream);

// pa_append: workgroup size for a sequence's kv_heads * head_dim / 8 16-byte chunks (whole
// waves, at most kAppendThreads; more chunks take more workgroups along grid y).
constexpr int kAppendThreads = 256;
inline int append_threads(long long row_chunks) {
    return row_chunks >= kAppendThreads ? kAppendThreads : (int)((row_chunks + 63) / 64 * 64);
}

// pa_decode_noalloc: the library's own scratch array on the current device.  The first
// call on a device looks up the array's device address (and the device's compute units);
// later calls return the cached values.  Returns false when the HIP runtime reports an
// error.
bool noalloc_scratch(void** ptr, size_t* bytes);

// Enqueue the kernel that stores one new key / value row per sequence (pa_append).
hipError_t launch_append(const Plan& plan, const void* new_k, const void* new_v, void* k_cache,
                         void* v_cache, const int32_t* block_tables, const int32_t* positions,
                         hipStream_t stream);

}  // namespace pa
