// pa_append.hip -- storing a decode step's new key and value rows in the paged cache
// (gfx950).
//
// The cache keeps the keys and values of a sequence's earlier tokens so that they are
// reused instead of recomputed ("Paged Attention" section of "[TIL] Optimizing paged
// attention"); each decode step first stores its own token.  Token position pos of
// sequence b lives in slot pos % page_size of physical page block_tables[b][pos /
// page_size], and the row of KV head g starts at element
// ((page * page_size + slot) * kv_heads + g) * head_dim ("Data Layout" section of the same
// page).
//
// The move is a scatter of batch * kv_heads rows of head_dim fp16 per cache: a few hundred
// KB at most for a decode batch, so its time is latency, not bandwidth.  Workgroup x of
// the grid serves sequence x, so the sequence's position and table entry are wave-uniform
// loads; one lane moves one 16-byte chunk of a key row and the same chunk of the value
// row (the lanes of a row are adjacent: full, coalesced 16-byte accesses).  The stores
// are unconditional buffer stores through a resource over the target page whose range is
// zero when the position names no slot (the hardware range check drops them), so nothing
// branches on the position and the new rows are loaded alongside it: a store waits for
// one dependent pair of loads (position, then table entry) rather than three.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// dword 3 of a raw buffer resource on this target
constexpr int kBufferFlags = 0x00020000;
// a byte offset past every page's range: a store there is dropped
constexpr uint32_t kNoSlot = 0x7FFFFF00u;

// kChunks = head_dim / 8: 16-byte chunks per row.  row_chunks = kv_heads * kChunks;
// page_bytes = page_size * kv_heads * head_dim * 2.
template <int kChunks>
__global__ void __launch_bounds__(kAppendThreads)
pa_append_kernel(const uint4* __restrict__ new_k, const uint4* __restrict__ new_v,
                 char* __restrict__ k_cache, char* __restrict__ v_cache,
                 const int32_t* __restrict__ block_tables, const int32_t* __restrict__ positions,
                 int row_chunks, int kv_heads, int ps_log2, int max_pages, int num_pages,
                 int page_bytes) {
    const int b = blockIdx.x;
    const int j = blockIdx.y * blockDim.x + threadIdx.x;  // chunk among the sequence's rows
    const bool lane_ok = j < row_chunks;
    const long long src = (long long)b * row_chunks + (lane_ok ? j : 0);
    const uint4 kk = new_k[src];
    const uint4 vv = new_v[src];
    // Positions outside the table row, and table entries outside the pool, name no slot:
    // nothing is stored for that sequence (a negative position asks for exactly that).
    const int pos = positions[b];
    bool ok = pos >= 0 && (long long)pos < ((long long)max_pages << ps_log2);
    const long long entry = (long long)b * max_pages + (ok ? (pos >> ps_log2) : 0);
    const int page = block_tables[entry];
    ok = ok && page >= 0 && page < num_pages;
    const long long page_off = ok ? (long long)page * page_bytes : 0;
    const int range = ok ? page_bytes : 0;
    const int slot = pos & ((1 << ps_log2) - 1);
    const int g = j / kChunks;
    const int c = j - g * kChunks;
    const uint32_t off = lane_ok ? (uint32_t)(((slot * kv_heads + g) * kChunks + c) * 16) : kNoSlot;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(k_cache + page_off, (short)0, range, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(v_cache + page_off, (short)0, range, kBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{kk.x, kk.y, kk.z, kk.w}, rk, (int)off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{vv.x, vv.y, vv.z, vv.w}, rv, (int)off, 0, 0);
}

}  // namespace

hipError_t launch_append(const Plan& pl, const void* new_k, const void* new_v, void* k_cache,
                         void* v_cache, const int32_t* block_tables, const int32_t* positions,
                         hipStream_t stream) {
    const pa_problem& p = pl.prob;
    const int row_chunks = p.kv_heads * (p.head_dim / 8);
    const int threads = append_threads(row_chunks);
    const dim3 grid((unsigned)p.batch, (unsigned)((row_chunks + threads - 1) / threads));
    const dim3 block(threads);
    const auto* nk = static_cast<const uint4*>(new_k);
    const auto* nv = static_cast<const uint4*>(new_v);
    auto* kc = static_cast<char*>(k_cache);
    auto* vc = static_cast<char*>(v_cache);
    const int page_bytes = p.page_size * row_chunks * 16;
    if (p.head_dim == 128)
        hipLaunchKernelGGL(pa_append_kernel<16>, grid, block, 0, stream, nk, nv, kc, vc,
                           block_tables, positions, row_chunks, p.kv_heads, pl.ps_log2,
                           p.max_pages_per_sequence, p.num_physical_pages, page_bytes);
    else
        hipLaunchKernelGGL(pa_append_kernel<8>, grid, block, 0, stream, nk, nv, kc, vc,
                           block_tables, positions, row_chunks, p.kv_heads, pl.ps_log2,
                           p.max_pages_per_sequence, p.num_physical_pages, page_bytes);
    return hipGetLastError();
}

}  // namespace pa
