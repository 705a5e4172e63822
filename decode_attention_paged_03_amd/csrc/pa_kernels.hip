// pa_kernels.hip -- gfx950 (CDNA4) kernels of one paged-attention decode step.
//
// Two routes over the same per-tile arithmetic:
//
//  * Balanced (the default): a resident grid of workgroups splits all token tiles of
//    the batch evenly -- streams (sequence, KV head, head chunk) laid end to end, each
//    workgroup taking an equal run of 16-token tiles, its waves equal sub-runs.  A
//    stream a wave holds entirely is finished there (the single-tile path of the
//    "paged_attention_v2_pytorch.py" commit page); a stream that crosses waves or
//    workgroups leaves (max, sum, acc) triples that are combined in LDS or, across
//    workgroups, by pa_merge_balanced -- the split/merge of the "V4 (Context-axis
//    parallelism)" section of "[TIL] Optimizing paged attention", with the split points
//    chosen for balance instead of fixed.
//  * Fixed partitions (a partition size or a flag given): one workgroup per (sequence,
//    KV head, head chunk, partition of partition_size tokens), partition triples in the
//    workspace, pa_merge_kernel per (sequence, query head) -- p2's PARTITION_SIZE scheme.
//
// Both combine triples as M = max m_p, L = sum exp(m_p - M) l_p,
// out = sum exp(m_p - M) acc_p / L (the V4 merge kernel's combination, with the global
// maximum first and the division once at the end, as the commit page's phase 2 does).
//
// The block-table gather follows the "Baseline" and "V3 (Shared memory data reuse)"
// sections of the first page: token t of a sequence is slot t % page_size of physical
// page block_tables[b][t / page_size]; one K/V read serves every query head of the GQA
// group (V3 stages a page in shared memory for this; here the group is scored from
// registers).  The streaming softmax is that page's Baseline recurrence.
//
// Scores are kept in base-2 units: z = (q . k) * |scale| * log2(e), so every exponential
// is the hardware exp2 (v_exp_f32).  A negative scale is folded into q (sign flip, exact).
//
// Per 16-token tile, one wave does:
//   Q.K^T  with v_mfma_f32_16x16x32_f16: B = the tile's K rows (lane l holds token l%16,
//          dims 32j + 8(l/16) .. +7 for MFMA j), A = the query heads, repeated over the
//          16 MFMA rows so that every lane ends up holding the scores of its column's
//          token for 4 heads.  This is a dense contraction over head_dim (fp16 products,
//          fp32 sums), the one place the matrix cores fit this memory-bound path.
//   softmax: tile max by a DPP max-reduction over the 16 lanes of a row; the reference
//          max of a head only moves (and the accumulators are rescaled) when a tile's max
//          exceeds it by more than kRescaleSlack (2^8), so in steady state a tile costs
//          one exp2 per score and no rescaling.  Any reference value gives the same
//          final ratio acc / l; the slack only bounds how large the weights may grow.
//   P.V    on the VALU: the V rows are loaded with D/8 lanes per token (each lane owns
//          8 dims of the output for every head); the weight of the lane's token is
//          fetched from the score lanes with ds_bpermute; fma_mix multiplies the fp16
//          value by the fp32 weight into fp32 accumulators.
// The next tile's loads (nontemporal, 128-bit) are in flight while a tile is consumed.
#include <hip/hip_runtime.h>

#include <math.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left alone (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, expcnt in 6:4, lgkmcnt in 11:8, vmcnt[5:4] in 15:14)
constexpr int kWaitVmcnt0 = 0x0F70;
// dword 3 of a raw buffer resource on this target, and the nontemporal cache policy bit
constexpr int kBufferFlags = 0x00020000;
constexpr int kLoadNontemporal = 2;
constexpr float kRescaleSlack = 8.0f;   // log2 units
#ifndef PA_BAL_PRIO
#define PA_BAL_PRIO 1   // balanced route: raise the issue priority of waves that fall behind
#endif

struct DecodeArgs {
    const _Float16* q;
    const char* k;          // byte pointers to the caches
    const char* v;
    const int32_t* bt;
    const int32_t* ctx;
    float* out;
    float* ws_acc;          // [batch][query_heads][n_part_max][D]
    float* ws_ml;           // [batch][query_heads][n_part_max][2] = (max in log2 units, sum)
    int4* ws_desc;          // balanced route: per-workgroup merge descriptor
    float scale_log2;       // |scale| * log2(e)
    uint32_t q_sign;        // 0x80008000 to negate q (negative scale), else 0
    int batch, query_heads, kv_heads, group, n_chunks, max_pages, partition, n_part_max, ps_log2;
    int force_split;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    // every lane has a valid source for the patterns used here, so bound_ctrl does not
    // matter; it lets the compiler fold the move into the consuming VALU op
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// All-reduce over each group of 16 consecutive lanes (a DPP row); every lane of the row
// gets the identical result (partners exchange operands; max and + are commutative).
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));    // quad_perm(1,0,3,2)
    x = fmaxf(x, dpp<0x4E>(x));    // quad_perm(2,3,0,1)
    x = fmaxf(x, dpp<0x141>(x));   // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));   // row_mirror
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Issue priority of the calling wave (0..3; s_setprio takes an immediate).  Between
// waves of equal priority a SIMD favours the oldest.
__device__ __forceinline__ void set_wave_priority(int p) {
    if (p >= 3) __builtin_amdgcn_s_setprio(3);
    else if (p == 2) __builtin_amdgcn_s_setprio(2);
    else if (p == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

__device__ __forceinline__ half8_t as_half8(const uint4& x) {
    return __builtin_bit_cast(half8_t, x);
}

__device__ __forceinline__ float lo_half(unsigned int w) {
    return (float)__builtin_bit_cast(half2_t, w).x;
}
__device__ __forceinline__ float hi_half(unsigned int w) {
    return (float)__builtin_bit_cast(half2_t, w).y;
}

__device__ __forceinline__ float readlane_f(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ float readfirst_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

template <int D, int HP>
struct Geo {
    static constexpr int T = 16;           // tokens per wave tile (MFMA N)
    static constexpr int UK = D / 32;      // K loads (and MFMAs) per tile
    static constexpr int LR = D / 8;       // lanes per V row
    static constexpr int NR = 64 / LR;     // V rows (tokens) per load
    static constexpr int UV = T / NR;      // V loads per tile
    static constexpr int C4 = D / 4;       // float4 columns of an output row
    static constexpr int QDUP = HP <= 4 ? 4 : 8;   // MFMA rows i hold head i % QDUP
};

// Lane coordinates inside a wave.
struct Lane {
    int lane, col, grp, vr, vc;
    template <int D>
    __device__ static Lane make(int lane) {
        Lane l;
        l.lane = lane;
        l.col = lane & 15;       // MFMA column (token within the tile)
        l.grp = lane >> 4;       // MFMA row group (k-chunk for operands, 4 rows for D)
        l.vr = lane / (D / 8);   // V row (token within a V load)
        l.vc = lane % (D / 8);   // V chunk (dims 8vc .. 8vc+7)
        return l;
    }
};

// A operand of the score MFMA: head (col % QDUP) of the chunk starting at query row
// `row0`, dims 32j + 8 grp .. +7; zero past HP heads; sign-flipped for a negative scale.
// Split into the loads and the fix-up, so that a prefetch does not wait for its data.
template <int D, int HP>
__device__ __forceinline__ void load_q_raw(const _Float16* q, size_t row0, const Lane& L,
                                           uint4 (&qr)[Geo<D, HP>::UK]) {
    using G = Geo<D, HP>;
    const int hq = L.col % G::QDUP;
    const uint4* qp = reinterpret_cast<const uint4*>(q + (row0 + (hq < HP ? hq : 0)) * D);
#pragma unroll
    for (int j = 0; j < G::UK; ++j) qr[j] = qp[4 * j + L.grp];
}
template <int D, int HP>
__device__ __forceinline__ void fix_q(const uint4 (&qr)[Geo<D, HP>::UK], uint32_t q_sign, const Lane& L,
                                      half8_t (&qa)[Geo<D, HP>::UK]) {
    using G = Geo<D, HP>;
    const bool used = (L.col % G::QDUP) < HP;
#pragma unroll
    for (int j = 0; j < G::UK; ++j) {
        uint4 w = qr[j];
        w.x ^= q_sign; w.y ^= q_sign; w.z ^= q_sign; w.w ^= q_sign;
        if (!used) w = uint4{0u, 0u, 0u, 0u};
        qa[j] = as_half8(w);
    }
}
template <int D, int HP>
__device__ __forceinline__ void load_q(const _Float16* q, size_t row0, uint32_t q_sign, const Lane& L,
                                       half8_t (&qa)[Geo<D, HP>::UK]) {
    uint4 qr[Geo<D, HP>::UK];
    load_q_raw<D, HP>(q, row0, L, qr);
    fix_q<D, HP>(qr, q_sign, L, qa);
}

// A raw buffer resource over `bytes` bytes at `base`.  Loads past `bytes` return zero
// without touching memory (the hardware range check), which is how rows past the valid
// tokens of a tile are kept out of the accumulators.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, kBufferFlags);
}
__device__ __forceinline__ uint4 buf_ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kLoadNontemporal);
    return uint4{t.x, t.y, t.z, t.w};
}

// Loads of one 16-token tile.  `kp`/`vp` point at the K/V row (this KV head) of the
// tile's first token; with pages of 8 the tile's tokens 8..15 sit in the next page,
// whose rows start at `kp2`/`vp2`.  Tokens past n_valid (0..16, wave-uniform) read as
// zero: their scores are masked, and their zero V rows add nothing.
template <int D, int HP, bool SPLIT>
__device__ __forceinline__ void load_kv(const char* kp, const char* vp, const char* kp2, const char* vp2,
                                        uint32_t koff, const uint32_t (&voff)[Geo<D, HP>::UV],
                                        uint32_t tok_bytes, int n_valid, const Lane& L,
                                        uint4 (&kb)[Geo<D, HP>::UK], uint4 (&vb)[Geo<D, HP>::UV]) {
    using G = Geo<D, HP>;
    n_valid = __builtin_amdgcn_readfirstlane(n_valid);   // uniform; keeps the resource in SGPRs
    if constexpr (!SPLIT) {
        const int bytes = n_valid * (int)tok_bytes;
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kp, bytes);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vp, bytes);
#pragma unroll
        for (int j = 0; j < G::UK; ++j) kb[j] = buf_ld(rk, koff + 64 * j);
#pragma unroll
        for (int u = 0; u < G::UV; ++u) vb[u] = buf_ld(rv, voff[u]);
    } else {
        const int n1 = min(n_valid, 8), n2 = max(n_valid - 8, 0);
        const __amdgpu_buffer_rsrc_t rk1 = tile_rsrc(kp, n1 * (int)tok_bytes);
        const __amdgpu_buffer_rsrc_t rk2 = tile_rsrc(kp2, n2 * (int)tok_bytes);
        const __amdgpu_buffer_rsrc_t rv1 = tile_rsrc(vp, n1 * (int)tok_bytes);
        const __amdgpu_buffer_rsrc_t rv2 = tile_rsrc(vp2, n2 * (int)tok_bytes);
        // Columns 0..7 read the first page, 8..15 the next one.  Both loads are issued by
        // every lane with a wave-uniform resource; the lane's offset into the page it does
        // not use is pushed past the resource's range, so that load returns zero and the
        // two results combine with an OR.
        const uint32_t k1 = (L.col < 8) ? koff : 0x7FFFFF00u;
        const uint32_t k2 = (L.col < 8) ? 0x7FFFFF00u : koff - 8 * tok_bytes;
#pragma unroll
        for (int j = 0; j < G::UK; ++j) {
            const uint4 x = buf_ld(rk1, k1 + 64 * j);
            const uint4 y = buf_ld(rk2, k2 + 64 * j);
            kb[j] = uint4{x.x | y.x, x.y | y.y, x.z | y.z, x.w | y.w};
        }
#pragma unroll
        for (int u = 0; u < G::UV; ++u) {
            // V load u covers tile rows u*NR .. u*NR+NR-1, all in one page (NR divides 8)
            if (u * G::NR < 8) vb[u] = buf_ld(rv1, voff[u]);
            else vb[u] = buf_ld(rv2, voff[u] - 8 * tok_bytes);
        }
    }
}

// Streaming softmax state of one wave for HP heads: a reference max per head, kept both
// wave-uniform (mref, for the V layout) and per lane in the score layout (mrow[e] = mref
// of the head in score register e of this lane's row group); running sums in the score
// layout; output accumulators in the V layout (8 dims per lane per head).
template <int D, int HP>
struct WaveState {
    using G = Geo<D, HP>;
    float mref[HP];
    float mrow[4];
    float lsum[4];
    float acc[HP][8];

    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            mref[h] = -INFINITY;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            mrow[e] = -INFINITY;
            lsum[e] = 0.f;
        }
    }

    // One tile: tokens with col >= n_valid are masked (n_valid in 0..16, wave-uniform).
    __device__ __forceinline__ void tile(const half8_t (&qa)[G::UK], const uint4 (&kb)[G::UK],
                                         const uint4 (&vb)[G::UV], int n_valid, float sl2, const Lane& L) {
        float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < G::UK; ++j)
            s = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[j], as_half8(kb[j]), s, 0, 0, 0);
        const bool valid = L.col < n_valid;
        float z[4], zt[4];
        bool grow = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            z[e] = valid ? s[e] * sl2 : -INFINITY;
            zt[e] = row16_max(z[e]);
            grow |= zt[e] > mrow[e] + kRescaleSlack;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // rare: move the reference max
            float mt[HP];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (e < HP) mt[e] = readfirst_f(zt[e]);
                if (HP > 4 && e + 4 < HP) mt[e + 4] = readlane_f(zt[e], 16);
            }
            float alpha[HP];
#pragma unroll
            for (int h = 0; h < HP; ++h) {
                const float mn = fmaxf(mref[h], mt[h]);
                alpha[h] = fast_exp2(mref[h] - mn);    // 0 when mref was -inf
                mref[h] = mn;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[h][j] *= alpha[h];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (HP <= 4) {
                    if (e < HP) {
                        lsum[e] *= alpha[e];
                        mrow[e] = mref[e];
                    }
                } else {
                    const bool hi = (L.grp & 1) != 0;
                    if (e + 4 < HP) {
                        lsum[e] *= hi ? alpha[e + 4] : alpha[e];
                        mrow[e] = hi ? mref[e + 4] : mref[e];
                    } else {
                        lsum[e] *= hi ? 1.f : alpha[e];
                        mrow[e] = hi ? 0.f : mref[e];
                    }
                }
            }
        }
        // weights in the score layout (rows of heads past HP carry unused values)
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] = fast_exp2(z[e] - mrow[e]);
            lsum[e] += p[e];
        }
        // P.V: lane (vr, vc) takes the weight of tile token u*NR + vr from its score lane
#pragma unroll
        for (int u = 0; u < G::UV; ++u) {
            float f[8];
            f[0] = lo_half(vb[u].x); f[1] = hi_half(vb[u].x);
            f[2] = lo_half(vb[u].y); f[3] = hi_half(vb[u].y);
            f[4] = lo_half(vb[u].z); f[5] = hi_half(vb[u].z);
            f[6] = lo_half(vb[u].w); f[7] = hi_half(vb[u].w);
#pragma unroll
            for (int h = 0; h < HP; ++h) {
                const int src_grp = (HP <= 4) ? L.grp : (h >> 2);
                const int src = u * G::NR + L.vr + 16 * src_grp;
                const float w = __builtin_bit_cast(
                    float, __builtin_amdgcn_ds_bpermute(src * 4, __builtin_bit_cast(int, p[h & 3])));
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(w, f[j], acc[h][j]);
            }
        }
    }

    // Sums over the 16 score columns (wave-uniform l per head) and over the V rows
    // (acc in place; every row then holds the full sums).
    __device__ __forceinline__ void reduce(float (&lw)[HP]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float r = row16_sum(lsum[e]);
            if (e < HP) lw[e] = readfirst_f(r);
            if (HP > 4 && e + 4 < HP) lw[e + 4] = readlane_f(r, 16);
        }
#pragma unroll
        for (int off = G::LR; off < 64; off <<= 1) {
#pragma unroll
            for (int h = 0; h < HP; ++h)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[h][j] += __shfl_xor(acc[h][j], off);
        }
    }
};

// ------------------------------------------------------------------------------------
// Fixed-partition route: one workgroup per (sequence, KV head, head chunk, partition).
// ------------------------------------------------------------------------------------

// D: head_dim (64 or 128); HP: query heads per workgroup (1..8); DEPTH: tile buffers per
// wave (DEPTH-1 tiles prefetched); NW: waves per workgroup; SPLIT: page_size < 16, so a
// 16-token tile spans two pages.
template <int D, int HP, int DEPTH, int NW, bool SPLIT>
__global__ void __launch_bounds__(NW * 64)
pa_decode_kernel(DecodeArgs a) {
    using G = Geo<D, HP>;
    constexpr int T = G::T;
    constexpr int C4 = G::C4;

    __shared__ int s_bt[kMaxPartitionPages];
    __shared__ float s_m[NW][HP];
    __shared__ float s_l[NW][HP];
    __shared__ float4_t s_acc[NW][HP][C4];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Lane L = Lane::make<D>(tid & 63);

    // Work item: partitions vary slowest, so every sequence's first (largest) partition
    // is dispatched before any remainder partition.
    int id = blockIdx.x;
    const int chunk = id % a.n_chunks; id /= a.n_chunks;
    const int kvh = id % a.kv_heads;   id /= a.kv_heads;
    const int nb = (int)(gridDim.x / (unsigned)(a.n_chunks * a.kv_heads * a.n_part_max));
    const int b = id % nb;
    const int part = id / nb;

    const int ctx = a.ctx[b];
    const int P = a.partition;
    const int t_begin = part * P;
    const int h0 = kvh * a.group + chunk * HP;
    const size_t row0 = (size_t)b * a.query_heads + h0;   // first output row of this WG

    if (t_begin >= ctx) {
        if (part == 0) {   // empty sequence: defined as a zero output
            for (int i = tid; i < HP * D; i += NW * 64) a.out[row0 * D + i] = 0.f;
        }
        return;
    }
    const int t_end = min(t_begin + P, ctx);
    const int n_part_b = (ctx + P - 1) / P;
    const bool direct = (n_part_b == 1) && !a.force_split;

    // The partition's block-table slice -> LDS.
    const int ps_log2 = a.ps_log2;
    const int pg0 = t_begin >> ps_log2;
    const int npg = ((t_end - 1) >> ps_log2) - pg0 + 1;
    const int32_t* bt_row = a.bt + (size_t)b * a.max_pages + pg0;
    for (int i = tid; i < npg; i += NW * 64) s_bt[i] = bt_row[i];

    half8_t qa[G::UK];
    load_q<D, HP>(a.q, row0, a.q_sign, L, qa);
    __syncthreads();

    const size_t tok_bytes = (size_t)a.kv_heads * D * 2;     // bytes between slots
    const size_t page_bytes = tok_bytes << ps_log2;
    const char* kbase = a.k + (size_t)kvh * D * 2;
    const char* vbase = a.v + (size_t)kvh * D * 2;
    const uint32_t koff = (uint32_t)(L.col * tok_bytes) + 16u * L.grp;   // + 64 j
    uint32_t voff[G::UV];
#pragma unroll
    for (int u = 0; u < G::UV; ++u) voff[u] = (uint32_t)((u * G::NR + L.vr) * tok_bytes) + 16u * L.vc;
    const float sl2 = a.scale_log2;

    WaveState<D, HP> st;
    st.reset();

    const int n_tok = t_end - t_begin;
    const int n_tiles = (n_tok + T - 1) / T;
    // This wave takes tiles wave, wave + NW, ...
    const int nk = wave < n_tiles ? (n_tiles - wave + NW - 1) / NW : 0;

    auto load_tile = [&](int k, uint4 (&kb)[G::UK], uint4 (&vb)[G::UV]) {
        const int t0 = t_begin + (wave + k * NW) * T;
        const int pg = (t0 >> ps_log2) - pg0;
        const int phys = __builtin_amdgcn_readfirstlane(s_bt[pg]);
        const size_t base = (size_t)phys * page_bytes + (size_t)(t0 & ((1 << ps_log2) - 1)) * tok_bytes;
        size_t base2 = base;
        if constexpr (SPLIT) {
            // tokens 8..15 of the tile sit in the next page, which exists only when the
            // tile reaches past token 8
            if (t0 + 8 < t_end) base2 = (size_t)__builtin_amdgcn_readfirstlane(s_bt[pg + 1]) * page_bytes;
        }
        load_kv<D, HP, SPLIT>(kbase + base, vbase + base, kbase + base2, vbase + base2, koff, voff,
                              (uint32_t)tok_bytes, max(0, min(T, t_end - t0)), L, kb, vb);
    };

    if (nk > 0) {
        // DEPTH register buffers; tile k + DEPTH - 1 is loaded before tile k is consumed.
        // The loop runs a multiple of DEPTH tiles and has no exit in its middle, so the
        // compiler's wait-count bookkeeping sees the same outstanding loads on every path
        // into the loop header.  Padding tiles (k >= nk) reload the last tile (already in
        // the caches) and are fully masked, which leaves the state unchanged.  The
        // scheduling barriers keep the compiler from sinking the loads below the
        // arithmetic of the tile before them.
        uint4 kb[DEPTH][G::UK], vb[DEPTH][G::UV];
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) load_tile(min(d, nk - 1), kb[d], vb[d]);
        for (int k = 0; k < nk; k += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int nxt = (d + DEPTH - 1) % DEPTH;
                load_tile(min(k + d + DEPTH - 1, nk - 1), kb[nxt], vb[nxt]);
                __builtin_amdgcn_sched_barrier(0);
                const int t0 = t_begin + (wave + (k + d) * NW) * T;
                st.tile(qa, kb[d], vb[d], max(0, min(T, t_end - t0)), sl2, L);
            }
        }
    }

    float lw[HP];
    st.reduce(lw);
    if (L.lane < G::LR) {
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            s_acc[wave][h][2 * L.vc] = float4_t{st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]};
            s_acc[wave][h][2 * L.vc + 1] = float4_t{st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]};
            if (L.lane == 0) {
                s_m[wave][h] = st.mref[h];
                s_l[wave][h] = lw[h];
            }
        }
    }
    __syncthreads();

    // Combine the NW wave states; wave 0 saw token t_begin, so M is finite and waves
    // without tokens (mref = -inf, l = 0, acc = 0) weigh 0.
    for (int idx = tid; idx < HP * C4; idx += NW * 64) {
        const int h = idx / C4;
        const int d4 = idx - h * C4;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
        float Ls = 0.f;
        float4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float e = fast_exp2(s_m[w][h] - M);
            Ls += e * s_l[w][h];
            o += e * s_acc[w][h][d4];
        }
        const size_t row = row0 + h;
        if (direct) {
            reinterpret_cast<float4_t*>(a.out + row * D)[d4] = o / Ls;
        } else {
            const size_t slot = row * a.n_part_max + part;
            reinterpret_cast<float4_t*>(a.ws_acc + slot * D)[d4] = o;
            if (d4 == 0) {
                a.ws_ml[slot * 2] = M;
                a.ws_ml[slot * 2 + 1] = Ls;
            }
        }
    }
}

struct MergeArgs {
    const int32_t* ctx;
    const float* ws_acc;
    const float* ws_ml;
    float* out;
    int query_heads, partition, n_part_max, force_split;
};

constexpr int kMergeThreads = 256;

// Combination of n (max, sum, acc) triples of one output row: out = sum_p e_p acc_p /
// sum_p e_p l_p with e_p = exp2(m_p - max m).  Triple p is row r(p) of the workspace
// (max, sum at ws_ml[2 r], acc at ws_acc[D r]) with r(0) = row_first and
// r(p) = row_rest + (p - 1) * stride.  One pass: thread (g, c) folds the triples
// p = g, g + GR, ... for float4 column c into a running triple, rescaling whenever its
// maximum grows; the GR partial triples are then combined through LDS.  Every thread of
// the block takes part.  Every triple has a finite maximum (it covers >= 1 token).
template <int D>
__device__ __forceinline__ void combine_rows(const float* ws_ml, const float* ws_acc, size_t row_first,
                                             size_t row_rest, size_t stride, int n, float* out_row) {
    constexpr int C4 = D / 4;                       // float4 columns
    constexpr int GR = kMergeThreads / C4;          // triple groups
    constexpr int UNR = 16;
    __shared__ float s_gm[GR];
    __shared__ float s_gl[GR];
    __shared__ float4_t s_go[GR][C4];
    const int tid = threadIdx.x;
    const int c = tid % C4;
    const int g = tid / C4;
    float m = -INFINITY, l = 0.f;
    float4_t o = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = g; p0 < n; p0 += GR * UNR) {
        float4_t av[UNR];
        float2 mv[UNR];
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const int p = p0 + k * GR;
            if (p < n) {
                const size_t r = p == 0 ? row_first : row_rest + (size_t)(p - 1) * stride;
                av[k] = reinterpret_cast<const float4_t*>(ws_acc + r * D)[c];
                mv[k] = reinterpret_cast<const float2*>(ws_ml)[r];
            } else {
                av[k] = float4_t{0.f, 0.f, 0.f, 0.f};
                mv[k] = make_float2(-INFINITY, 0.f);
            }
        }
        float mb = m;
#pragma unroll
        for (int k = 0; k < UNR; ++k) mb = fmaxf(mb, mv[k].x);
        if (mb != -INFINITY) {
            const float a0 = fast_exp2(m - mb);     // 0 while nothing was folded in yet
            l *= a0;
            o *= a0;
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const float e = fast_exp2(mv[k].x - mb);
                l += e * mv[k].y;
                o += e * av[k];
            }
            m = mb;
        }
    }
    if (c == 0) {
        s_gm[g] = m;
        s_gl[g] = l;
    }
    s_go[g][c] = o;
    __syncthreads();
    if (tid < C4) {
        float M = s_gm[0];
#pragma unroll
        for (int k = 1; k < GR; ++k) M = fmaxf(M, s_gm[k]);
        float4_t O = {0.f, 0.f, 0.f, 0.f};
        float L = 0.f;
#pragma unroll
        for (int k = 0; k < GR; ++k) {
            const float e = fast_exp2(s_gm[k] - M);   // 0 for a group without triples
            L += e * s_gl[k];
            O += e * s_go[k][tid];
        }
        reinterpret_cast<float4_t*>(out_row)[tid] = O / L;
    }
    __syncthreads();   // the shared arrays are reused by the next call
}

// One workgroup per (sequence, query head) of the fixed-partition route.
template <int D>
__global__ void __launch_bounds__(kMergeThreads)
pa_merge_kernel(MergeArgs a) {
    const int bh = blockIdx.x;
    const int b = bh / a.query_heads;
    const int ctx = a.ctx[b];
    const int n = (ctx + a.partition - 1) / a.partition;
    if (n == 0 || (n == 1 && !a.force_split)) return;   // written by the decode kernel
    const size_t r0 = (size_t)bh * a.n_part_max;
    combine_rows<D>(a.ws_ml, a.ws_acc, r0, r0 + 1, 1, n, a.out + (size_t)bh * D);
}

// ------------------------------------------------------------------------------------
// Balanced route: one resident workgroup per CU splits all token tiles evenly.
//
// A stream is one (sequence b, KV head, head chunk): ceil(ctx_b / 16) tiles.  The
// streams are laid end to end in the order (b, KV head, chunk); workgroup w takes the
// tiles [w N / W, (w+1) N / W) of the N in total, and its NW waves split that range into
// NW contiguous pieces.  A wave walks its piece tile by tile across stream boundaries,
// with one tile (or DEPTH - 1 tiles ahead) in flight: many waves per CU, each with little
// in flight, keep the memory system fuller than few waves with deep queues.
// A stream that lies wholly inside one wave is finished by that wave (the single-pass
// case); pieces of a stream that crosses waves are combined in LDS at the end of the
// workgroup, and a stream that crosses workgroups leaves one (max, sum, acc) triple per
// workgroup in the workspace for the merge kernel.
// ------------------------------------------------------------------------------------

// Lengths -> LDS, exclusive prefix sums of tiles per sequence.  Every thread of the
// block calls it; returns the total tile count of one (KV head, chunk) plane.
template <int NT>
__device__ __forceinline__ int tile_prefix(const int32_t* ctx, int B, int* s_pref, int* s_ctx, int* s_wsum) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    constexpr int NWV = NT / 64;
    const int per = (B + NT - 1) / NT;
    const int i0 = min(B, tid * per);
    const int i1 = min(B, i0 + per);
    int mine = 0;
    for (int i = i0; i < i1; ++i) {
        const int c = ctx[i];
        s_ctx[i] = c;
        mine += (c + 15) >> 4;
    }
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        const int v = s_wsum[w];
        if (w < wave) before += v;
        total += v;
    }
    int run = before + incl - mine;
    for (int i = i0; i < i1; ++i) {
        s_pref[i] = run;
        run += (s_ctx[i] + 15) >> 4;
    }
    if (tid == 0) s_pref[B] = total;
    __syncthreads();
    return total;
}

// Stream position of global tile t (0 <= t < N): sequence b (the smallest with
// KC * pref[b+1] > t), stream index within the sequence sidx = kvh * n_chunks + chunk,
// tile lt in the stream.  The host keeps N below 2^31.
__device__ __forceinline__ void locate_tile(int t, int B, int KC, const int* s_pref, int& b, int& sidx, int& lt) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (KC * s_pref[mid + 1] > t) hi = mid;
        else lo = mid + 1;
    }
    b = lo;
    const int Tb = s_pref[b + 1] - s_pref[b];
    const int off = t - KC * s_pref[b];
    sidx = off / Tb;
    lt = off - sidx * Tb;
}

// floor(x * N / W) for 0 <= x <= W.  Exact in double: x N < 2^53 is represented exactly,
// and a quotient that is not an integer lies at least 1/W below the next integer, far
// more than the rounding error of the (correctly rounded) division.
__device__ __forceinline__ int split_point(int x, int N, int W) {
    return (int)floor((double)x * (double)N / (double)W);
}

template <int D, int HP, int DEPTH, int NW, bool SPLIT>
__global__ void __launch_bounds__(NW * 64)
pa_decode_balanced(DecodeArgs a) {
    using G = Geo<D, HP>;
    constexpr int T = G::T;
    constexpr int C4 = G::C4;
    constexpr int NT = NW * 64;
    constexpr int NS = 2 * NW;       // partial slots: a wave's first and last segment
    static_assert(NS <= 64, "slot runs are found by one wave");

    extern __shared__ int s_dyn[];
    __shared__ int s_wsum[NW];
    __shared__ float s_m[NS][HP];
    __shared__ float s_l[NS][HP];
    __shared__ float4_t s_acc[NS][HP][C4];
    __shared__ int s_meta[NS][3];    // stream id (-1: empty), first tile, end tile (global)
    __shared__ int s_runs[NS + 1];   // first slot of each run of one stream's slots, then NS
    __shared__ int s_nruns;

    const int B = a.batch;
    int* s_pref = s_dyn;             // [B + 1]
    int* s_ctx = s_dyn + B + 1;      // [B]
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Lane L = Lane::make<D>(tid & 63);

    if (tid < NS) s_meta[tid][0] = -1;
    const int plane = tile_prefix<NT>(a.ctx, B, s_pref, s_ctx, s_wsum);

    // empty sequences: a zero output, written by one workgroup each
    for (int b = blockIdx.x; b < B; b += gridDim.x)
        if (s_ctx[b] == 0)
            for (int i = tid; i < a.query_heads * D; i += NT) a.out[(size_t)b * a.query_heads * D + i] = 0.f;

    const int KC = a.kv_heads * a.n_chunks;
    const int N = KC * plane;
    const int NWG = gridDim.x;
    const int w = blockIdx.x;
    const int g0 = split_point(w, N, NWG);
    const int g1 = split_point(w + 1, N, NWG);
    const int wr0 = g0 + (int)((long long)(g1 - g0) * wave / NW);
    const int wr1 = g0 + (int)((long long)(g1 - g0) * (wave + 1) / NW);
    const int nk = wr1 - wr0;

    const int ps_log2 = a.ps_log2;
    const size_t tok_bytes = (size_t)a.kv_heads * D * 2;
    const size_t page_bytes = tok_bytes << ps_log2;
    const uint32_t koff = (uint32_t)(L.col * tok_bytes) + 16u * L.grp;   // + 64 j
    uint32_t voff[G::UV];
#pragma unroll
    for (int u = 0; u < G::UV; ++u) voff[u] = (uint32_t)((u * G::NR + L.vr) * tok_bytes) + 16u * L.vc;
    const float sl2 = a.scale_log2;

    // Physical pages of the wave's tiles, 64 at a time: lane i holds the page of tile
    // (wr0 + batch + i) (and, for pages of 8, the page of its second half).
    int btv = 0, btv2 = 0;
    auto load_pages = [&](int batch) {
        const int t = wr0 + batch + L.lane;
        if (t < wr1) {
            int b, sidx, lt;
            locate_tile(t, B, KC, s_pref, b, sidx, lt);
            const int tok = lt * T;
            const int32_t* row = a.bt + (size_t)b * a.max_pages;
            btv = row[tok >> ps_log2];
            if constexpr (SPLIT) btv2 = (tok + 8 < s_ctx[b]) ? row[(tok >> ps_log2) + 1] : btv;
        }
        // Wait here for the page gather (and whatever loads precede it): otherwise the
        // compiler, seeing this conditional reload, assumes it may be in flight at every
        // tile and drains all loads before each tile's page lookup.  This path runs once
        // per 64 tiles.
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };

    // A wave-uniform cursor over the tiles to load, and the description of a loaded tile.
    struct Desc {
        int b, sidx, lt, T, n_valid;
        bool first;   // the tile opens a segment of this wave (its first, or a stream start)
    };
    // cursor: sequence cb, stream index cs, tile cl of cT tiles, sequence length cctx,
    // KV head ckvh of the stream (all wave-uniform)
    int cb = 0, cs = 0, cl = 0, cT = 1, cctx = 0, ckvh = 0;
    if (nk > 0) {
        locate_tile(wr0, B, KC, s_pref, cb, cs, cl);
        cb = __builtin_amdgcn_readfirstlane(cb);
        cs = __builtin_amdgcn_readfirstlane(cs);
        cl = __builtin_amdgcn_readfirstlane(cl);
        cT = __builtin_amdgcn_readfirstlane(s_pref[cb + 1] - s_pref[cb]);
        cctx = __builtin_amdgcn_readfirstlane(s_ctx[cb]);
        ckvh = cs / a.n_chunks;
        load_pages(0);
    }
    auto advance = [&]() {
        if (++cl == cT) {
            cl = 0;
            if (++cs == KC) {
                cs = 0;
                do {
                    ++cb;
                } while (cb < B && s_pref[cb + 1] == s_pref[cb]);
                if (cb >= B) cb = B - 1;    // past the last tile; never loaded
                cT = __builtin_amdgcn_readfirstlane(s_pref[cb + 1] - s_pref[cb]);
                cctx = __builtin_amdgcn_readfirstlane(s_ctx[cb]);
            }
            ckvh = cs / a.n_chunks;
        }
    };
    // Load tile i of the wave (i < nk) with the cursor at it into (kb, vb); when it opens
    // a segment, the segment's query rows come with it (into qb), so a new stream costs
    // no extra round trip.
    auto load_tile = [&](int i, Desc& d, uint4 (&kb)[G::UK], uint4 (&vb)[G::UV], uint4 (&qb)[G::UK]) {
        if ((i & 63) == 0 && i > 0) load_pages(i);
        const int kvh = ckvh;
        const int tok = cl * T;
        d.b = cb;
        d.sidx = cs;
        d.lt = cl;
        d.T = cT;
        d.n_valid = min(T, cctx - tok);
        d.first = (i == 0) || (cl == 0);
        const int phys = __builtin_amdgcn_readlane(btv, i & 63);
        const size_t base = (size_t)phys * page_bytes + (size_t)(tok & ((1 << ps_log2) - 1)) * tok_bytes;
        size_t base2 = base;
        if constexpr (SPLIT) base2 = (size_t)__builtin_amdgcn_readlane(btv2, i & 63) * page_bytes;
        const char* kbase = a.k + (size_t)kvh * D * 2;
        const char* vbase = a.v + (size_t)kvh * D * 2;
        load_kv<D, HP, SPLIT>(kbase + base, vbase + base, kbase + base2, vbase + base2, koff, voff,
                              (uint32_t)tok_bytes, d.n_valid, L, kb, vb);
        if (d.first) {
            const int chunk = cs - kvh * a.n_chunks;
            load_q_raw<D, HP>(a.q, (size_t)cb * a.query_heads + kvh * a.group + chunk * HP, L, qb);
        }
    };

    WaveState<D, HP> st;
    half8_t qa[G::UK];
    int seg_lt0 = 0;       // first stream tile of the open segment
    int seg_i0 = 0;        // first wave tile of the open segment
    auto consume = [&](const Desc& d, const uint4 (&kb)[G::UK], const uint4 (&vb)[G::UV],
                       const uint4 (&qb)[G::UK], int i) {
        if (d.first) {   // a new segment: its query rows and a fresh state
            fix_q<D, HP>(qb, a.q_sign, L, qa);
            seg_lt0 = d.lt;
            seg_i0 = i;
            st.reset();
        }
        st.tile(qa, kb, vb, d.n_valid, sl2, L);
        if (d.lt == d.T - 1 || i == nk - 1) {   // the segment ends here
            const int kvh = d.sidx / a.n_chunks;
            const int chunk = d.sidx - kvh * a.n_chunks;
            const size_t row0 = (size_t)d.b * a.query_heads + kvh * a.group + chunk * HP;
            float lw[HP];
            st.reduce(lw);
            if (seg_lt0 == 0 && d.lt == d.T - 1) {
                // the whole stream: finish it
                if (L.lane < G::LR) {
#pragma unroll
                    for (int h = 0; h < HP; ++h) {
                        float4_t* o = reinterpret_cast<float4_t*>(a.out + (row0 + h) * D) + 2 * L.vc;
                        const float r = 1.f / lw[h];
                        o[0] = float4_t{st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]} * r;
                        o[1] = float4_t{st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]} * r;
                    }
                }
            } else {
                // a piece of a stream that continues in another wave: slot 2 wave for the
                // wave's first segment, 2 wave + 1 for its last one
                const int slot = 2 * wave + (seg_i0 == 0 ? 0 : 1);
                if (L.lane < G::LR) {
#pragma unroll
                    for (int h = 0; h < HP; ++h) {
                        s_acc[slot][h][2 * L.vc] = float4_t{st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]};
                        s_acc[slot][h][2 * L.vc + 1] = float4_t{st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]};
                    }
                    if (L.lane == 0) {
#pragma unroll
                        for (int h = 0; h < HP; ++h) {
                            s_m[slot][h] = st.mref[h];
                            s_l[slot][h] = lw[h];
                        }
                        s_meta[slot][0] = d.b * KC + d.sidx;
                        s_meta[slot][1] = wr0 + seg_i0;
                        s_meta[slot][2] = wr0 + i + 1;
                    }
                }
            }
        }
    };

    if (nk > 0) {
        // DEPTH register buffers: tile i + DEPTH - 1 is loaded before tile i is consumed.
        // The loop runs a multiple of DEPTH tiles and has no exit in its middle (see the
        // fixed route); a padding tile (i >= nk) repeats the last load and is not
        // consumed.
        uint4 kb[DEPTH][G::UK], vb[DEPTH][G::UV];
        uint4 qb[DEPTH][G::UK];
        Desc dsc[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) {
            if (d > 0 && d < nk) advance();
            load_tile(min(d, nk - 1), dsc[d], kb[d], vb[d], qb[d]);
        }
        // The waves of a workgroup have equal work, but a SIMD serves its oldest wave
        // first, so the youngest would finish last with the CU's other waves idle.  A
        // wave's priority is therefore the quarter of its range it has left: a wave
        // that has fallen behind is served first.
        const int q1 = nk / 4, q2 = nk / 2, q3 = (3 * nk) / 4;
        int prio = -1;
        for (int i = 0; i < nk; i += DEPTH) {
            if (PA_BAL_PRIO) {
                const int left = nk - i;
                const int p = (left > q3) + (left > q2) + (left > q1);
                if (p != prio) {
                    set_wave_priority(p);
                    prio = p;
                }
            }
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int nxt = (d + DEPTH - 1) % DEPTH;
                const int inext = i + d + DEPTH - 1;
                if (inext > 0 && inext < nk) advance();
                load_tile(min(inext, nk - 1), dsc[nxt], kb[nxt], vb[nxt], qb[nxt]);
                __builtin_amdgcn_sched_barrier(0);
                if (DEPTH == 1 || i + d < nk) consume(dsc[d], kb[d], vb[d], qb[d], i + d);
                else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // see below
            }
        }
        // (The skipped padding tile's loads are waited for on the spot -- this happens
        // only at the very end -- so that no path reaches the loop header with loads
        // outstanding into registers the compiler may reuse; otherwise it inserts waits
        // into every iteration.)
        if (PA_BAL_PRIO) set_wave_priority(0);
    }
    __syncthreads();

    // Runs of slots: the non-empty slots of one stream are adjacent (slots are in tile
    // order and a stream's tiles are contiguous).  Wave 0 finds where each run starts;
    // meanwhile the last wave writes the workgroup's merge descriptor.
    if (wave == 0) {
        const int lane = L.lane;
        const int sid = lane < NS ? s_meta[lane][0] : -1;
        int last = sid;   // stream of the nearest non-empty slot at or below this one
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(last, off);
            if (last < 0 && lane >= off) last = y;
        }
        int prev = __shfl_up(last, 1);
        if (lane == 0) prev = -1;
        const bool start = sid >= 0 && sid != prev;
        const uint64_t bal = __builtin_amdgcn_ballot_w64(start);
        const int idx = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        const int nr = __popcll(bal);
        if (start) s_runs[idx] = lane;
        if (lane == 0) {
            s_runs[nr] = NS;
            s_nruns = nr;
        }
    }
    if (wave == NW - 1 && L.lane == 0) {
        // The stream holding the last tile, if it starts here and goes on, is merged by
        // the merge kernel's blocks of this workgroup: {first output row, pieces, the
        // workspace row of the first piece}.
        int4 desc = {0, 0, 0, 0};
        if (g1 > g0) {
            int b, sidx, lt;
            locate_tile(g1 - 1, B, KC, s_pref, b, sidx, lt);
            const int Tb = s_pref[b + 1] - s_pref[b];
            const int S = KC * s_pref[b] + sidx * Tb;
            const int E = S + Tb;
            if (E > g1 && S >= g0) {
                // last workgroup the stream reaches: the largest x with split(x) <= E - 1,
                // i.e. floor((E W - 1) / N) (exact in double, as for split_point)
                int wl = (int)floor(((double)E * (double)NWG - 1.0) / (double)N);
                wl = min(wl, NWG - 1);
                const int kvh = sidx / a.n_chunks;
                const int chunk = sidx - kvh * a.n_chunks;
                desc.x = b * a.query_heads + kvh * a.group + chunk * HP;
                desc.y = wl - w + 1;
                desc.z = (w * 2 + (S == g0 ? 0 : 1)) * HP;
            }
        }
        a.ws_desc[w] = desc;
    }
    if (g1 == g0) {
        // no tiles: an empty triple (weight 0) for a merge whose stream spans this
        // workgroup's (empty) range
        const size_t wslot = (size_t)w * 2 * HP;
        for (int idx = tid; idx < HP * C4; idx += NT) {
            const int h = idx / C4;
            const int d4 = idx - h * C4;
            reinterpret_cast<float4_t*>(a.ws_acc + (wslot + h) * D)[d4] = float4_t{0.f, 0.f, 0.f, 0.f};
            if (d4 == 0) {
                a.ws_ml[(wslot + h) * 2] = -INFINITY;
                a.ws_ml[(wslot + h) * 2 + 1] = 0.f;
            }
        }
    }
    __syncthreads();

    // Combine each run: HP * C4 threads per run, as many runs at once as the block holds.
    // A stream covered entirely is finished; otherwise it crosses a workgroup boundary and
    // its triple goes to the workspace: slot 0 for the stream holding the workgroup's
    // first tile, slot 1 for the one holding its last tile.
    constexpr int PER = HP * C4;
    constexpr int RPAR = NT / PER;
    static_assert(RPAR >= 1, "a run needs HP * D / 4 threads");
    const int nr = s_nruns;
    const int rsub = tid / PER;
    if (rsub < RPAR) {
        const int e = tid - rsub * PER;
        const int h = e / C4;
        const int d4 = e - h * C4;
        for (int r = rsub; r < nr; r += RPAR) {
            const int s0 = s_runs[r], s1 = s_runs[r + 1];
            const int sid = s_meta[s0][0];
            const int tb = s_meta[s0][1];
            int te = s_meta[s0][2];
            float M = -INFINITY;
            for (int s = s0; s < s1; ++s)
                if (s_meta[s][0] >= 0) {
                    M = fmaxf(M, s_m[s][h]);
                    te = s_meta[s][2];
                }
            float Ls = 0.f;
            float4_t o = {0.f, 0.f, 0.f, 0.f};
            for (int s = s0; s < s1; ++s)
                if (s_meta[s][0] >= 0) {
                    const float f = fast_exp2(s_m[s][h] - M);
                    Ls += f * s_l[s][h];
                    o += f * s_acc[s][h][d4];
                }
            const int b = sid / KC;
            const int sidx = sid - b * KC;
            const int Tb = s_pref[b + 1] - s_pref[b];
            const int S = KC * s_pref[b] + sidx * Tb;
            const int kvh = sidx / a.n_chunks;
            const int chunk = sidx - kvh * a.n_chunks;
            const size_t row0 = (size_t)b * a.query_heads + kvh * a.group + chunk * HP;
            if (tb == S && te == S + Tb) {
                reinterpret_cast<float4_t*>(a.out + (row0 + h) * D)[d4] = o / Ls;
            } else {
                const size_t wslot = ((size_t)w * 2 + (tb == g0 ? 0 : 1)) * HP;
                reinterpret_cast<float4_t*>(a.ws_acc + (wslot + h) * D)[d4] = o;
                if (d4 == 0) {
                    a.ws_ml[(wslot + h) * 2] = M;
                    a.ws_ml[(wslot + h) * 2 + 1] = Ls;
                }
            }
        }
    }
}

// Merge of the balanced route: block (w, h) combines head h of the stream that the
// decode kernel's workgroup w owns (the stream holding w's last tile, when it starts in
// w and continues past it, so each crossing stream has exactly one owner).  The decode
// kernel leaves per workgroup a descriptor {first output row, number of pieces, workspace
// row of the first piece}; the pieces are slot 1 of w (slot 0 if the stream is also w's
// first) and slot 0 of each following workgroup it reaches, 2 * HP rows apart.
template <int D, int HP>
__global__ void __launch_bounds__(kMergeThreads)
pa_merge_balanced(DecodeArgs a) {
    const int w = blockIdx.x / HP;
    const int h = blockIdx.x - w * HP;
    const int4 d = a.ws_desc[w];
    if (d.y <= 0) return;
    combine_rows<D>(a.ws_ml, a.ws_acc, (size_t)d.z + h, ((size_t)w + 1) * 2 * HP + h, 2 * HP, d.y,
                    a.out + ((size_t)d.x + h) * D);
}

#ifndef PA_WAVES
#define PA_WAVES 4   // waves per decode workgroup
#endif
#ifndef PA_DEPTH
#define PA_DEPTH 2   // tile buffers per wave (fixed route)
#endif
constexpr int kWaves = PA_WAVES;
constexpr int kDepth = PA_DEPTH;

// Workgroups of a kernel that are resident at once on this device (CUs x blocks per CU),
// capped at kMaxBalancedWG.  Host-side queries only; nothing is enqueued.
template <typename K>
int resident_grid(K kernel, int block, size_t lds) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, block, lds) != hipSuccess) return 0;
    const long long g = (long long)cus * (per > 0 ? per : 1);
    return (int)(g < kMaxBalancedWG ? g : kMaxBalancedWG);
}

#ifndef PA_BAL_WAVES
#define PA_BAL_WAVES 12  // waves per balanced workgroup (one workgroup per CU)
#endif
#ifndef PA_BAL_DEPTH
#define PA_BAL_DEPTH 1   // tile buffers per wave (balanced route)
#endif
constexpr int kBalWaves = PA_BAL_WAVES;
constexpr int kBalDepth = PA_BAL_DEPTH;

template <int D, int HP, bool SPLIT>
hipError_t launch_balanced(const Plan& pl, const DecodeArgs& args, hipStream_t stream) {
    // 12 waves (3 per SIMD) fit the register budget up to 6 heads (4 with pages of 8);
    // more heads take 8 waves
    constexpr int NW = (HP <= 4 || (HP <= 6 && !SPLIT)) ? kBalWaves : 8;
    const auto kern = pa_decode_balanced<D, HP, kBalDepth, NW, SPLIT>;
    const size_t lds = (size_t)(2 * pl.prob.batch + 1) * sizeof(int);
    const int grid = resident_grid(kern, NW * 64, lds);
    if (grid <= 0) return hipErrorInvalidDevice;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), lds, stream, args);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((pa_merge_balanced<D, HP>), dim3((unsigned)(grid * HP)), dim3(kMergeThreads), 0,
                       stream, args);
    return hipGetLastError();
}

template <int D, int HP>
hipError_t launch_decode(const Plan& pl, const DecodeArgs& args, hipStream_t stream) {
    const bool split = pl.prob.page_size < 16;
    if (pl.balanced)
        return split ? launch_balanced<D, HP, true>(pl, args, stream) : launch_balanced<D, HP, false>(pl, args, stream);
    if (!split)
        hipLaunchKernelGGL((pa_decode_kernel<D, HP, kDepth, kWaves, false>),
                           dim3((unsigned)pl.decode_grid), dim3(kWaves * 64), 0, stream, args);
    else
        hipLaunchKernelGGL((pa_decode_kernel<D, HP, kDepth, kWaves, true>),
                           dim3((unsigned)pl.decode_grid), dim3(kWaves * 64), 0, stream, args);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const Plan& pl, const DecodeArgs& args, hipStream_t stream) {
    switch (pl.heads_per_wg) {
        case 1: return launch_decode<D, 1>(pl, args, stream);
        case 2: return launch_decode<D, 2>(pl, args, stream);
        case 3: return launch_decode<D, 3>(pl, args, stream);
        case 4: return launch_decode<D, 4>(pl, args, stream);
        case 5: return launch_decode<D, 5>(pl, args, stream);
        case 6: return launch_decode<D, 6>(pl, args, stream);
        case 7: return launch_decode<D, 7>(pl, args, stream);
        case 8: return launch_decode<D, 8>(pl, args, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch(const Plan& pl, const void* q, const void* k, const void* v,
                  const int32_t* block_tables, const int32_t* ctx, float scale, float* out,
                  void* workspace, hipStream_t stream) {
    const pa_problem& p = pl.prob;
    float* ws_acc = nullptr;
    float* ws_ml = nullptr;
    int4* ws_desc = nullptr;
    if (pl.need_merge) {
        ws_acc = static_cast<float*>(workspace);
        ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ws_ml_offset);
        if (pl.balanced) ws_desc = reinterpret_cast<int4*>(static_cast<char*>(workspace) + pl.ws_desc_offset);
    }
    DecodeArgs da;
    da.q = static_cast<const _Float16*>(q);
    da.k = static_cast<const char*>(k);
    da.v = static_cast<const char*>(v);
    da.bt = block_tables;
    da.ctx = ctx;
    da.out = out;
    da.ws_acc = ws_acc;
    da.ws_ml = ws_ml;
    da.ws_desc = ws_desc;
    da.scale_log2 = fabsf(scale) * kLog2e;
    da.q_sign = scale < 0.f ? 0x80008000u : 0u;
    da.batch = p.batch;
    da.query_heads = p.query_heads;
    da.kv_heads = p.kv_heads;
    da.group = pl.group;
    da.n_chunks = pl.n_chunks;
    da.max_pages = p.max_pages_per_sequence;
    da.partition = pl.partition;
    da.n_part_max = pl.n_part_max;
    da.ps_log2 = pl.ps_log2;
    da.force_split = pl.force_split ? 1 : 0;

    hipError_t err = (p.head_dim == 128) ? launch_decode_d<128>(pl, da, stream)
                                         : launch_decode_d<64>(pl, da, stream);
    if (err != hipSuccess || pl.balanced || !pl.need_merge) return err;

    MergeArgs ma;
    ma.ctx = ctx;
    ma.ws_acc = ws_acc;
    ma.ws_ml = ws_ml;
    ma.out = out;
    ma.query_heads = p.query_heads;
    ma.partition = pl.partition;
    ma.n_part_max = pl.n_part_max;
    ma.force_split = da.force_split;
    if (p.head_dim == 128)
        hipLaunchKernelGGL(pa_merge_kernel<128>, dim3((unsigned)pl.merge_grid), dim3(kMergeThreads), 0,
                           stream, ma);
    else
        hipLaunchKernelGGL(pa_merge_kernel<64>, dim3((unsigned)pl.merge_grid), dim3(kMergeThreads), 0,
                           stream, ma);
    return hipGetLastError();
}

}  // namespace pa
