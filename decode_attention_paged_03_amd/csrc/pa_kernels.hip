// pa_kernels.hip -- gfx950 (CDNA4) kernels of one paged-attention decode step.
//
// Two routes over the same per-tile arithmetic:
//
//  * Balanced (the default): a resident grid, one workgroup per CU, splits all token
//    tiles of the batch evenly.  A sequence's streams (KV head, head chunk) are grouped in
//    bands of `spw` streams that are read side by side: the waves of a workgroup take
//    different streams of the same token range, so that a CU reads neighbouring row
//    offsets of a page (the KV heads of a token sit next to each other) and the memory
//    channels are loaded evenly.  (The plan halves spw when the batch holds few bands;
//    each band then spans many workgroups and fewer rows per band make its merge
//    cheaper.)  Bands are laid end to end; workgroup w takes the units
//    [w N / W, (w+1) N / W) of the N (band, 16-token tile) units, and the waves reading
//    one stream split that range in runs, the earlier rounds of waves taking somewhat
//    more (they are issued first).  A stream that a wave holds entirely is
//    finished there (the single-tile path of the "paged_attention_v2_pytorch.py" commit
//    page); pieces of a stream that crosses waves are combined in LDS, and pieces that
//    cross workgroups leave (max, sum, acc) triples for pa_merge_balanced -- the
//    split/merge of the "V4 (Context-axis parallelism)" section of "[TIL] Optimizing
//    paged attention", with the split points chosen for balance instead of fixed.
//  * Fixed partitions (a partition size or a flag given): one workgroup per (sequence,
//    KV head, head chunk, partition of partition_size tokens), partition triples in the
//    workspace, pa_merge_kernel per (sequence, query head) -- the PARTITION_SIZE scheme of
//    the "paged_attention_v2_pytorch.py" commit page.  When the host's bound keeps every
//    context short, the plan takes this route with one partition per sequence: each
//    workgroup writes its rows, with no merge and no workspace (that page's single-tile
//    fast path for the whole batch).
//
// Both combine triples as M = max m_p, L = sum exp(m_p - M) l_p,
// out = sum exp(m_p - M) acc_p / L (the V4 merge kernel's combination, with the global
// maximum first and the division once at the end, as the commit page's phase 2 does).
//
// The block-table gather follows the "Baseline" and "V3 (Shared memory data reuse)"
// sections of the first page: token t of a sequence is slot t % page_size of physical
// page block_tables[b][t / page_size]; one K/V read serves every query head of the GQA
// group (V3 stages a page in shared memory for this; here both products run on the
// matrix cores straight from registers).  The streaming softmax is that page's Baseline
// recurrence.
//
// Scores are kept in base-2 units: z = (q . k) * |scale| * log2(e), so every exponential
// is the hardware exp2 (v_exp_f32).  A negative scale is folded into q (sign flip, exact).
//
// Per 16-token tile, one wave does (lane l: n = l % 16, g = l / 16):
//   scores  S^T = K Q^T with v_mfma_f32_16x16x32_f16 over head_dim: A = the tile's K rows
//           (MFMA row m holds token pi(m) = m / 4 + 4 (m % 4)), B = the query heads of the
//           chunk (column n = head n, zero past the chunk).  Lane (n, g) then holds the
//           scores of head n for tokens g, g + 4, g + 8, g + 12.
//   softmax the reference max of a head only moves (and the accumulators are rescaled)
//           when a score exceeds it by more than kRescaleSlack (2^8), so in steady state
//           a tile costs one exp2 per score and no reduction.  Any reference value gives
//           the same ratio acc / l; the slack only bounds the weights (<= 256, inside
//           fp16's range).
//   P.V     with v_mfma_f32_16x16x32_f16: A = each weight as two fp16 terms, p_hi =
//           fp16(p) and p_lo = fp16(p - p_hi) -- the score layout already is the A
//           layout (lane (n, g) holds head n, tokens g + 4i) -- and B = the same four V
//           rows twice, once against each term.  Lane (n, g) loads dims E n .. E n + E - 1
//           (E = D / 16) of rows g, g + 4, g + 8, g + 12 with one wide load per row (a load
//           instruction covers four whole rows), and v_perm regroups them into four tokens
//           of one dim; MFMA c takes dims E n + c.  The weight sum l adds the same
//           p_hi + p_lo, so the output is a convex combination of V rows with weights
//           within about 2^-23 of exact.  Lane (n, g) ends up holding head 4g + i
//           (register i), dims E n .. E n + E - 1.
// The next tile's loads (nontemporal) are issued before a tile is consumed when the
// route prefetches.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>

#include "pa_internal.h"

namespace pa {
namespace {

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
// Row stride, in 16-byte chunks, of the whole-row K staging (16 chunks of data per row).
// Measured with SQ_LDS_BANK_CONFLICT: 16 or 17 or 20 chunks leave the staging writes or
// operand reads with bank conflicts (17: 0.66 M conflict cycles per call at 64 x 8 heads);
// 18 chunks (288 bytes) has none.
constexpr int kKtStride = 18;

constexpr float kRescaleSlack = 8.0f;   // log2 units
// byte offset that lies past every tile's buffer range (loads there return zero)
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;
#ifndef PA_XCD_REMAP
#define PA_XCD_REMAP 1   // balanced route: contiguous work per XCD (see xcd_major)
#endif
#ifndef PA_KROW
#define PA_KROW 1    // load K in whole rows and regroup them through LDS (head_dim 128, both routes)
#endif
#ifndef PA_RUN_SKEW
#define PA_RUN_SKEW 20   // balanced route: percent by which early rounds of waves get more work
#endif
#ifndef PA_BAL_PRIO
#define PA_BAL_PRIO 1    // balanced route: raise the issue priority of waves that fall behind
#endif

struct DecodeArgs {
    const _Float16* q;
    const char* k;          // byte pointers to the caches
    const char* v;
    const int32_t* bt;
    const int32_t* ctx;
    float* out;
    float* ws_acc;          // partial rows of D floats
    float* ws_ml;           // partial rows' (max in log2 units, sum)
    int4* ws_desc;          // balanced route: two merge records per workgroup
    int* ws_cnt;            // single launch: band counters [grid], then group counters [2 grid]
    int single_launch;      // balanced route: the decode kernel merges crossing bands itself
    float scale_log2;       // |scale| * log2(e)
    uint32_t q_sign;        // 0x80008000 to negate q (negative scale), else 0
    int batch, query_heads, kv_heads, group, n_chunks, max_pages, partition, n_part_max, ps_log2;
    int force_split;
    int spw, waves_per_stream, bands;   // balanced route (see Plan)
    int num_pages;          // pages in the pool: table entries outside [0, num_pages) read as zeros
};

// A table entry outside the pool [0, num_pages) names no page: it becomes -1, which the
// tile loads treat as a page of zeros (a zero buffer range, so nothing is read).
__device__ __forceinline__ int pool_page(int entry, int num_pages) {
    return (uint32_t)entry < (uint32_t)num_pages ? entry : -1;
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

__device__ __forceinline__ half8_t as_half8(const uint4& x) { return __builtin_bit_cast(half8_t, x); }

template <int D>
struct Geo {
    static constexpr int T = 16;          // tokens per wave tile
    static constexpr int UK = D / 32;     // K loads (and score MFMAs) per tile
    static constexpr int E = D / 16;      // V dims per lane (fp16), and P.V MFMAs
    static constexpr int VW = E / 2;      // 32-bit words of a lane's V chunk
    static constexpr int C4 = D / 4;      // float4 columns of an output row
};

// Lane coordinates inside a wave.
struct Lane {
    int lane, n, g;
    int ktok;   // tile token whose K row this lane loads (MFMA row n)
    __device__ static Lane make(int lane) {
        Lane l;
        l.lane = lane;
        l.n = lane & 15;
        l.g = lane >> 4;
        l.ktok = (l.n >> 2) + 4 * (l.n & 3);
        return l;
    }
};

// B operand of the score MFMA: lane (n, g) holds q[row0 + n][32 j + 8 g .. + 7], zero
// for n >= HP; sign-flipped for a negative scale.  Split into the loads and the fix-up,
// so that a prefetch does not wait for its data.
template <int D, int HP>
__device__ __forceinline__ void load_q_raw(const _Float16* q, size_t row0, const Lane& L,
                                           uint4 (&qr)[Geo<D>::UK]) {
    const uint4* qp = reinterpret_cast<const uint4*>(q + (row0 + (L.n < HP ? L.n : 0)) * D);
#pragma unroll
    for (int j = 0; j < Geo<D>::UK; ++j) qr[j] = qp[4 * j + L.g];
}
template <int D, int HP>
__device__ __forceinline__ void fix_q(const uint4 (&qr)[Geo<D>::UK], uint32_t q_sign, const Lane& L,
                                      uint4 (&qb)[Geo<D>::UK]) {
#pragma unroll
    for (int j = 0; j < Geo<D>::UK; ++j) {
        uint4 w = qr[j];
        w.x ^= q_sign; w.y ^= q_sign; w.z ^= q_sign; w.w ^= q_sign;
        if (L.n >= HP) w = uint4{0u, 0u, 0u, 0u};
        qb[j] = w;
    }
}

// A raw buffer resource over `bytes` bytes at `base`.  Loads past `bytes` return zero
// without touching memory (the hardware range check), which is how rows past the valid
// tokens of a tile are kept out of the accumulators.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, kBufferFlags);
}
// `off` is the lane's byte offset, `soff` a wave-uniform one (an SGPR operand).
__device__ __forceinline__ uint4 buf_ld128(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, kLoadNontemporal);
    return uint4{t.x, t.y, t.z, t.w};
}
// VW (2 or 4) words of one lane's V chunk
template <int VW>
__device__ __forceinline__ void buf_ldv(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff, uint32_t (&w)[VW]) {
    if constexpr (VW == 4) {
        const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, kLoadNontemporal);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else {
        static_assert(VW == 2, "V chunks of 4 or 8 halves");
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t t = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, kLoadNontemporal);
        w[0] = t.x; w[1] = t.y;
    }
}

// Loads of one 16-token tile.  `kp`/`vp` point at the K/V row (this KV head) of the
// tile's first token; with pages of 8 the tile's tokens 8..15 sit in the next page, whose
// rows start at `kp2`/`vp2`.  Tokens past n_valid (0..16, wave-uniform) read as zero:
// their scores are masked, and their zero V rows add nothing.  ok1 / ok2 (wave-uniform):
// whether the first / second page is in the pool; a page that is not reads as zeros.
//   K: kb[j] = 16 bytes of row ktok, dims 32 j + 8 g .. + 7 (koff = ktok * tok + 16 g);
//      with KROW (D = 128) K is loaded like V instead: kb[i] = dims 8 n .. 8 n + 7 of row
//      4 i + g (koff = voff), whole rows per instruction, and regrouped through LDS.
//   V: vb[i] = dims E n .. E n + E - 1 of row 4 i + g (voff = g * tok + 2 E n).
template <int D, bool SPLIT, bool KROW = false>
__device__ __forceinline__ void load_kv(const char* kp, const char* vp, const char* kp2, const char* vp2,
                                        uint32_t koff, uint32_t voff, uint32_t tok_bytes, int n_valid,
                                        bool ok1, bool ok2, const Lane& L, uint4 (&kb)[Geo<D>::UK],
                                        uint32_t (&vb)[4][Geo<D>::VW]) {
    using G = Geo<D>;
    n_valid = __builtin_amdgcn_readfirstlane(n_valid);   // uniform; keeps the resource in SGPRs
    if constexpr (!SPLIT) {
        const int bytes = ok1 ? n_valid * (int)tok_bytes : 0;
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kp, bytes);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vp, bytes);
        if constexpr (KROW) {
#pragma unroll
            for (int i = 0; i < 4; ++i) kb[i] = buf_ld128(rk, koff, 4 * i * tok_bytes);
        } else {
#pragma unroll
            for (int j = 0; j < G::UK; ++j) kb[j] = buf_ld128(rk, koff + 64 * j);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) buf_ldv<G::VW>(rv, voff, 4 * i * tok_bytes, vb[i]);
    } else {
        const int n1 = ok1 ? min(n_valid, 8) : 0, n2 = ok2 ? max(n_valid - 8, 0) : 0;
        const __amdgpu_buffer_rsrc_t rk1 = tile_rsrc(kp, n1 * (int)tok_bytes);
        const __amdgpu_buffer_rsrc_t rk2 = tile_rsrc(kp2, n2 * (int)tok_bytes);
        const __amdgpu_buffer_rsrc_t rv1 = tile_rsrc(vp, n1 * (int)tok_bytes);
        const __amdgpu_buffer_rsrc_t rv2 = tile_rsrc(vp2, n2 * (int)tok_bytes);
        // K rows 0..7 are in the first page, 8..15 in the next.  Both loads are issued by
        // every lane with a wave-uniform resource; the lane's offset into the page it
        // does not use is pushed past the resource's range, so that load returns zero and
        // the two results combine with an OR.
        if constexpr (KROW) {
            // K group i covers rows 4 i .. 4 i + 3, like V
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < 2) kb[i] = buf_ld128(rk1, koff, 4 * i * tok_bytes);
                else kb[i] = buf_ld128(rk2, koff, (4 * i - 8) * tok_bytes);
            }
        } else {
            const bool first = L.ktok < 8;
            const uint32_t k1 = first ? koff : kOutOfRange;
            const uint32_t k2 = first ? kOutOfRange : koff - 8 * tok_bytes;
#pragma unroll
            for (int j = 0; j < G::UK; ++j) {
                const uint4 x = buf_ld128(rk1, k1 + 64 * j);
                const uint4 y = buf_ld128(rk2, k2 + 64 * j);
                kb[j] = uint4{x.x | y.x, x.y | y.y, x.z | y.z, x.w | y.w};
            }
        }
        // V group i covers rows 4 i .. 4 i + 3: groups 0, 1 in the first page, 2, 3 in the next
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < 2) buf_ldv<G::VW>(rv1, voff, 4 * i * tok_bytes, vb[i]);
            else buf_ldv<G::VW>(rv2, voff, (4 * i - 8) * tok_bytes, vb[i]);
        }
    }
}

// Streaming softmax state of one wave for HP (<= 8) heads.  Lane (n, g): mref = reference
// max of head n (equal on the four lanes of a head), lsum = this lane's share of head n's
// weight sum, acc[c][i] = output of head 4 g + i, dim E n + c.
template <int D, int HP>
struct WaveState {
    using G = Geo<D>;
    float mref;
    float lsum;
    float4_t acc[G::E];

    __device__ __forceinline__ void reset() {
        mref = -INFINITY;
        lsum = 0.f;
#pragma unroll
        for (int c = 0; c < G::E; ++c) acc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    // One tile: tokens at or past n_valid are masked (n_valid in 1..16, wave-uniform).
    // With KROW, kb holds whole-row K chunks (see load_kv) and kt is this wave's LDS
    // staging area of 16 slots x kKtStride 16-byte chunks: slot m holds token pi(m); the
    // score operands are read back in the MFMA layout.
    template <bool KROW = false>
    __device__ __forceinline__ void tile(const uint4 (&qb)[G::UK], const uint4 (&kb)[G::UK],
                                         const uint32_t (&vb)[4][G::VW], int n_valid, float sl2,
                                         const Lane& L, uint4* kt = nullptr) {
        float4_t s = {0.f, 0.f, 0.f, 0.f};
        if constexpr (KROW) {
            static_assert(D == 128, "whole-row K staging is laid out for 16 chunks per row");
            // the wave's reads of the previous tile are issued before these writes, and
            // these writes before the reads below (one wave; LDS executes in order)
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
            for (int i = 0; i < 4; ++i) kt[(4 * L.g + i) * kKtStride + L.n] = kb[i];   // token 4 i + g = pi(4 g + i)
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
            for (int j = 0; j < G::UK; ++j) {
                const uint4 kj = kt[L.n * kKtStride + 4 * j + L.g];
                s = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(kj), as_half8(qb[j]), s, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < G::UK; ++j)
                s = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(kb[j]), as_half8(qb[j]), s, 0, 0, 0);
        }
        // register i: token g + 4 i of head n
        float z[4];
        bool grow = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = (L.g + 4 * i < n_valid) ? s[i] * sl2 : -INFINITY;
            grow |= z[i] > mref + kRescaleSlack;
        }
        grow = grow && L.n < HP;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {   // rare: move the reference max
            // token 0 is valid, so every head's tile maximum is finite
            float zt = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
            zt = fmaxf(zt, __shfl_xor(zt, 16));
            zt = fmaxf(zt, __shfl_xor(zt, 32));
            const float mn = fmaxf(mref, zt);
            const float alpha = fast_exp2(mref - mn);   // 0 while mref is -inf
            mref = mn;
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * L.g + i);   // head 4 g + i
#pragma unroll
                for (int c = 0; c < G::E; ++c) acc[c][i] *= ai;
            }
        }
        // Weights in two fp16 terms: p_hi = fp16(p), p_lo = fp16(p - p_hi) (about 22 bits of
        // p; a single fp16 rounding would cost up to 2^-12 of each weight, an error that
        // grows with the spread of the value rows).  A operand of the 16x16x32 product:
        // k = 8 g + i holds p_hi of token g + 4 i, k = 8 g + 4 + i its p_lo.
        half8_t pw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e = fast_exp2(z[i] - mref);
            const _Float16 hi = (_Float16)e;
            const _Float16 lo = (_Float16)(e - (float)hi);
            pw[i] = hi;
            pw[4 + i] = lo;
            lsum += (float)hi + (float)lo;   // exact in fp32: the weight the product uses
        }
        // B operand of P.V for dim E n + c: tokens g, g + 4, g + 8, g + 12 (half c of
        // the rows' chunks), twice -- once against p_hi, once against p_lo
#pragma unroll
        for (int j = 0; j < G::VW; ++j) {
            const uint32_t w0 = vb[0][j], w1 = vb[1][j], w2 = vb[2][j], w3 = vb[3][j];
            const uint32_t e0 = __builtin_amdgcn_perm(w1, w0, 0x05040100u), e1 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
            const uint32_t o0 = __builtin_amdgcn_perm(w1, w0, 0x07060302u), o1 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
            const uint4 even = {e0, e1, e0, e1};
            const uint4 odd = {o0, o1, o0, o1};
            acc[2 * j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pw, as_half8(even), acc[2 * j], 0, 0, 0);
            acc[2 * j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pw, as_half8(odd), acc[2 * j + 1], 0, 0, 0);
        }
    }

    // Weight sum of head n (returned on every lane of head n).  All lanes must call it.
    __device__ __forceinline__ float head_sum() const {
        float l = lsum;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        return l;
    }

    // Visit this lane's output values: f(head, dim, float4 at dims dim .. dim + 3, i).
    template <typename F>
    __device__ __forceinline__ void for_each_out(const Lane& L, F&& f) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = 4 * L.g + i;
            if (hh < HP) {
#pragma unroll
                for (int c = 0; c < G::E; c += 4)
                    f(hh, G::E * L.n + c, float4_t{acc[c][i], acc[c + 1][i], acc[c + 2][i], acc[c + 3][i]}, i);
            }
        }
    }

    // Write the finished rows out[row0 + h] = acc / l for h < HP.  All lanes must call it.
    __device__ __forceinline__ void write_out(float* out, size_t row0, const Lane& L) const {
        const float l = head_sum();
        float rl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) rl[i] = 1.f / __shfl(l, 4 * L.g + i);
        for_each_out(L, [&](int hh, int dim, float4_t v, int i) {
            *reinterpret_cast<float4_t*>(out + (row0 + hh) * D + dim) = v * rl[i];
        });
    }

    // Store the unnormalised triple: m[h], l[h], acc[h * D + dim] for h < HP.  All lanes
    // must call it.
    __device__ __forceinline__ void store_triple(float* m, float* l_out, float* accp, const Lane& L) const {
        const float l = head_sum();
        if (L.g == 0 && L.n < HP) {
            m[L.n] = mref;
            l_out[L.n] = l;
        }
        for_each_out(L, [&](int hh, int dim, float4_t v, int) {
            *reinterpret_cast<float4_t*>(accp + hh * D + dim) = v;
        });
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
    using G = Geo<D>;
    constexpr int T = G::T;
    constexpr int C4 = G::C4;

    __shared__ int s_bt[kMaxPartitionPages];
    __shared__ float s_m[NW][HP];
    __shared__ float s_l[NW][HP];
    __shared__ float4_t s_acc[NW][HP][C4];
    // K in whole rows, regrouped through LDS as on the balanced route (head_dim 128)
    constexpr bool KR = PA_KROW && D == 128;
    __shared__ uint4 s_kt[KR ? NW * 16 * kKtStride : 1];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Lane L = Lane::make(tid & 63);

    // Work item: partitions vary slowest, so every sequence's first (largest) partition
    // is dispatched before any remainder partition.  Workgroups are dealt to the XCDs in
    // turn, so with the KV head varying fastest each XCD would read the same head's rows
    // throughout; the head is rotated by sequence + partition instead (a permutation of
    // the items of one (sequence, partition)).  Measured on partitions of 1024: batch64
    // 77.4 -> 73.4 us, mixed128 284.6 -> 265.4 us; long100k +0.9 and small_batch +0.5 us.
    int id = blockIdx.x;
    const int chunk = id % a.n_chunks; id /= a.n_chunks;
    const int kvh_dealt = id % a.kv_heads; id /= a.kv_heads;
    const int nb = (int)(gridDim.x / (unsigned)(a.n_chunks * a.kv_heads * a.n_part_max));
    const int b = id % nb;
    const int part = id / nb;
    const int kvh = (kvh_dealt + b + part) % a.kv_heads;

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
    for (int i = tid; i < npg; i += NW * 64) s_bt[i] = pool_page(bt_row[i], a.num_pages);

    uint4 qb[G::UK];
    load_q_raw<D, HP>(a.q, row0, L, qb);
    fix_q<D, HP>(qb, a.q_sign, L, qb);
    __syncthreads();

    const size_t tok_bytes = (size_t)a.kv_heads * D * 2;     // bytes between slots
    const size_t page_bytes = tok_bytes << ps_log2;
    const char* kbase = a.k + (size_t)kvh * D * 2;
    const char* vbase = a.v + (size_t)kvh * D * 2;
    const uint32_t voff = (uint32_t)(L.g * tok_bytes) + 2u * G::E * L.n;
    const uint32_t koff = KR ? voff : (uint32_t)(L.ktok * tok_bytes) + 16u * L.g;
    uint4* const kt = KR ? &s_kt[wave * 16 * kKtStride] : nullptr;
    const float sl2 = a.scale_log2;

    WaveState<D, HP> st;
    st.reset();

    const int n_tok = t_end - t_begin;
    const int n_tiles = (n_tok + T - 1) / T;
    // This wave takes tiles wave, wave + NW, ...
    const int nk = wave < n_tiles ? (n_tiles - wave + NW - 1) / NW : 0;

    auto load_tile = [&](int k, uint4 (&kb)[G::UK], uint32_t (&vb)[4][G::VW]) {
        const int t0 = t_begin + (wave + k * NW) * T;
        const int pg = (t0 >> ps_log2) - pg0;
        const int phys = __builtin_amdgcn_readfirstlane(s_bt[pg]);   // -1: outside the pool
        const size_t base = (size_t)max(phys, 0) * page_bytes + (size_t)(t0 & ((1 << ps_log2) - 1)) * tok_bytes;
        size_t base2 = base;
        int phys2 = phys;
        if constexpr (SPLIT) {
            // tokens 8..15 of the tile sit in the next page, which exists only when the
            // tile reaches past token 8
            if (t0 + 8 < t_end) {
                phys2 = __builtin_amdgcn_readfirstlane(s_bt[pg + 1]);
                base2 = (size_t)max(phys2, 0) * page_bytes;
            }
        }
        load_kv<D, SPLIT, KR>(kbase + base, vbase + base, kbase + base2, vbase + base2, koff, voff,
                          (uint32_t)tok_bytes, max(0, min(T, t_end - t0)), phys >= 0, phys2 >= 0, L,
                          kb, vb);
    };

    if (nk > 0) {
        // DEPTH register buffers; tile k + DEPTH - 1 is loaded before tile k is consumed.
        // The loop runs a multiple of DEPTH tiles and has no exit in its middle, so the
        // compiler's wait-count bookkeeping sees the same outstanding loads on every path
        // into the loop header.  Padding tiles (k >= nk) reload the last tile (already in
        // the caches) and are skipped after their loads are waited for.  The scheduling
        // barriers keep the compiler from sinking the loads below the arithmetic of the
        // tile before them.
        uint4 kb[DEPTH][G::UK];
        uint32_t vb[DEPTH][4][G::VW];
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) load_tile(min(d, nk - 1), kb[d], vb[d]);
        for (int k = 0; k < nk; k += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int nxt = (d + DEPTH - 1) % DEPTH;
                load_tile(min(k + d + DEPTH - 1, nk - 1), kb[nxt], vb[nxt]);
                __builtin_amdgcn_sched_barrier(0);
                const int t0 = t_begin + (wave + (k + d) * NW) * T;
                if (k + d < nk) st.template tile<KR>(qb, kb[d], vb[d], max(0, min(T, t_end - t0)), sl2, L, kt);
                else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            }
        }
    }

    st.store_triple(&s_m[wave][0], &s_l[wave][0], reinterpret_cast<float*>(&s_acc[wave][0][0]), L);
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

constexpr int kMergeThreads = 512;
// Balanced route: the merge tasks of a band (one row, kSliceCols float4 columns: 128
// bytes) are dealt over the blocks of the workgroups the band spans.  In a band of at most
// kShortMerge pieces one thread loads all pieces of its column; in longer bands a thread
// takes kLongUnroll of them (4 measured faster than 8 or 2 on a 128-piece band: more
// threads share a task's loads, and the extra combining goes through LDS in one step).
constexpr int kShortMerge = 16;
constexpr int kSliceCols = 8;
constexpr int kLongUnroll = 4;
// a lane offset past every merge resource (at most 2^31 - 2^24 bytes, so that adding a
// piece offset cannot wrap past 2^32)
constexpr uint32_t kPastRange = 0x7F000000u;

// a compile-time int carried by a value (for generic lambdas)
template <int N>
struct IntC {
    static constexpr int value = N;
};

// (m, l, o) <- the combination of two (max, sum, acc) triples; a triple with maximum
// -inf weighs nothing, and two of them give (-inf, 0, 0).
__device__ __forceinline__ void fold_triple(float& m, float& l, float4_t& o, float m2, float l2, float4_t o2) {
    const float M = fmaxf(m, m2);
    const float Ms = M == -INFINITY ? 0.f : M;
    const float a1 = fast_exp2(m - Ms);
    const float a2 = fast_exp2(m2 - Ms);
    l = a1 * l + a2 * l2;
    o = a1 * o + a2 * o2;
    m = M;
}

// Combination of n (max, sum, acc) triples of one output row: out = sum_p e_p acc_p /
// sum_p e_p l_p with e_p = exp2(m_p - max m).  Triple p is row r(p) of the workspace
// (max, sum at ws_ml[2 r], acc at ws_acc[D r]) with r(0) = row_first and
// r(p) = row_rest + (p - 1) * stride.  One pass: thread (g, c) folds triple 0 (group 0)
// and the triples p = 1 + g, 1 + g + GR, ... for float4 column c into a running triple,
// rescaling whenever its maximum grows; the GR partial triples are then combined through
// LDS.  Triples past the first are read with buffer loads over exactly their rows: the
// lane's part of the offset stays in one register and the part shared by the wave
// (which triple of the group) is a scalar operand, so a batch of UNR loads in flight
// costs no address registers.  Every thread of the block takes part.  At least one
// triple has a finite maximum.
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
    if (g == 0) {   // triple 0
        o = reinterpret_cast<const float4_t*>(ws_acc + row_first * D)[c];
        const float2 ml = reinterpret_cast<const float2*>(ws_ml)[row_first];
        m = ml.x;
        l = ml.y;
    }
    const int nr = n - 1;                           // triples at row_rest + q * stride
    if (nr > 0) {
        const uint32_t acc_row = (uint32_t)(stride * D * 4);   // bytes between triples
        const uint32_t ml_row = (uint32_t)(stride * 8);
        const __amdgpu_buffer_rsrc_t racc =
            tile_rsrc(reinterpret_cast<const char*>(ws_acc + row_rest * D), (int)(nr * acc_row));
        const __amdgpu_buffer_rsrc_t rml =
            tile_rsrc(reinterpret_cast<const char*>(ws_ml + row_rest * 2), (int)(nr * ml_row));
        const uint32_t vacc = (uint32_t)g * acc_row + 16u * c;
        const uint32_t vml = (uint32_t)g * ml_row;
        typedef float f32x2_t __attribute__((ext_vector_type(2)));
        for (int q0 = 0; q0 < nr; q0 += GR * UNR) {
            float4_t av[UNR];
            float2 mv[UNR];
#pragma unroll
            for (int k = 0; k < UNR; ++k) {
                const uint32_t qs = (uint32_t)(q0 + k * GR);   // wave-uniform
                // (scalar offsets are wave-uniform; readfirstlane keeps the compiler from
                // carrying them in vector registers, which costs a loop per load)
                const int sacc = __builtin_amdgcn_readfirstlane((int)(qs * acc_row));
                const int sml = __builtin_amdgcn_readfirstlane((int)(qs * ml_row));
                av[k] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(racc, (int)vacc, sacc, 0));
                // (the whole vector is reinterpreted: bit-casting single elements of the
                // load's result made clang read one dword for both)
                const f32x2_t t = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rml, (int)vml, sml, 0));
                const bool live = q0 + k * GR + g < nr;
                mv[k] = make_float2(live ? t.x : -INFINITY, t.y);
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
                    const float e = fast_exp2(mv[k].x - mb);   // 0 for a triple past the end
                    l += e * mv[k].y;
                    o += e * av[k];
                }
                m = mb;
            }
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
    const int n = (int)min(((long long)ctx + a.partition - 1) / a.partition, (long long)a.n_part_max);
    if (n <= 0 || (n == 1 && !a.force_split)) return;   // written by the decode kernel
    const size_t r0 = (size_t)bh * a.n_part_max;
    combine_rows<D>(a.ws_ml, a.ws_acc, r0, r0 + 1, 1, n, a.out + (size_t)bh * D);
}

// Fixed-partition route, rows with few partitions: one thread per (output row, float4
// column), kMergeThreads / (D / 4) rows per block.  A thread folds its column over the
// row's partitions in batches of kRowFoldUnroll (every load of a batch issued before any
// is used), so a row with n partitions costs ceil(n / kRowFoldUnroll) round trips and a
// row written by the decode kernel (one partition) nothing.  Used when no row can have
// more than kRowFoldMax partitions; longer rows take pa_merge_kernel.
constexpr int kRowFoldUnroll = 8;
constexpr int kRowFoldMax = 32;

template <int D>
__global__ void __launch_bounds__(kMergeThreads)
pa_merge_rows_kernel(MergeArgs a, int rows) {
    constexpr int C4 = D / 4;
    constexpr int RPB = kMergeThreads / C4;
    const int row = blockIdx.x * RPB + (int)threadIdx.x / C4;   // b * query_heads + h
    const int c4 = (int)threadIdx.x % C4;
    if (row >= rows) return;
    // (a length past the plan's bound is a broken precondition: its row reads no slot past
    // its own)
    const int n = (int)min(((long long)a.ctx[row / a.query_heads] + a.partition - 1) / a.partition,
                           (long long)a.n_part_max);
    if (n <= 0 || (n == 1 && !a.force_split)) return;   // written by the decode kernel
    const size_t base = (size_t)row * a.n_part_max;
    float m = -INFINITY, l = 0.f;
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < n; p0 += kRowFoldUnroll) {
        float4_t pa[kRowFoldUnroll];
        float pm[kRowFoldUnroll], pl[kRowFoldUnroll];
#pragma unroll
        for (int k = 0; k < kRowFoldUnroll; ++k) {
            const size_t slot = base + (p0 + k < n ? p0 + k : p0);   // past the row: weight 0
            pa[k] = reinterpret_cast<const float4_t*>(a.ws_acc + slot * D)[c4];
            pm[k] = p0 + k < n ? a.ws_ml[slot * 2] : -INFINITY;
            pl[k] = a.ws_ml[slot * 2 + 1];
        }
        float M = m;
#pragma unroll
        for (int k = 0; k < kRowFoldUnroll; ++k) M = fmaxf(M, pm[k]);
        // partition 0 holds token 0, so M is finite from the first batch on
        const float a0 = fast_exp2(m - M);      // 0 while nothing was folded in yet
        l *= a0;
        acc *= a0;
#pragma unroll
        for (int k = 0; k < kRowFoldUnroll; ++k) {
            const float e = fast_exp2(pm[k] - M);
            l += e * pl[k];
            acc += e * pa[k];
        }
        m = M;
    }
    reinterpret_cast<float4_t*>(a.out + (size_t)row * D)[c4] = acc / l;
}

// ------------------------------------------------------------------------------------
// Balanced route: one resident workgroup per CU splits all token tiles evenly.
//
// Streams of a sequence: s = kv_head * n_chunks + chunk, S of them.  They are grouped in
// bands of spw consecutive streams (band = s / spw); a unit is (sequence b, band, tile lt)
// and the units are laid end to end in the order (b, band, lt), N in total.  Workgroup w
// takes the units [w N / W, (w+1) N / W).  Its waves form spw groups of
// waves_per_stream: wave (sp, r) reads stream band * spw + sp of every unit in the r-th
// equal run of the workgroup's range, crossing band and sequence boundaries as the units
// do, one tile (or one tile ahead) at a time.
// A stream that lies wholly inside one wave is finished by that wave (the single-pass
// case); pieces of a stream that crosses waves are combined in LDS at the end of the
// workgroup, and a stream that crosses workgroups leaves one (max, sum, acc) triple per
// workgroup in the workspace for the merge kernel.
// ------------------------------------------------------------------------------------

// Inclusive sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8 lanes within each row
// of 16 (zeros shifted in), then row 0's last lane added to row 1, and lane 31's total to
// rows 2 and 3 (rows 1 and 3 already hold rows 0 and 2).  All DPP moves on the VALU.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2, 3
    return x;
}

// Lengths -> LDS, exclusive prefix sums of tiles per sequence.  Every thread of the
// block calls it; returns the total tile count of one band plane.  Up to 64 sequences,
// every wave computes the whole prefix itself (one length per lane, a DPP scan) and
// writes the same values: no barrier, and a wave reads what it wrote.  Callers must
// therefore not count on a barrier here.
template <int NT>
__device__ __forceinline__ int tile_prefix(const int32_t* ctx, int B, int* s_pref, int* s_ctx, int* s_wsum) {
    if (B <= 64) {
        const int lane = threadIdx.x & 63;
        const int c = lane < B ? ctx[lane] : 0;
        const int mine = (c + 15) >> 4;
        const int incl = wave_incl_scan(mine);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (lane < B) {
            s_ctx[lane] = c;
            s_pref[lane] = incl - mine;
        }
        if (lane == 0) s_pref[B] = total;
        return total;
    }
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

// Position of unit t (0 <= t < N): sequence b (the smallest with SG * pref[b+1] > t),
// band within the sequence, tile lt of the band.  The host keeps N below 2^31.
// The sequence holding unit t, for a wave-uniform t: the number of sequences 1 .. B-1
// whose first unit is at or before t (the prefix sums are non-decreasing), counted 64
// entries per LDS read across the wave -- one read for up to 65 sequences, where a binary
// search takes one dependent read per halving.  Large batches use the binary search.
__device__ __forceinline__ int seq_of_unit_wave(int t, int B, int SG, const int* s_pref, int lane) {
    if (B > 256) {
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (SG * s_pref[mid + 1] > t) hi = mid;
            else lo = mid + 1;
        }
        return lo;
    }
    int b = 0;
    for (int base = 1; base < B; base += 64) {
        const int l = base + lane;
        const bool at_or_before = l < B && SG * s_pref[l] <= t;
        b += __popcll(__builtin_amdgcn_ballot_w64(at_or_before));
    }
    return b;
}

// The sequence holding unit t, given a sequence b0 at or before it (wave-uniform): the next
// four sequence starts are read at once; only a unit more than four sequences past b0
// falls back to a binary search.
__device__ __forceinline__ int seq_of_unit_from(int t, int b0, int B, int SG, const int* s_pref) {
    int c = 0;
#pragma unroll
    for (int k = 1; k <= 4; ++k) {
        const int l = b0 + k;
        c += (l < B && SG * s_pref[l] <= t) ? 1 : 0;
    }
    int lo = b0 + c;
    if (c == 4) {
        int hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (SG * s_pref[mid + 1] > t) hi = mid;
            else lo = mid + 1;
        }
    }
    return lo;
}

__device__ __forceinline__ void locate_unit(int t, int B, int SG, const int* s_pref, int& b, int& band, int& lt) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (SG * s_pref[mid + 1] > t) hi = mid;
        else lo = mid + 1;
    }
    b = lo;
    const int Tb = s_pref[b + 1] - s_pref[b];
    const int off = t - SG * s_pref[b];
    band = off / Tb;
    lt = off - band * Tb;
}

// Workgroups are handed to the XCDs in turn (workgroup i to XCD i % kXcds), and each XCD
// has its own L2.  This renumbering gives each XCD a contiguous run of the work, so that
// the pieces of a stream split between workgroups mostly meet in one L2.
// A bijection of [0, G): XCD x's k-th workgroup becomes x * (G / X) + min(x, G % X) + k.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_major(int b, int G) {
    const int x = b % kXcds, k = b / kXcds, q = G / kXcds, r = G % kXcds;
    return x * q + min(x, r) + k;
}

// floor(x * N / W) for 0 <= x <= W.  Exact in double: x N < 2^53 is represented exactly,
// and a quotient that is not an integer lies at least 1/W below the next integer, far
// more than the rounding error of the (correctly rounded) division.
__device__ __forceinline__ int split_point(int x, int N, int W) {
    return (int)floor((double)x * (double)N / (double)W);
}

// The workgroup holding unit c (0 <= c < N): the largest x with split_point(x) <= c,
// i.e. floor(((c + 1) W - 1) / N) (exact in double, as for split_point).
__device__ __forceinline__ int wg_of_unit(int c, int N, int W) {
    const int x = (int)floor((((double)c + 1.0) * (double)W - 1.0) / (double)N);
    return min(x, W - 1);
}

// Single launch (PA_FLAG_SINGLE_LAUNCH): the workgroups of a crossing band merge it
// themselves, at the end of the decode kernel, instead of a second kernel -- the
// "last-arriving workgroup merges" form of the split/merge of the "V4 (Context-axis
// parallelism)" section of "[TIL] Optimizing paged attention".
//
// Workgroup x holds a piece of at most two crossing bands (records: the band holding its
// first unit, started in an earlier workgroup o -- piece on side 0; the band it owns --
// piece on the records' side).  A band owned by o has participants o .. o + n - 1, in
// groups of kArrivalGroup from the owner: group g has leader L = o + kArrivalGroup g.
// Each participant, once its pieces are in memory, increments its group's counter (group
// counter slot 2 L + 1 when L is the owner, else 2 L); the one that sees the group's
// size - 1 folds the group's pieces (in participant order) into the leader's piece slot,
// or straight into the output when the band has one group, and resets the counter.  With
// several groups, each group merger then increments the band counter (slot o); the one
// that sees the group count - 1 folds the group triples into the output and resets it.
// So no workgroup folds more than kArrivalGroup triples, and every counter is zero again
// when the kernel ends (the caller zeroes them once, before the first call).
// Arrivals are release atomics at device scope (the pieces are written back from this
// XCD's L2 first); a merger's acquire invalidates its caches before it reads.
constexpr int kArrivalGroup = 16;

// Fold np (<= NP) triples of every row of a band, in order p = 0 .. np - 1: triple p of row
// r is workspace row src(p) + r.  The result goes to workspace rows dst + r (unnormalised,
// when to_out is false) or to the band's output rows.  Every load of a task is issued
// before any is used; lanes past np reload triple 0 and weigh nothing.
template <int D, int HP, int NP, typename Src>
__device__ __forceinline__ void fold_band(const DecodeArgs& a, int spw, int np, Src src, bool to_out,
                                          size_t dst, int b, int band, int nthreads) {
    constexpr int C4 = D / 4;
    const int rows = spw * HP;
    for (int task = threadIdx.x; task < rows * C4; task += nthreads) {
        const int r = task / C4;
        const int c4 = task - r * C4;
        float4_t pa[NP];
        float pm[NP], pl[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const size_t row = src(p < np ? p : 0) + r;
            pa[p] = reinterpret_cast<const float4_t*>(a.ws_acc + row * D)[c4];
            pm[p] = a.ws_ml[row * 2];
            pl[p] = a.ws_ml[row * 2 + 1];
        }
        float M = -INFINITY;
#pragma unroll
        for (int p = 0; p < NP; ++p) M = fmaxf(M, p < np ? pm[p] : -INFINITY);
        const float Ms = M == -INFINITY ? 0.f : M;   // a group of empty workgroups: weight 0
        float L = 0.f;
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const float e = p < np ? fast_exp2(pm[p] - Ms) : 0.f;
            L += e * pl[p];
            acc += e * pa[p];
        }
        if (to_out) {
            const int sp = r / HP;
            const int h = r - sp * HP;
            const int s = band * spw + sp;
            const int kvh = s / a.n_chunks;
            const int chunk = s - kvh * a.n_chunks;
            reinterpret_cast<float4_t*>(a.out + ((size_t)b * a.query_heads + kvh * a.group + chunk * HP + h) * D)[c4] = acc / L;
        } else {
            reinterpret_cast<float4_t*>(a.ws_acc + (dst + r) * D)[c4] = acc;
            if (c4 == 0) {
                a.ws_ml[(dst + r) * 2] = M;
                a.ws_ml[(dst + r) * 2 + 1] = L;
            }
        }
    }
}

template <int D, int HP, typename Src>
__device__ __forceinline__ void fold_band_n(const DecodeArgs& a, int spw, int np, Src src, bool to_out,
                                            size_t dst, int b, int band, int nthreads) {
    static_assert(kArrivalGroup == 16, "fold shapes below cover up to 16 triples");
    if (np <= 4) fold_band<D, HP, 4>(a, spw, np, src, to_out, dst, b, band, nthreads);
    else if (np <= 8) fold_band<D, HP, 8>(a, spw, np, src, to_out, dst, b, band, nthreads);
    else fold_band<D, HP, 16>(a, spw, np, src, to_out, dst, b, band, nthreads);
}

// The arrivals of one thread on up to two counters (release once, then both atomics in
// flight together): bit t of the result says whether the caller was the last of
// expected[t] on counter[t] (then with an acquire done and that counter reset).
__device__ __forceinline__ int arrive_last2(int* const (&counter)[2], const int (&expected)[2]) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    int old[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        old[t] = counter[t] ? __hip_atomic_fetch_add(counter[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -1;
    int last = 0;
#pragma unroll
    for (int t = 0; t < 2; ++t)
        if (counter[t] && old[t] == expected[t] - 1) last |= 1 << t;
    if (last) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
        for (int t = 0; t < 2; ++t)
            if (last & (1 << t)) __hip_atomic_store(counter[t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return last;
}

template <int D, int HP, int NT>
__device__ __forceinline__ void single_launch_merge(const DecodeArgs& a, int w, int NWG, int spw,
                                                    const int4 (&s_rec)[2], int (&s_last)[4]) {
    const size_t rows = (size_t)spw * HP;
    auto slot = [&](int x, int side) { return ((size_t)x * 2 + side) * rows; };
    int* band_cnt = a.ws_cnt;
    int* grp_cnt = a.ws_cnt + NWG;
    // band t (0: the covering band, 1: the own band): owner, pieces, owner's side, group
    int n[2], o[2], side_o[2], L[2], sg[2], ng[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int4 r = s_rec[t == 0 ? 1 : 0];
        n[t] = t == 0 ? r.w : r.z;
        o[t] = t == 0 ? (r.z >> 1) : w;
        side_o[t] = t == 0 ? (r.z & 1) : r.w;
        const int g = n[t] > 0 ? (w - o[t]) / kArrivalGroup : 0;
        L[t] = o[t] + kArrivalGroup * g;
        sg[t] = min(kArrivalGroup, n[t] - kArrivalGroup * g);
        ng[t] = (n[t] + kArrivalGroup - 1) / kArrivalGroup;
    }
    if (n[0] <= 0 && n[1] <= 0) return;              // block-uniform: no crossing band
    // this wave's piece stores have reached L2 (the counter counts stores on this target);
    // after the barrier, every piece of this workgroup has
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        int* c[2];
        int e[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            c[t] = n[t] > 0 ? grp_cnt + 2 * L[t] + (L[t] == o[t] ? 1 : 0) : nullptr;
            e[t] = sg[t];
        }
        s_last[0] = arrive_last2(c, e);
    }
    __syncthreads();
    const int last1 = s_last[0];
    int need2 = 0;                                    // bands whose group triple needs a band merge
    for (int t = 0; t < 2; ++t) {
        if (!(last1 & (1 << t))) continue;            // block-uniform
        const int4 r = s_rec[t == 0 ? 1 : 0];
        const int ot = o[t], st = side_o[t], Lt = L[t];
        fold_band_n<D, HP>(a, spw, sg[t], [&](int p) { return slot(Lt + p, Lt + p == ot ? st : 0); },
                           ng[t] == 1, slot(Lt, Lt == ot ? st : 0), r.x, r.y, NT);
        if (ng[t] > 1) need2 |= 1 << t;
    }
    if (!need2) return;                               // block-uniform
    __builtin_amdgcn_s_waitcnt(0);                    // the group triples have reached L2
    __syncthreads();
    if (threadIdx.x == 0) {
        int* c[2];
        int e[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            c[t] = (need2 & (1 << t)) ? band_cnt + o[t] : nullptr;
            e[t] = ng[t];
        }
        s_last[1] = arrive_last2(c, e);
    }
    __syncthreads();
    const int last2 = s_last[1];
    for (int t = 0; t < 2; ++t) {
        if (!(last2 & (1 << t))) continue;
        const int4 r = s_rec[t == 0 ? 1 : 0];
        const int ot = o[t], st = side_o[t];
        fold_band_n<D, HP>(a, spw, ng[t],
                           [&](int p) {
                               const int Lg = ot + kArrivalGroup * p;
                               return slot(Lg, Lg == ot ? st : 0);
                           },
                           true, 0, r.x, r.y, NT);
    }
}

// How a call of the balanced route is organised (a template argument, so that the default
// kernel carries no code of the other):
//   kModeSplit : the even split; crossing bands leave pieces for pa_merge_balanced;
//   kModeSingle: the even split, crossing bands merged by their own workgroups at the end
//                (PA_FLAG_SINGLE_LAUNCH).
constexpr int kModeSplit = 0;
constexpr int kModeSingle = 1;

template <int D, int HP, int DEPTH, int NW, bool SPLIT, bool KROW, int MODE>
__global__ void __launch_bounds__(NW * 64)
pa_decode_balanced(DecodeArgs a) {
    using G = Geo<D>;
    constexpr int T = G::T;
    constexpr int C4 = G::C4;
    constexpr int NT = NW * 64;
    constexpr int NS = 2 * NW;       // partial slots: a wave's first and last segment
    static_assert(NS <= 64 && NW <= 63, "a wave's lanes hold the slots and the run bounds");

    extern __shared__ int s_dyn[];
    __shared__ int s_wsum[NW];
    __shared__ float s_m[NS][HP];
    __shared__ float s_l[NS][HP];
    __shared__ float4_t s_acc[NS][HP][C4];
    // per slot: {stream id (-1: empty), first unit, end unit, band's first unit},
    // {band's end unit, first output row, stream within the band, -}
    __shared__ int4 s_meta[NS][2];
    __shared__ int4 s_rec[2];        // the workgroup's merge records (own band, covering band)
    __shared__ int s_last[4];        // single launch: whether this workgroup merges (per stage)
    __shared__ uint4 s_kt[KROW ? NW * 16 * kKtStride : 1];   // whole-row K staging, per wave

    const int B = a.batch;
    int* s_pref = s_dyn;             // [B + 1]
    int* s_ctx = s_dyn + B + 1;      // [B]
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Lane L = Lane::make(tid & 63);

    const int SPW = a.spw;                    // streams side by side
    const int RW = a.waves_per_stream;        // waves per stream
    const int SG = a.bands;                   // bands per sequence
    const int S = SG * SPW;                   // streams per sequence
    // Waves are handed to the SIMDs in turn (wave i to SIMD i % 4) and a SIMD serves its
    // older waves first, so the waves of later rounds (i / 4) start later and progress
    // more slowly.  Runs are therefore assigned round-major -- run rr = wave / SPW, stream
    // sp = wave % SPW -- and weighted: run rr gets a share proportional to
    // 1 + skew (RW - 1 - 2 rr) / (RW - 1).  li orders the waves stream-major, so that the
    // LDS slots of one stream's runs are adjacent.
    const int rr = wave / SPW;                // this wave's run of the workgroup's range
    const int sp = wave - rr * SPW;           // this wave's stream within a band
    const int li = sp * RW + rr;

    // each wave starts its own two slots empty (the prefix below has no barrier for
    // small batches)
    if (L.lane < 2) s_meta[2 * li + L.lane][0] = int4{-1, 0, -1, 0};
    const int plane = tile_prefix<NT>(a.ctx, B, s_pref, s_ctx, s_wsum);

    // empty sequences: a zero output, written by one workgroup each
    for (int b = blockIdx.x; b < B; b += gridDim.x)
        if (s_ctx[b] == 0)
            for (int i = tid; i < a.query_heads * D; i += NT) a.out[(size_t)b * a.query_heads * D + i] = 0.f;

    const int N = SG * plane;
    const int NWG = gridDim.x;
    const int w = PA_XCD_REMAP ? xcd_major((int)blockIdx.x, NWG) : (int)blockIdx.x;
    const int g0 = split_point(w, N, NWG);
    const int g1 = split_point(w + 1, N, NWG);
    auto run_start = [&](int r) {   // cumulative weight of runs 0 .. r-1, over the total
        if (RW == 1) return r == 0 ? g0 : g1;
        const long long cum = (long long)r * (RW - 1) * (100 + PA_RUN_SKEW) - (long long)PA_RUN_SKEW * r * (r - 1);
        const long long total = (long long)RW * (RW - 1) * 100;
        return g0 + (int)((long long)(g1 - g0) * cum / total);
    };
    const int wr0 = run_start(rr);
    const int wr1 = run_start(rr + 1);
    const int nk = wr1 - wr0;

    const int ps_log2 = a.ps_log2;
    const size_t tok_bytes = (size_t)a.kv_heads * D * 2;
    const size_t page_bytes = tok_bytes << ps_log2;
    const uint32_t voff = (uint32_t)(L.g * tok_bytes) + 2u * G::E * L.n;
    const uint32_t koff = KROW ? voff : (uint32_t)(L.ktok * tok_bytes) + 16u * L.g;
    uint4* const kt = KROW ? &s_kt[wave * 16 * kKtStride] : nullptr;
    const float sl2 = a.scale_log2;

    // Physical pages of the wave's units, 64 at a time: lane i holds the page of unit
    // (wr0 + batch + i) (and, for pages of 8, the page of its second half).
    int btv = 0, btv2 = 0;
    auto load_pages = [&](int batch, int b0) {
        const int t = wr0 + batch + L.lane;
        if (t < wr1) {
            // b0: the sequence of unit wr0 + batch (where the cursor stands)
            const int b = seq_of_unit_from(t, b0, B, SG, s_pref);
            const int Tb = s_pref[b + 1] - s_pref[b];
            const int off = t - SG * s_pref[b];
            const int lt = off - (off / Tb) * Tb;
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
        btv = pool_page(btv, a.num_pages);
        if constexpr (SPLIT) btv2 = pool_page(btv2, a.num_pages);
    };

    // A wave-uniform cursor over the units to load, and the description of a loaded tile.
    struct Desc {
        int b, s, lt, T, n_valid;
        bool first;   // the tile opens a segment of this wave (its first, or a stream start)
    };
    // cursor: sequence cb, band cband, tile cl of cT tiles, sequence length cctx; stream
    // cs = cband * SPW + sp, its KV head ckvh and head chunk cchunk (all wave-uniform)
    int cb = 0, cband = 0, cl = 0, cT = 1, cctx = 0, cs = 0, ckvh = 0, cchunk = 0;
    auto set_stream = [&]() {
        cs = cband * SPW + sp;
        ckvh = cs / a.n_chunks;
        cchunk = cs - ckvh * a.n_chunks;
    };
    if (nk > 0) {
        cb = seq_of_unit_wave(wr0, B, SG, s_pref, L.lane);
        {
            const int Tb = s_pref[cb + 1] - s_pref[cb];
            const int off = wr0 - SG * s_pref[cb];
            cband = off / Tb;
            cl = off - cband * Tb;
        }
        cb = __builtin_amdgcn_readfirstlane(cb);
        cband = __builtin_amdgcn_readfirstlane(cband);
        cl = __builtin_amdgcn_readfirstlane(cl);
        cT = __builtin_amdgcn_readfirstlane(s_pref[cb + 1] - s_pref[cb]);
        cctx = __builtin_amdgcn_readfirstlane(s_ctx[cb]);
        set_stream();
        load_pages(0, cb);
    }
    auto advance = [&]() {
        if (++cl == cT) {
            cl = 0;
            if (++cband == SG) {
                cband = 0;
                do {
                    ++cb;
                } while (cb < B && s_pref[cb + 1] == s_pref[cb]);
                if (cb >= B) cb = B - 1;    // past the last unit; never loaded
                cT = __builtin_amdgcn_readfirstlane(s_pref[cb + 1] - s_pref[cb]);
                cctx = __builtin_amdgcn_readfirstlane(s_ctx[cb]);
            }
            set_stream();
        }
    };
    // Load tile i of the wave (i < nk) with the cursor at it into (kb, vb); when it opens
    // a segment, the segment's query rows come with it (into qr), so a new stream costs
    // no extra round trip.
    auto load_tile = [&](int i, Desc& d, uint4 (&kb)[G::UK], uint32_t (&vb)[4][G::VW], uint4 (&qr)[G::UK]) {
        if ((i & 63) == 0 && i > 0) load_pages(i, cb);
        const int tok = cl * T;
        d.b = cb;
        d.s = cs;
        d.lt = cl;
        d.T = cT;
        d.n_valid = min(T, cctx - tok);
        d.first = (i == 0) || (cl == 0);
        const int phys = __builtin_amdgcn_readlane(btv, i & 63);   // -1: outside the pool
        const size_t base = (size_t)max(phys, 0) * page_bytes + (size_t)(tok & ((1 << ps_log2) - 1)) * tok_bytes;
        size_t base2 = base;
        int phys2 = phys;
        if constexpr (SPLIT) {
            phys2 = __builtin_amdgcn_readlane(btv2, i & 63);
            base2 = (size_t)max(phys2, 0) * page_bytes;
        }
        const char* kbase = a.k + (size_t)ckvh * D * 2;
        const char* vbase = a.v + (size_t)ckvh * D * 2;
        load_kv<D, SPLIT, KROW>(kbase + base, vbase + base, kbase + base2, vbase + base2, koff, voff,
                                (uint32_t)tok_bytes, d.n_valid, phys >= 0, phys2 >= 0, L, kb, vb);
        if (d.first) load_q_raw<D, HP>(a.q, (size_t)cb * a.query_heads + ckvh * a.group + cchunk * HP, L, qr);
    };

    WaveState<D, HP> st;
    uint4 qb[G::UK];       // B operand of the scores (with one tile buffer, also the load target)
    int seg_lt0 = 0;       // first stream tile of the open segment
    int seg_i0 = 0;        // first wave tile of the open segment
    auto consume = [&](const Desc& d, const uint4 (&kb)[G::UK], const uint32_t (&vb)[4][G::VW],
                       const uint4 (&qr)[G::UK], int i) {
        if (d.first) {   // a new segment: its query rows and a fresh state
            fix_q<D, HP>(qr, a.q_sign, L, qb);
            seg_lt0 = d.lt;
            seg_i0 = i;
            st.reset();
        }
        st.template tile<KROW>(qb, kb, vb, d.n_valid, sl2, L, kt);
        if (d.lt == d.T - 1 || i == nk - 1) {   // the segment ends here
            const int kvh = d.s / a.n_chunks;
            const int chunk = d.s - kvh * a.n_chunks;
            const size_t row0 = (size_t)d.b * a.query_heads + kvh * a.group + chunk * HP;
            if (seg_lt0 == 0 && d.lt == d.T - 1) {
                st.write_out(a.out, row0, L);   // the whole stream: finish it
            } else {
                // a piece of a stream that continues in another wave: slot 2 wave for the
                // wave's first segment, 2 wave + 1 for its last one
                const int slot = 2 * li + (seg_i0 == 0 ? 0 : 1);
                st.store_triple(&s_m[slot][0], &s_l[slot][0], reinterpret_cast<float*>(&s_acc[slot][0][0]), L);
                if (L.lane == 0) {
                    // units of this stream's band: [SG pref[b] + band Tb, + Tb); with them,
                    // where the run's result goes
                    const int band = d.s / SPW;
                    const int ubase = SG * s_pref[d.b] + band * d.T;
                    s_meta[slot][0] = int4{d.b * S + d.s, ubase + seg_lt0, ubase + d.lt + 1, ubase};
                    s_meta[slot][1] = int4{ubase + d.T, (int)row0, sp, 0};
                }
            }
        }
    };

    // A wave's two partial slots (2 li, 2 li + 1) start empty -- weight 0, zero sums --
    // so that the combine at the end can fold every slot of a run without first asking
    // which were written.  Done while the wave's first tile's loads are in flight.
    auto clear_my_slots = [&]() {
        for (int i = L.lane; i < 2 * HP * C4; i += 64) {
            const int sl = 2 * li + i / (HP * C4);
            const int rest = i % (HP * C4);
            s_acc[sl][rest / C4][rest % C4] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (L.lane < 2 * HP) {
            s_m[2 * li + L.lane / HP][L.lane % HP] = -INFINITY;
            s_l[2 * li + L.lane / HP][L.lane % HP] = 0.f;
        }
    };
    // The workgroup's two merge records, written by lane 0 of the last wave while its
    // first tile's loads are in flight (or after the loop when it has no tile): they
    // depend only on the split, and computing them costs one lane about a microsecond.
    auto write_records = [&]() {
        if (L.lane != 0) return;
        // [0]: the band holding the last unit, if it starts here and goes on --
        // {sequence, band, pieces n, side of the first piece}; the pieces are this
        // workgroup's and one per following workgroup up to the one holding the band's
        // last unit.  [1]: the band holding the first unit, if that band started in an
        // earlier workgroup o: this workgroup's merge block then takes a share of its
        // tasks -- {sequence, band, 2 o + side of o's piece, n}; n = 0 otherwise.
        int4 own = {0, 0, 0, 0};
        int4 cov = {0, 0, 0, 0};
        if (g1 > g0) {
            int b, band, lt;
            locate_unit(g1 - 1, B, SG, s_pref, b, band, lt);
            const int Tb = s_pref[b + 1] - s_pref[b];
            const int S0 = SG * s_pref[b] + band * Tb;
            const int E = S0 + Tb;
            if (E > g1 && S0 >= g0) own = int4{b, band, wg_of_unit(E - 1, N, NWG) - w + 1, S0 == g0 ? 0 : 1};
        }
        if (g0 < N) {
            int b, band, lt;
            locate_unit(g0, B, SG, s_pref, b, band, lt);
            const int Tb = s_pref[b + 1] - s_pref[b];
            const int S0 = SG * s_pref[b] + band * Tb;
            if (S0 < g0) {
                const int o = wg_of_unit(S0, N, NWG);
                const int n = wg_of_unit(S0 + Tb - 1, N, NWG) - o + 1;
                cov = int4{b, band, 2 * o + (S0 == split_point(o, N, NWG) ? 0 : 1), n};
            }
        }
        a.ws_desc[2 * w] = own;
        a.ws_desc[2 * w + 1] = cov;
        s_rec[0] = own;
        s_rec[1] = cov;
    };
    if (nk > 0) {
        // DEPTH register buffers: tile i + DEPTH - 1 is loaded before tile i is consumed.
        // The loop runs a multiple of DEPTH tiles and has no exit in its middle (see the
        // fixed route); a padding tile (i >= nk) repeats the last load and is not
        // consumed.
        uint4 kb[DEPTH][G::UK];
        uint32_t vb[DEPTH][4][G::VW];
        // query rows of a segment's first tile: loaded straight into the operand when there
        // is one tile buffer (the previous tile is consumed before the next is loaded)
        uint4 qr[DEPTH > 1 ? DEPTH : 1][G::UK];
        Desc dsc[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) {
            if (d > 0 && d < nk) advance();
            load_tile(min(d, nk - 1), dsc[d], kb[d], vb[d], qr[d]);   // DEPTH > 1 only
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
                if constexpr (DEPTH == 1) load_tile(min(inext, nk - 1), dsc[nxt], kb[nxt], vb[nxt], qb);
                else load_tile(min(inext, nk - 1), dsc[nxt], kb[nxt], vb[nxt], qr[nxt]);
                __builtin_amdgcn_sched_barrier(0);
                if (i + d == 0) {
                    clear_my_slots();
                    if (wave == NW - 1) write_records();
                }
                if constexpr (DEPTH == 1) consume(dsc[d], kb[d], vb[d], qb, i + d);
                else if (i + d < nk) consume(dsc[d], kb[d], vb[d], qr[d], i + d);
                else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // see below
            }
        }
        // (The skipped padding tile's loads are waited for on the spot -- this happens
        // only at the very end -- so that no path reaches the loop header with loads
        // outstanding into registers the compiler may reuse; otherwise it inserts waits
        // into every iteration.)
        if (PA_BAL_PRIO) set_wave_priority(0);
    } else {
        // no tiles: empty slots, and the records from the last wave all the same
        clear_my_slots();
        if (wave == NW - 1) write_records();
    }
    __syncthreads();

    // Runs of slots: the non-empty slots of one stream are adjacent (waves of one stream
    // are adjacent, slots are in unit order and a band's units are contiguous).  Every
    // wave finds the run starts itself -- a ballot of the filled slots, each slot's
    // nearest filled neighbour below, a ballot of the starts -- so no barrier follows.
    // Run r spans slots [its start, the next start), or up to NS for the last.
    uint64_t run_starts, filled;
    {
        const int lane = L.lane;
        const int sid = lane < NS ? s_meta[lane][0].x : -1;
        filled = __builtin_amdgcn_ballot_w64(sid >= 0);
        const uint64_t below = filled & ((1ull << lane) - 1ull);
        const int pidx = below ? 63 - __builtin_clzll(below) : 0;
        const int prev_sid = __shfl(sid, pidx);
        run_starts = __builtin_amdgcn_ballot_w64(sid >= 0 && (below == 0 || sid != prev_sid));
    }
    const int nr = __popcll(run_starts);
    // first slot of run r (< nr): the r-th set bit of run_starts, by halving
    auto run_slot = [&](int r) {
        int pos = 0;
#pragma unroll
        for (int wdt = 32; wdt >= 1; wdt >>= 1) {
            const int c = __popcll((run_starts >> pos) & ((1ull << wdt) - 1ull));
            if (c <= r) {
                r -= c;
                pos += wdt;
            }
        }
        return pos;
    };
    if (g1 == g0) {
        // no units: empty triples (weight 0) for a merge whose band spans this
        // workgroup's (empty) range
        const size_t wslot = (size_t)w * 2 * SPW * HP;
        for (int idx = tid; idx < SPW * HP * C4; idx += NT) {
            const int row = idx / C4;
            const int d4 = idx - row * C4;
            reinterpret_cast<float4_t*>(a.ws_acc + (wslot + row) * D)[d4] = float4_t{0.f, 0.f, 0.f, 0.f};
            if (d4 == 0) {
                a.ws_ml[(wslot + row) * 2] = -INFINITY;
                a.ws_ml[(wslot + row) * 2 + 1] = 0.f;
            }
        }
    }

    // Combine each run: HP * C4 / EPT threads per run, EPT float4 elements each, as many
    // runs at once as the block holds.  A stream covered entirely is finished; otherwise it
    // crosses a workgroup boundary and its triple goes to the workspace: side 0 for the
    // band holding the workgroup's first unit, side 1 for the one holding its last unit.
    auto combine = [&](auto ept) {
        constexpr int EPT = decltype(ept)::value;
        constexpr int PER = HP * C4 / EPT;
        constexpr int RPAR = NT / PER;
        static_assert(PER * EPT == HP * C4 && RPAR >= 1, "a run needs HP * D / 4 / EPT threads");
        const int rsub = tid / PER;
        if (rsub >= RPAR) return;
        int h[EPT], d4[EPT];
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            const int e = tid - rsub * PER + j * PER;
            h[j] = e / C4;
            d4[j] = e - h[j] * C4;
        }
        for (int r = rsub; r < nr; r += RPAR) {
            const int s0 = run_slot(r);
            const uint64_t above = s0 < 63 ? run_starts & ~((2ull << s0) - 1ull) : 0ull;
            const int s1 = above ? __builtin_ctzll(above) : NS;
            const int4 m0 = s_meta[s0][0];
            const int4 m1 = s_meta[s0][1];
            const int tb = m0.y;
            int te = -1;
            float M[EPT], Ls[EPT];
            float4_t o[EPT];
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                M[j] = -INFINITY;
                Ls[j] = 0.f;
                o[j] = float4_t{0.f, 0.f, 0.f, 0.f};
            }
            // The run's filled slots (one per wave holding a piece; the slots between them
            // are empty) are read all at once, 3, 6 or 12 at a time; past the last, the
            // first is re-read with weight 0.
            const uint64_t fm0 = filled & (s1 >= 64 ? ~0ull : (1ull << s1) - 1ull) & ~((1ull << s0) - 1ull);
            const int nf = __popcll(fm0);
            auto fold_slots = [&](auto kf) {
                constexpr int KF = decltype(kf)::value;
                uint64_t fm = fm0;
                int sl[KF];
#pragma unroll
                for (int k = 0; k < KF; ++k) {
                    sl[k] = k < nf ? __builtin_ctzll(fm) : s0;
                    fm &= fm - 1ull;
                    te = max(te, k < nf ? s_meta[sl[k]][0].z : -1);
                }
#pragma unroll
                for (int j = 0; j < EPT; ++j) {
                    float mk[KF], lk[KF];
                    float4_t ak[KF];
#pragma unroll
                    for (int k = 0; k < KF; ++k) {
                        mk[k] = k < nf ? s_m[sl[k]][h[j]] : -INFINITY;
                        lk[k] = s_l[sl[k]][h[j]];
                        ak[k] = s_acc[sl[k]][h[j]][d4[j]];
                        M[j] = fmaxf(M[j], mk[k]);
                    }
#pragma unroll
                    for (int k = 0; k < KF; ++k) {
                        const float f = fast_exp2(mk[k] - M[j]);
                        Ls[j] += f * lk[k];
                        o[j] += f * ak[k];
                    }
                }
            };
            // (a thread holds at most 12 slots: with 2 or 4 elements it is never given runs
            // of more than 6 or 3 filled slots, and those folds are not compiled)
            bool done = false;
            if (nf <= 3) {
                fold_slots(IntC<3>());
                done = true;
            }
            if constexpr (EPT <= 2) {
                if (!done && nf <= 6) {
                    fold_slots(IntC<6>());
                    done = true;
                }
            }
            if constexpr (EPT == 1) {
                if (!done && nf <= 12) {
                    fold_slots(IntC<12>());
                    done = true;
                }
            }
            if (!done) {   // (more than 12 waves per stream)
                for (uint64_t mm = fm0; mm; mm &= mm - 1ull) te = max(te, s_meta[__builtin_ctzll(mm)][0].z);
#pragma unroll
                for (int j = 0; j < EPT; ++j) {
                    for (uint64_t mm = fm0; mm; mm &= mm - 1ull) M[j] = fmaxf(M[j], s_m[__builtin_ctzll(mm)][h[j]]);
                    for (uint64_t mm = fm0; mm; mm &= mm - 1ull) {
                        const int sl = __builtin_ctzll(mm);
                        const float f = fast_exp2(s_m[sl][h[j]] - M[j]);
                        Ls[j] += f * s_l[sl][h[j]];
                        o[j] += f * s_acc[sl][h[j]][d4[j]];
                    }
                }
            }
            const int U0 = m0.w;
            const int spr = m1.z;
            const size_t row0 = (size_t)m1.y;
            const bool complete = tb == U0 && te == m1.x;
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                if (complete) {
                    reinterpret_cast<float4_t*>(a.out + (row0 + h[j]) * D)[d4[j]] = o[j] / Ls[j];
                } else {
                    const size_t wrow = (((size_t)w * 2 + (tb == g0 ? 0 : 1)) * SPW + spr) * HP + h[j];
                    reinterpret_cast<float4_t*>(a.ws_acc + wrow * D)[d4[j]] = o[j];
                    if (d4[j] == 0) {
                        a.ws_ml[wrow * 2] = M[j];
                        a.ws_ml[wrow * 2 + 1] = Ls[j];
                    }
                }
            }
        }
    };
    // Elements per thread: one, unless the runs outnumber the block's run groups; then 2 or
    // 4, so that every run is folded in one pass, as long as a thread holds at most 12
    // slots of pieces (a run has one filled slot per wave of its stream).
    {
        constexpr int RPAR1 = NT / (HP * C4);
        const int kfmax = RW <= 3 ? 3 : RW <= 6 ? 6 : 12;
        if (nr > RPAR1 && NT / (HP * C4 / 2) >= nr && 2 * kfmax <= 12) combine(IntC<2>());
        else if (nr > RPAR1 && (HP * C4) % 4 == 0 && 4 * kfmax <= 12) combine(IntC<4>());
        else combine(IntC<1>());
    }
    if constexpr (MODE == kModeSingle) single_launch_merge<D, HP, NT>(a, w, NWG, SPW, s_rec, s_last);
}

// Merge of the balanced route.  Workgroup w of the decode kernel owns the band that
// holds its last unit when that band starts in w and goes on past it (each crossing band
// has exactly one owner); the pieces of stream sp, head h of such a band are rows
// r(0) = ((w * 2 + side) * spw + sp) * HP + h of workgroup w and, for p >= 1,
// r(p) = ((w + p) * 2 * spw + sp) * HP + h (side 0 of the following workgroups).  Merge
// block x reads workgroup x's two records
// (written by the decode kernel, no search here): the band it owns and the band that
// covers its first unit.  A band spanning n workgroups has rows x (D / 32) tasks -- one
// row, 128 bytes of columns -- and block o + j of its n blocks takes the j-th of n equal
// shares, so the loads of every band are spread over all blocks it spans:
//   * bands of at most kShortMerge pieces: one thread per (task, float4 column) loads all
//     pieces at once; the block's shares of both its bands form one task list, taken 1, 2
//     or 4 tasks per thread so that it usually needs one pass;
//   * longer bands: the pieces of a task are split over groups of kLongUnroll, one group
//     per thread, and the groups are combined through lane shuffles (and LDS when a task
//     spans several waves).
// Every load of a pass is issued before any of its results is used: one round trip per
// pass.
template <int D, int HP>
__global__ void __launch_bounds__(kMergeThreads)
pa_merge_balanced(DecodeArgs a) {
    constexpr int C4 = D / 4;
    constexpr int SC = kSliceCols;                  // float4 columns per task
    constexpr int NSL = C4 / SC;                    // tasks per row
    static_assert(C4 % SC == 0, "a row is a whole number of tasks");
    const int x = blockIdx.x;
    const int tid = threadIdx.x;
    const int rows = a.spw * HP;
    const int T = rows * NSL;                       // tasks of one band
    const uint32_t row_bytes = (uint32_t)D * 4u;
    const uint32_t acc_wg = (uint32_t)(2 * rows) * row_bytes;      // bytes per workgroup
    const uint32_t ml_wg = (uint32_t)(2 * rows) * 8u;
    const char* acc0 = reinterpret_cast<const char*>(a.ws_acc);
    const char* ml0 = reinterpret_cast<const char*>(a.ws_ml);
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    auto out_ptr = [&](int b, int band, int row, int col4) {
        const int sp = row / HP;
        const int h = row - sp * HP;
        const int s = band * a.spw + sp;
        const int kvh = s / a.n_chunks;
        const int chunk = s - kvh * a.n_chunks;
        return reinterpret_cast<float4_t*>(a.out + ((size_t)b * a.query_heads + kvh * a.group + chunk * HP + h) * D) + col4;
    };
    // the records are block-uniform: said so, so that everything derived from them (buffer
    // resources, scalar offsets) stays in scalar registers
    auto uniform4 = [](int4 v) {
        return int4{__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                    __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w)};
    };
    const int4 d = uniform4(a.ws_desc[2 * x]);      // own band {b, band, n, side}, n = 0: none
    const int4 cv = uniform4(a.ws_desc[2 * x + 1]); // covering band {b, band, 2 o + side, n}
    const int n_o = d.z, n_c = cv.w;
    const int o_c = cv.z >> 1;
    const int own_hi = n_o > 0 ? T / n_o : 0;       // own share: tasks [0, own_hi)
    const int cov_lo = n_c > 0 ? (x - o_c) * T / n_c : 0;
    const int cov_hi = n_c > 0 ? (x - o_c + 1) * T / n_c : 0;
    const bool own_short = n_o > 0 && n_o <= kShortMerge;
    const bool cov_short = n_c > 0 && n_c <= kShortMerge;

    // Short bands: both shares in one list of tasks, one thread per (task, column).  The
    // pieces of both bands lie in workgroups base .. end - 1 (a covering band that goes on
    // past x leaves x no band of its own), one buffer resource spans them; the lane's
    // (band, row, column) part of an offset is a register, the piece's a scalar.
    if (own_short || cov_short) {
        const int na = own_short ? own_hi : 0;
        const int tot = na + (cov_short ? cov_hi - cov_lo : 0);
        const int base = cov_short ? o_c : x;
        const int end = own_short ? x + n_o : o_c + n_c;
        const int nmax = max(own_short ? n_o : 0, cov_short ? n_c : 0);
        const __amdgpu_buffer_rsrc_t racc = tile_rsrc(acc0 + (size_t)base * acc_wg, (int)((end - base) * acc_wg));
        const __amdgpu_buffer_rsrc_t rml = tile_rsrc(ml0 + (size_t)base * ml_wg, (int)((end - base) * ml_wg));
        const int col = tid % SC;
        constexpr int TPP = kMergeThreads / SC;     // tasks per pass and task slot
        // A thread takes KT tasks (v, v + TPP, ...) of KP pieces each (KT * KP =
        // kShortMerge registers of pieces), all loads first: one round trip per pass.
        auto pass = [&](auto kt, auto kp) {
            constexpr int KT = decltype(kt)::value;
            constexpr int KP = decltype(kp)::value;
            for (int v0 = tid / SC; v0 < tot; v0 += TPP * KT) {
                float4_t pa[KT][KP];
                f32x2_t pml[KT][KP];
                int n[KT], row[KT], col4[KT];
                bool in_own[KT];
#pragma unroll
                for (int j = 0; j < KT; ++j) {
                    const int v = v0 + j * TPP;
                    in_own[j] = v < na;
                    const int task = in_own[j] ? v : cov_lo + (v - na);
                    row[j] = task / NSL;
                    col4[j] = (task - row[j] * NSL) * SC + col;
                    const int o = in_own[j] ? x : o_c;
                    const int side = in_own[j] ? d.w : (cv.z & 1);
                    n[j] = v < tot ? (in_own[j] ? n_o : n_c) : 0;
                    // a slot past the last task loads from past the resources: zeros
                    const uint32_t la = v < tot ? (uint32_t)(o - base) * acc_wg + (uint32_t)row[j] * row_bytes + 16u * col4[j] : kPastRange;
                    const uint32_t lm = v < tot ? (uint32_t)(o - base) * ml_wg + (uint32_t)row[j] * 8u : kPastRange;
                    pa[j][0] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(racc, (int)(la + (uint32_t)side * rows * row_bytes), 0, 0));
                    pml[j][0] = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rml, (int)(lm + (uint32_t)side * rows * 8u), 0, 0));
                    // Pieces past a band's last are zeros past the resource or data of
                    // other workgroups; they are masked below.  (Scalar offsets are
                    // wave-uniform; readfirstlane keeps the compiler from carrying them in
                    // vector registers.  The whole vector is reinterpreted: bit-casting
                    // single elements of the load's result made clang read one dword for
                    // both.)
#pragma unroll
                    for (int p = 1; p < KP; ++p) {
                        pa[j][p] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(racc, (int)la, __builtin_amdgcn_readfirstlane((int)(p * acc_wg)), 0));
                        pml[j][p] = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rml, (int)lm, __builtin_amdgcn_readfirstlane((int)(p * ml_wg)), 0));
                    }
                }
#pragma unroll
                for (int j = 0; j < KT; ++j) {
                    if (n[j] == 0) continue;
                    float M = -INFINITY;
#pragma unroll
                    for (int p = 0; p < KP; ++p)
                        if (p < n[j]) M = fmaxf(M, pml[j][p].x);
                    float Ls = 0.f;
                    float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int p = 0; p < KP; ++p)
                        if (p < n[j]) {
                            const float e = fast_exp2(pml[j][p].x - M);
                            Ls += e * pml[j][p].y;
                            acc += e * pa[j][p];
                        }
                    *out_ptr(in_own[j] ? d.x : cv.x, in_own[j] ? d.y : cv.y, row[j], col4[j]) = acc / Ls;
                }
            }
        };
        // pieces per task: the band's count rounded up to 4, 8 or 16; tasks per thread:
        // as few as cover the block's tasks in one pass, within 16 pieces
        static_assert(kShortMerge == 16, "the pass shapes below hold 16 pieces per thread");
        const int slots = (tot + TPP - 1) / TPP;
        if (nmax <= 4) {
            if (slots <= 1) pass(IntC<1>(), IntC<4>());
            else if (slots <= 2) pass(IntC<2>(), IntC<4>());
            else pass(IntC<4>(), IntC<4>());
        } else if (nmax <= 8) {
            if (slots <= 1) pass(IntC<1>(), IntC<8>());
            else pass(IntC<2>(), IntC<8>());
        } else {
            pass(IntC<1>(), IntC<16>());
        }
    }

    // Long bands, one at a time: a task takes SC * PG threads (PG a power of two, groups
    // of kLongUnroll pieces), kMergeThreads / (SC * PG) tasks per pass.
    __shared__ float s_rm[kMergeThreads / 64][SC];
    __shared__ float s_rl[kMergeThreads / 64][SC];
    __shared__ float4_t s_ro[kMergeThreads / 64][SC];
#pragma unroll 1
    for (int t = 0; t < 2; ++t) {
        const bool own = t == 0;
        const int n = own ? n_o : n_c;
        if (n <= kShortMerge) continue;
        const int o = own ? x : o_c;
        const int side = own ? d.w : (cv.z & 1);
        const int b = own ? d.x : cv.x;
        const int band = own ? d.y : cv.y;
        const int lo = own ? 0 : cov_lo;
        const int hi = own ? own_hi : cov_hi;
        int pg2 = 1;
        while (pg2 * kLongUnroll < n && pg2 * SC < kMergeThreads) pg2 <<= 1;
        const int tpt = pg2 * SC;                   // threads per task
        const int tl = tid / tpt;
        const int pg = (tid / SC) % pg2;
        const int col = tid % SC;
        const int wave = tid >> 6;
        const __amdgpu_buffer_rsrc_t racc = tile_rsrc(acc0 + (size_t)o * acc_wg, (int)(n * acc_wg));
        const __amdgpu_buffer_rsrc_t rml = tile_rsrc(ml0 + (size_t)o * ml_wg, (int)(n * ml_wg));
        for (int t0 = lo; t0 < hi; t0 += kMergeThreads / tpt) {
            // threads past the last task load from past the resources: zeros, no traffic
            const bool live = t0 + tl < hi;
            const int task = live ? t0 + tl : lo;
            const int row = task / NSL;
            const int col4 = (task - row * NSL) * SC + col;
            const uint32_t la = live ? (uint32_t)row * row_bytes + 16u * col4 : kPastRange;
            const uint32_t lm = live ? (uint32_t)row * 8u : kPastRange;
            float m = -INFINITY, l = 0.f;
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
            for (int q = 0; q < n; q += pg2 * kLongUnroll) {
                const int p0 = q + pg * kLongUnroll;                    // this thread's first piece
                const uint32_t va = la + (p0 == 0 ? (uint32_t)side * rows * row_bytes : (uint32_t)p0 * acc_wg);
                const uint32_t vm = lm + (p0 == 0 ? (uint32_t)side * rows * 8u : (uint32_t)p0 * ml_wg);
                const uint32_t va1 = la + (uint32_t)p0 * acc_wg;
                const uint32_t vm1 = lm + (uint32_t)p0 * ml_wg;
                float4_t pa[kLongUnroll];
                f32x2_t pml[kLongUnroll];
                pa[0] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(racc, (int)va, 0, 0));
                pml[0] = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rml, (int)vm, 0, 0));
#pragma unroll
                for (int k = 1; k < kLongUnroll; ++k) {
                    pa[k] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(racc, (int)va1, __builtin_amdgcn_readfirstlane((int)(k * acc_wg)), 0));
                    pml[k] = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rml, (int)vm1, __builtin_amdgcn_readfirstlane((int)(k * ml_wg)), 0));
                }
                // Pieces past the band's last are zeros past the resource: their maximum is
                // made -inf, so they weigh 0.  No branch: a load used only under a branch
                // is moved into it by the compiler, a second round trip.
                float mk[kLongUnroll];
                float M = m;
#pragma unroll
                for (int k = 0; k < kLongUnroll; ++k) {
                    mk[k] = p0 + k < n ? pml[k].x : -INFINITY;
                    M = fmaxf(M, mk[k]);
                }
                const float Ms = M == -INFINITY ? 0.f : M;
                const float a0 = fast_exp2(m - Ms);
                l *= a0;
                acc *= a0;
#pragma unroll
                for (int k = 0; k < kLongUnroll; ++k) {
                    const float e = fast_exp2(mk[k] - Ms);
                    l += e * pml[k].y;
                    acc += e * pa[k];
                }
                m = M;
            }
            // groups of one task: lanes pg * SC + col of its waves
            for (int s = SC; s < min(64, tpt); s <<= 1) {
                const float m2 = __shfl_xor(m, s);
                const float l2 = __shfl_xor(l, s);
                const float4_t o2 = {__shfl_xor(acc.x, s), __shfl_xor(acc.y, s), __shfl_xor(acc.z, s), __shfl_xor(acc.w, s)};
                fold_triple(m, l, acc, m2, l2, o2);
            }
            if (tpt > 64) {                         // several waves per task: through LDS
                if ((tid & 63) < SC) {
                    s_rm[wave][col] = m;
                    s_rl[wave][col] = l;
                    s_ro[wave][col] = acc;
                }
                __syncthreads();
                const int wpt = tpt / 64;
                if (tid < (kMergeThreads / tpt) * SC) {
                    const int w0 = (tid / SC) * wpt;
                    m = s_rm[w0][col];
                    l = s_rl[w0][col];
                    acc = s_ro[w0][col];
                    for (int k = 1; k < wpt; ++k) fold_triple(m, l, acc, s_rm[w0 + k][col], s_rl[w0 + k][col], s_ro[w0 + k][col]);
                    const int tk = t0 + tid / SC;
                    const int rk = tk / NSL;
                    if (tk < hi) *out_ptr(b, band, rk, (tk - rk * NSL) * SC + col) = acc / l;
                }
                __syncthreads();                    // the shared arrays are reused by the next pass
            } else if (pg == 0 && live) {
                *out_ptr(b, band, row, col4) = acc / l;
            }
        }
    }
}

// PA_FLAG_DEBUG_BOUNDS: word w of the bitmap holds the bits of table entries 32 w ..
// 32 w + 31 (row-major, b * max_pages + logical page) that a context dereferences (logical
// page < ceil(ctx[b] / page_size)) and that lie outside the pool.  One thread writes each
// word whole, so the bitmap needs no clearing pass and no atomics.
__global__ void __launch_bounds__(256)
pa_bad_entries_kernel(const int32_t* bt, const int32_t* ctx, int max_pages, int ps_log2, int num_pages,
                      uint32_t* bits, long long words, long long entries) {
    const long long w = (long long)blockIdx.x * 256 + threadIdx.x;
    if (w >= words) return;
    uint32_t word = 0;
    for (int i = 0; i < 32; ++i) {
        const long long e = 32 * w + i;
        if (e >= entries) break;
        const long long b = e / max_pages;
        const long long lp = e - b * max_pages;
        const long long pages = ((long long)ctx[b] + (1 << ps_log2) - 1) >> ps_log2;
        if (lp < pages && (uint32_t)bt[e] >= (uint32_t)num_pages) word |= 1u << i;
    }
    bits[w] = word;
}

#ifndef PA_WAVES
#define PA_WAVES kFixedWaves   // waves per decode workgroup (fixed route)
#endif
#ifndef PA_DEPTH
// tile buffers per wave (fixed route): one buffer leaves registers for more resident waves;
// measured against two (4 waves per workgroup, partitions of 1024): batch64 77.0 vs
// 83.5 us, long100k 49.9 vs 51.1, mixed128 281.6 vs 300.6; 8 or 12 waves were no faster
#define PA_DEPTH 1
#endif
#ifndef PA_BAL_DEPTH
#define PA_BAL_DEPTH 1   // tile buffers per wave (balanced route)
#endif
constexpr int kWaves = PA_WAVES;
constexpr int kWavesWide = kFixedWavesWide;   // fixed route, at most one workgroup per compute unit
constexpr int kDepth = PA_DEPTH;
constexpr int kBalDepth = PA_BAL_DEPTH;

int balanced_grid() { return device_compute_units(); }

// LDS a gfx950 workgroup may use (the CU's 160 KB).
constexpr size_t kLdsPerWorkgroup = 160 * 1024;

// Static LDS bytes of a kernel (host-side query; nothing is enqueued).
template <typename K>
size_t static_lds_bytes(K kern) {
    hipFuncAttributes attr{};
    if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kern)) != hipSuccess) return SIZE_MAX;
    return attr.sharedSizeBytes;
}

template <int D, int HP, int NW, bool SPLIT>
hipError_t launch_balanced_nw(const Plan& pl, const DecodeArgs& args, int ws_slots, hipStream_t stream) {
    // Whole-row K loads (staged through LDS) were measured faster at every head count
    // (serving shape with 4 heads per wave: -1.1 us per call; long context, 6 heads:
    // -0.7 us; mixed batch, 8 heads: -3 us).  Their 55 KB of staging is used when the
    // kernel's LDS still fits next to the per-sequence arrays; otherwise K is loaded in
    // the MFMA layout.
    // (the staging is per wave: with 16 waves it would not fit next to the partial slots)
    constexpr bool kRow = PA_KROW && D == 128 && NW <= 12;
    const size_t lds = (size_t)(2 * pl.prob.batch + 1) * sizeof(int);
    static const size_t row_static = static_lds_bytes(pa_decode_balanced<D, HP, kBalDepth, NW, SPLIT, kRow, kModeSplit>);
    const bool use_row = row_static != SIZE_MAX && row_static + lds <= kLdsPerWorkgroup;
    const auto pick = [&](auto mode) {
        constexpr int M = decltype(mode)::value;
        return use_row ? pa_decode_balanced<D, HP, kBalDepth, NW, SPLIT, kRow, M>
                       : pa_decode_balanced<D, HP, kBalDepth, NW, SPLIT, false, M>;
    };
    const auto kern = args.single_launch ? pick(IntC<kModeSingle>()) : pick(IntC<kModeSplit>());
    const int grid = balanced_grid();
    if (grid <= 0) return hipErrorInvalidDevice;
    if (grid > ws_slots) return hipErrorInvalidValue;   // the workspace holds fewer workgroups' rows
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NW * 64), lds, stream, args);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || args.single_launch) return err;
    hipLaunchKernelGGL((pa_merge_balanced<D, HP>), dim3((unsigned)grid), dim3(kMergeThreads), 0, stream, args);
    return hipGetLastError();
}

template <int D, int HP, bool SPLIT>
hipError_t launch_balanced(const Plan& pl, const DecodeArgs& args, int ws_slots, hipStream_t stream) {
    switch (pl.bal_waves) {
        case 12: return launch_balanced_nw<D, HP, 12, SPLIT>(pl, args, ws_slots, stream);
#ifdef PA_BAL_WAVES
        case 8: return launch_balanced_nw<D, HP, 8, SPLIT>(pl, args, ws_slots, stream);
        case 16: return launch_balanced_nw<D, HP, 16, SPLIT>(pl, args, ws_slots, stream);
#endif
        default: return hipErrorInvalidValue;
    }
}

template <int D, int HP>
hipError_t launch_decode(const Plan& pl, const DecodeArgs& args, int ws_slots, hipStream_t stream) {
    const bool split = pl.prob.page_size < 16;
    if (pl.balanced)
        return split ? launch_balanced<D, HP, true>(pl, args, ws_slots, stream)
                     : launch_balanced<D, HP, false>(pl, args, ws_slots, stream);
    // Fixed partitions: with no more workgroups than compute units, 8 waves per workgroup
    // share a partition's tiles; otherwise 4, so that more workgroups stay resident per
    // CU.  (Partitions of 1024: small_batch, 256 workgroups, 24.7 -> 21.4 us with 8 waves;
    // batch64, long100k and mixed128, with 2 to 16 workgroups per CU, were slower with 8.)
    const int cus = device_compute_units();
    const bool wide = cus > 0 && pl.decode_grid <= cus;
    const dim3 grid((unsigned)pl.decode_grid);
    if (wide) {
        if (!split) hipLaunchKernelGGL((pa_decode_kernel<D, HP, kDepth, kWavesWide, false>), grid, dim3(kWavesWide * 64), 0, stream, args);
        else hipLaunchKernelGGL((pa_decode_kernel<D, HP, kDepth, kWavesWide, true>), grid, dim3(kWavesWide * 64), 0, stream, args);
    } else {
        if (!split) hipLaunchKernelGGL((pa_decode_kernel<D, HP, kDepth, kWaves, false>), grid, dim3(kWaves * 64), 0, stream, args);
        else hipLaunchKernelGGL((pa_decode_kernel<D, HP, kDepth, kWaves, true>), grid, dim3(kWaves * 64), 0, stream, args);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const Plan& pl, const DecodeArgs& args, int ws_slots, hipStream_t stream) {
    static_assert(kMaxHeadsPerWave == 8, "instantiations below cover 1..8 heads");
    switch (pl.heads_per_wg) {
        case 1: return launch_decode<D, 1>(pl, args, ws_slots, stream);
        case 2: return launch_decode<D, 2>(pl, args, ws_slots, stream);
        case 3: return launch_decode<D, 3>(pl, args, ws_slots, stream);
        case 4: return launch_decode<D, 4>(pl, args, ws_slots, stream);
        case 5: return launch_decode<D, 5>(pl, args, ws_slots, stream);
        case 6: return launch_decode<D, 6>(pl, args, ws_slots, stream);
        case 7: return launch_decode<D, 7>(pl, args, ws_slots, stream);
        case 8: return launch_decode<D, 8>(pl, args, ws_slots, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

namespace {
constexpr int kMaxDevices = 256;
std::atomic<int> g_cus[kMaxDevices];   // 0: not asked yet
}  // namespace

int device_compute_units() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 0;
    cus = cus < kMaxBalancedWG ? cus : kMaxBalancedWG;
    if (dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

hipError_t launch(const Plan& pl, const void* q, const void* k, const void* v,
                  const int32_t* block_tables, const int32_t* ctx, float scale, float* out,
                  void* workspace, const WsLayout& layout, hipStream_t stream) {
    const pa_problem& p = pl.prob;
    // the single-launch merge folds at most kArrivalGroup groups of kArrivalGroup pieces, so
    // a band may span at most that many workgroups (checked before anything is enqueued)
    if (pl.single_launch && pl.balanced &&
        device_compute_units() > kArrivalGroup * kArrivalGroup)
        return hipErrorInvalidConfiguration;
    float* ws_acc = nullptr;
    float* ws_ml = nullptr;
    int4* ws_desc = nullptr;
    if (pl.need_merge) {
        ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + layout.acc_offset);
        ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + layout.ml_offset);
        if (pl.balanced) ws_desc = reinterpret_cast<int4*>(static_cast<char*>(workspace) + layout.desc_offset);
    }
    int* ws_cnt = pl.single_launch ? reinterpret_cast<int*>(static_cast<char*>(workspace) + layout.cnt_offset)
                                   : nullptr;
    if (pl.debug_bounds) {
        const long long words = (long long)layout.bitmap_words;
        hipLaunchKernelGGL(pa_bad_entries_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                           block_tables, ctx, p.max_pages_per_sequence, pl.ps_log2, p.num_physical_pages,
                           static_cast<uint32_t*>(workspace), words,
                           (long long)p.batch * p.max_pages_per_sequence);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
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
    da.ws_cnt = ws_cnt;
    da.single_launch = pl.single_launch ? 1 : 0;
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
    da.spw = pl.spw;
    da.waves_per_stream = pl.waves_per_stream;
    da.bands = pl.bands;
    da.num_pages = p.num_physical_pages;

    hipError_t err = (p.head_dim == 128) ? launch_decode_d<128>(pl, da, layout.wg_slots, stream)
                                         : launch_decode_d<64>(pl, da, layout.wg_slots, stream);
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
    if (pl.n_part_max <= kRowFoldMax) {
        const int rows = (int)pl.merge_grid;   // batch * query_heads
        const int rpb = kMergeThreads / (p.head_dim / 4);
        const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
        if (p.head_dim == 128)
            hipLaunchKernelGGL(pa_merge_rows_kernel<128>, grid, dim3(kMergeThreads), 0, stream, ma, rows);
        else
            hipLaunchKernelGGL(pa_merge_rows_kernel<64>, grid, dim3(kMergeThreads), 0, stream, ma, rows);
    } else if (p.head_dim == 128) {
        hipLaunchKernelGGL(pa_merge_kernel<128>, dim3((unsigned)pl.merge_grid), dim3(kMergeThreads), 0,
                           stream, ma);
    } else {
        hipLaunchKernelGGL(pa_merge_kernel<64>, dim3((unsigned)pl.merge_grid), dim3(kMergeThreads), 0,
                           stream, ma);
    }
    return hipGetLastError();
}

}  // namespace pa
