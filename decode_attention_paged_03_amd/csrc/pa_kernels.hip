// pa_kernels.hip -- gfx950 (CDNA4) kernels of one paged-attention decode step.
//
// Two kernels:
//
//  * pa_decode_kernel: one workgroup per (sequence, KV head, head chunk, partition).
//    Its waves stream the partition's K/V rows through the block table with 128-bit
//    fp16 loads (the block-table gather of the "Baseline" and "V3 (Shared memory data
//    reuse)" sections of "[TIL] Optimizing paged attention"), score them against every
//    query head of the GQA group held in registers -- one K/V read serves the whole
//    group, which is what V3 achieves by staging a page in shared memory -- and keep a
//    streaming softmax state (running max, running sum, unnormalised output) per head,
//    the online recurrence of that page's Baseline kernel.  A sequence that fits one
//    partition is finished here (the single-tile path of the
//    "paged_attention_v2_pytorch.py" commit page); otherwise the workgroup writes its
//    partition's (max, sum, acc) triple, as the V4 split kernel does.
//
//  * pa_merge_kernel: per (sequence, query head) with more than one partition,
//    combines the partition triples: M = max m_p, L = sum exp(m_p - M) l_p,
//    out = sum exp(m_p - M) acc_p / L (the V4 merge kernel's combination, evaluated
//    with the global maximum first and the division once at the end, as the phase-2
//    reduction of the commit page does).
//
// Scores are kept in base-2 units: s = (q . k) * scale * log2(e), so every exponential
// is the hardware exp2 (v_exp_f32).
//
// Register layout of one wave (64 lanes) for head_dim D: a K or V row (D fp16 = D*2
// bytes) is spread over LR = D/8 lanes, 16 bytes (8 dims) per lane, so one 128-bit load
// instruction covers NR = 64/LR consecutive tokens of one page.  A lane keeps the query
// dims it needs for every head of its chunk (8 per head) and the output accumulator for
// the same 8 dims per head.  A token's dot product is finished by an all-reduce over
// its LR lanes with DPP (quad_perm, row_half_mirror, row_mirror), which leaves the same
// bits in every lane of the row, so the rows of a wave run independent softmax streams
// over disjoint token subsets with no cross-lane traffic until the epilogue.
#include <hip/hip_runtime.h>

#include <math.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
    const _Float16* q;
    const _Float16* k;
    const _Float16* v;
    const int32_t* bt;
    const int32_t* ctx;
    float* out;
    float* ws_acc;   // [batch][query_heads][n_part_max][D]
    float* ws_ml;    // [batch][query_heads][n_part_max][2] = (max in log2 units, sum)
    float scale_log2;
    int query_heads, kv_heads, group, n_chunks, max_pages, partition, n_part_max, ps_log2;
    int force_split;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over groups of LR consecutive lanes (LR = 8 or 16); every lane of a group gets
// the identical sum (each step adds two operands that are exchanged between partner
// lanes, and IEEE addition is commutative).
template <int LR>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm(1,0,3,2): partner lane ^1
    x += dpp<0x4E>(x);   // quad_perm(2,3,0,1): partner lane ^2
    x += dpp<0x141>(x);  // row_half_mirror: lane i <-> 7-i within 8
    if constexpr (LR == 16) x += dpp<0x140>(x);  // row_mirror: lane i <-> 15-i within 16
    return x;
}

__device__ __forceinline__ float dot8(const uint4& a, const uint4& b) {
    float c = 0.f;
    c = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a.x), __builtin_bit_cast(half2_t, b.x), c, false);
    c = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a.y), __builtin_bit_cast(half2_t, b.y), c, false);
    c = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a.z), __builtin_bit_cast(half2_t, b.z), c, false);
    c = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a.w), __builtin_bit_cast(half2_t, b.w), c, false);
    return c;
}

__device__ __forceinline__ void unpack8(const uint4& x, float (&f)[8]) {
    half2_t h;
    h = __builtin_bit_cast(half2_t, x.x); f[0] = (float)h.x; f[1] = (float)h.y;
    h = __builtin_bit_cast(half2_t, x.y); f[2] = (float)h.x; f[3] = (float)h.y;
    h = __builtin_bit_cast(half2_t, x.z); f[4] = (float)h.x; f[5] = (float)h.y;
    h = __builtin_bit_cast(half2_t, x.w); f[6] = (float)h.x; f[7] = (float)h.y;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// D: head_dim; HP: query heads per workgroup; U: 128-bit loads per K (and V) tile per
// lane; NW: waves per workgroup.
template <int D, int HP, int U, int NW>
__global__ void __launch_bounds__(NW * 64)
pa_decode_kernel(DecodeArgs a) {
    constexpr int LR = D / 8;       // lanes per K/V row
    constexpr int NR = 64 / LR;     // rows (tokens) per load instruction
    constexpr int T = NR * U;       // tokens per wave tile
    constexpr int C4 = D / 4;       // float4 columns of an output row

    __shared__ int s_bt[kMaxPartitionPages];
    __shared__ float s_m[NW][HP];
    __shared__ float s_l[NW][HP];
    __shared__ float4_t s_acc[NW][HP][C4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane % LR;
    const int r = lane / LR;

    int id = blockIdx.x;
    const int chunk = id % a.n_chunks; id /= a.n_chunks;
    const int kvh = id % a.kv_heads;   id /= a.kv_heads;
    const int part = id % a.n_part_max; id /= a.n_part_max;
    const int b = id;

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
    const int ps_mask = (1 << ps_log2) - 1;
    const int pg0 = t_begin >> ps_log2;
    const int npg = ((t_end - 1) >> ps_log2) - pg0 + 1;
    const int32_t* bt_row = a.bt + (size_t)b * a.max_pages + pg0;
    for (int i = tid; i < npg; i += NW * 64) s_bt[i] = bt_row[i];

    // Query dims [8c, 8c+8) of each head of the chunk.
    uint4 qv[HP];
    {
        const uint4* qp = reinterpret_cast<const uint4*>(a.q + row0 * D) + c;
#pragma unroll
        for (int h = 0; h < HP; ++h) qv[h] = qp[h * (D / 8)];
    }
    __syncthreads();

    const size_t tok_stride = (size_t)a.kv_heads * D;       // fp16 elements between slots
    const _Float16* kbase = a.k + (size_t)kvh * D + c * 8;
    const _Float16* vbase = a.v + (size_t)kvh * D + c * 8;
    const float sl2 = a.scale_log2;

    float m[HP], l[HP], acc[HP][8];
#pragma unroll
    for (int h = 0; h < HP; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
    }

    const int n_tok = t_end - t_begin;
    const int n_tiles = (n_tok + T - 1) / T;
    // This wave takes tiles wave, wave + NW, ...
    const int nk = wave < n_tiles ? (n_tiles - wave + NW - 1) / NW : 0;

    // Issue the loads of the wave's k-th tile.  Token indices past the partition end are
    // clamped to its last token, so every address is a valid row of a referenced page;
    // their scores are masked to -inf below.
    auto load_tile = [&](int k, uint4 (&kb)[U], uint4 (&vb)[U]) {
        const int t0 = t_begin + (wave + k * NW) * T;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tu = min(t0 + u * NR, t_end - 1);          // wave-uniform
            const int tl = min(t0 + u * NR + r, t_end - 1);      // same page as tu
            const int phys = __builtin_amdgcn_readfirstlane(s_bt[(tu >> ps_log2) - pg0]);
            const size_t off = (((size_t)phys << ps_log2) | (size_t)(tl & ps_mask)) * tok_stride;
            kb[u] = *reinterpret_cast<const uint4*>(kbase + off);
            vb[u] = *reinterpret_cast<const uint4*>(vbase + off);
        }
    };

    auto compute_tile = [&](int k, const uint4 (&kb)[U], const uint4 (&vb)[U]) {
        const int t0 = t_begin + (wave + k * NW) * T;
        float s[U][HP];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int h = 0; h < HP; ++h) s[u][h] = group_sum<LR>(dot8(qv[h], kb[u])) * sl2;
        if (t0 + T > t_end) {   // partial tile (wave-uniform branch)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (t0 + u * NR + r >= t_end) {
#pragma unroll
                    for (int h = 0; h < HP; ++h) s[u][h] = -INFINITY;
                }
            }
        }
        float vf[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) unpack8(vb[u], vf[u]);
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            float mt = s[0][h];
#pragma unroll
            for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u][h]);
            const float mn = fmaxf(m[h], mt);
            const float ms = (mn == -INFINITY) ? 0.f : mn;   // keeps exp2 arguments non-NaN
            const float alpha = fast_exp2(m[h] - ms);
            m[h] = mn;
            l[h] *= alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[h][j] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = fast_exp2(s[u][h] - ms);
                l[h] += p;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(p, vf[u][j], acc[h][j]);
            }
        }
    };

    if (nk > 0) {
        uint4 kA[U], vA[U], kB[U], vB[U];
        load_tile(0, kA, vA);
        for (int k = 0; k < nk; k += 2) {
            // the next tile's loads are in flight while this one is consumed; past the
            // wave's last tile they repeat that tile (already in the caches)
            load_tile(min(k + 1, nk - 1), kB, vB);
            compute_tile(k, kA, vA);
            if (k + 1 >= nk) break;
            load_tile(min(k + 2, nk - 1), kA, vA);
            compute_tile(k + 1, kB, vB);
        }
    }

    // Combine the NR row streams of the wave (lanes with the same c).
#pragma unroll
    for (int off = LR; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            const float m2 = __shfl_xor(m[h], off);
            const float l2 = __shfl_xor(l[h], off);
            const float M = fmaxf(m[h], m2);
            const float Ms = (M == -INFINITY) ? 0.f : M;
            const float a1 = fast_exp2(m[h] - Ms);
            const float a2 = fast_exp2(m2 - Ms);
            l[h] = l[h] * a1 + l2 * a2;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[h][j] = acc[h][j] * a1 + __shfl_xor(acc[h][j], off) * a2;
            m[h] = M;
        }
    }
    if (lane < LR) {
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            s_acc[wave][h][2 * c] = float4_t{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
            s_acc[wave][h][2 * c + 1] = float4_t{acc[h][4], acc[h][5], acc[h][6], acc[h][7]};
            if (lane == 0) {
                s_m[wave][h] = m[h];
                s_l[wave][h] = l[h];
            }
        }
    }
    __syncthreads();

    // Combine the NW wave states; the partition holds at least one token (wave 0's first
    // tile starts at t_begin < ctx), so M is finite and waves without tokens weigh 0.
    for (int idx = tid; idx < HP * C4; idx += NW * 64) {
        const int h = idx / C4;
        const int d4 = idx - h * C4;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.f;
        float4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float e = fast_exp2(s_m[w][h] - M);
            L += e * s_l[w][h];
            o += e * s_acc[w][h][d4];
        }
        const size_t row = row0 + h;
        if (direct) {
            reinterpret_cast<float4_t*>(a.out + row * D)[d4] = o / L;
        } else {
            const size_t slot = row * a.n_part_max + part;
            reinterpret_cast<float4_t*>(a.ws_acc + slot * D)[d4] = o;
            if (d4 == 0) {
                a.ws_ml[slot * 2] = M;
                a.ws_ml[slot * 2 + 1] = L;
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

// One workgroup per (sequence, query head).
template <int D>
__global__ void __launch_bounds__(kMergeThreads)
pa_merge_kernel(MergeArgs a) {
    constexpr int C4 = D / 4;                       // float4 columns
    constexpr int GR = kMergeThreads / C4;          // partition groups
    constexpr int UNR = 8;
    __shared__ float s_red[kMergeThreads / 64];
    __shared__ float4_t s_o[GR][C4];
    __shared__ float s_L[GR];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / a.query_heads;
    const int ctx = a.ctx[b];
    const int n = (ctx + a.partition - 1) / a.partition;
    if (n == 0 || (n == 1 && !a.force_split)) return;   // written by the decode kernel

    const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + (size_t)bh * a.n_part_max;
    const float4_t* acc = reinterpret_cast<const float4_t*>(a.ws_acc) + (size_t)bh * a.n_part_max * C4;

    // M = max over partitions
    float M = -INFINITY;
    for (int p = tid; p < n; p += kMergeThreads) M = fmaxf(M, ml[p].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if ((tid & 63) == 0) s_red[tid >> 6] = M;
    __syncthreads();
    M = s_red[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, s_red[w]);

    const int col = tid % C4;
    const int grp = tid / C4;
    float L = 0.f;
    float4_t o = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = grp; p0 < n; p0 += GR * UNR) {
        float4_t av[UNR];
        float2 mv[UNR];
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const int p = p0 + k * GR;
            if (p < n) {
                av[k] = acc[(size_t)p * C4 + col];
                mv[k] = ml[p];
            } else {
                av[k] = float4_t{0.f, 0.f, 0.f, 0.f};
                mv[k] = make_float2(-INFINITY, 0.f);
            }
        }
#pragma unroll
        for (int k = 0; k < UNR; ++k) {
            const float e = fast_exp2(mv[k].x - M);
            L += e * mv[k].y;
            o += e * av[k];
        }
    }
    s_o[grp][col] = o;
    if (col == 0) s_L[grp] = L;
    __syncthreads();
    if (tid < C4) {
        float4_t O = s_o[0][tid];
        float Ls = s_L[0];
#pragma unroll
        for (int g = 1; g < GR; ++g) {
            O += s_o[g][tid];
            Ls += s_L[g];
        }
        reinterpret_cast<float4_t*>(a.out + (size_t)bh * D)[tid] = O / Ls;
    }
}

constexpr int kWaves = 4;
constexpr int kLoads = 4;

template <int D, int HP>
hipError_t launch_decode(const Plan& pl, const DecodeArgs& args, hipStream_t stream) {
    hipLaunchKernelGGL((pa_decode_kernel<D, HP, kLoads, kWaves>), dim3((unsigned)pl.decode_grid),
                       dim3(kWaves * 64), 0, stream, args);
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
    if (pl.need_merge) {
        ws_acc = static_cast<float*>(workspace);
        ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ws_ml_offset);
    }
    DecodeArgs da;
    da.q = static_cast<const _Float16*>(q);
    da.k = static_cast<const _Float16*>(k);
    da.v = static_cast<const _Float16*>(v);
    da.bt = block_tables;
    da.ctx = ctx;
    da.out = out;
    da.ws_acc = ws_acc;
    da.ws_ml = ws_ml;
    da.scale_log2 = scale * kLog2e;
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
    if (err != hipSuccess || !pl.need_merge) return err;

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
