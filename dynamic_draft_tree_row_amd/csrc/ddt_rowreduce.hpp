// Vocabulary-wide row reduction: max, sigma' and top-K of logit rows.
//
// One workgroup reduces TPW consecutive fixed-size chunks ("tiles") of one row,
// streaming them from HBM once with 16-byte non-temporal loads; the next
// tile's loads are issued before the current one is processed.  Each thread
// keeps four independent online-softmax chains (running max, first index of
// the max, and sigma' = sum of exp(x - max) over the chain with the max element
// itself left out), so a tile costs one exp per element and no cross-lane
// traffic.  Top-K candidates are filtered against a threshold: the K-th largest
// per-lane maximum of the first tile, which cannot exceed the workgroup's K-th
// largest element; survivors go to an LDS list and the workgroup's top-K is
// picked from it by rank counting.  The workgroup writes one partial (max,
// sigma', top-K keys); consumers merge the partials of a row.
//
// The statistics give the log confidence log c = (l - max) - log1p(sigma') of
// a draft token, the confidence being the draft softmax probability (EAGLE-2
// explainer, section on confidence as an acceptance proxy; the Graft review's
// step 1 keeps it as a summed log-prob).
#pragma once
#include "ddt_device.hpp"

#define RR_NT 256           // threads per workgroup
#define RR_NV 4             // 16-byte loads per thread per tile
#define RR_CAP 1024         // LDS candidate list

template <bool BF16> struct RRShape {
    static constexpr int VEC = BF16 ? 8 : 4;          // elements per 16-byte load
    static constexpr int EPT = VEC * RR_NV;           // elements per thread per tile
    static constexpr int CH = RR_NT * EPT;            // elements per tile (chunk)
};

// Rows (i0, i1) with i0 < n0 (grid-derived) and i1 < n1; row base at
// base + i0*s0 + i1*s1 elements.  Rows with i1 >= count[i0] + count_add are
// skipped when count is given.
struct RowSrc {
    const void* base;
    int64_t s0, s1;
    int n1;
    const int32_t* count;
    int count_add;
};

// Partial layout per (row, group): PS = 2 + 2K words: [0] max, [1] sigma',
// [2 + 2k .. 3 + 2k] candidate key k (uint64, descending, key 0 = none).
__host__ __device__ __forceinline__ int rr_ps(int K) { return 2 + 2 * K; }

// ---------------------------------------------------------------------------
// DPP wave reductions (all 64 lanes active); result is wave-uniform
// ---------------------------------------------------------------------------
template <class Op>
__device__ __forceinline__ uint32_t dpp_reduce_u32(uint32_t v, uint32_t ident, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0xB1, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x4E, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x141, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x140, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x142, 0xA, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return dpp_reduce_u32(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return dpp_reduce_u32(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ float wave_sumf(float v) {
    return __uint_as_float(dpp_reduce_u32(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}
// largest 64-bit key in the wave: max high word, then max low word among ties
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    const uint32_t hi = wave_max_u32((uint32_t)(k >> 32));
    const uint32_t lo = wave_max_u32((uint32_t)(k >> 32) == hi ? (uint32_t)k : 0u);
    return ((uint64_t)hi << 32) | lo;
}

template <bool BF16, int NL>
__device__ __forceinline__ void rr_load(u32x4 (&raw)[NL], const void* row, bool al, int start,
                                        int V, int tid) {
    using SH = RRShape<BF16>;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e0 = start + (i * RR_NT + tid) * SH::VEC;
        if (al && e0 + SH::VEC <= V) {
            raw[i] = __builtin_nontemporal_load(
                (const u32x4*)((const char*)row + (size_t)e0 * (BF16 ? 2 : 4)));
        } else {
            // ragged tail or unaligned row: element-wise, -inf past V
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (BF16) {
                    const int a = e0 + 2 * q, b = a + 1;
                    const uint32_t lo = a < V ? (uint32_t)((const uint16_t*)row)[a] : 0xFF80u;
                    const uint32_t hi = b < V ? (uint32_t)((const uint16_t*)row)[b] : 0xFF80u;
                    w[q] = lo | (hi << 16);
                } else {
                    const int a = e0 + q;
                    w[q] = a < V ? ((const uint32_t*)row)[a] : 0xFF800000u;
                }
            }
            raw[i] = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
}

// element e of 16-byte word vector r
#define RR_X(r, e) (BF16 ? __uint_as_float(((e) & 1) ? ((r)[(e) >> 1] & 0xFFFF0000u) : ((r)[(e) >> 1] << 16)) \
                         : __uint_as_float((r)[(e)]))

// One workgroup: TPW consecutive chunks of one row, all loads issued up front
// and held in registers.  Pass 1 takes the thread maximum; one barrier gives
// the workgroup maximum M and the candidate threshold; pass 2 sums
// exp(x - M).  The single element that sigma' leaves out (the first occurrence
// of M) is removed exactly by the thread that holds it, in a branch only such
// threads take.
template <bool BF16, int TPW>
__global__ __launch_bounds__(RR_NT) void k_row_partial(RowSrc rs, int V, int groups, int K,
                                                       uint32_t* __restrict__ part) {
    using SH = RRShape<BF16>;
    constexpr int VEC = SH::VEC, CH = SH::CH, NW = RR_NT / DDT_WAVE, NL = RR_NV * TPW;
    __shared__ uint32_t s_wmax[NW], s_wtau[NW], s_wtie[NW];
    __shared__ float s_wsum[NW];
    __shared__ int s_cnt, s_ties;
    __shared__ uint64_t s_list[RR_CAP];

    const int g = blockIdx.x % groups;
    const int rowg = blockIdx.x / groups;
    const int i0 = rowg / rs.n1, i1 = rowg - i0 * rs.n1;
    if (rs.count != nullptr && i1 >= rs.count[i0] + rs.count_add) return;   // block-uniform
    const int tid = threadIdx.x, lane = tid & (DDT_WAVE - 1), wid = tid / DDT_WAVE;
    const int64_t off = (int64_t)i0 * rs.s0 + (int64_t)i1 * rs.s1;
    const void* row = (const char*)rs.base + off * (BF16 ? 2 : 4);
    const bool al = (((uintptr_t)row) & 15u) == 0;
    uint32_t* out = part + ((size_t)rowg * groups + g) * rr_ps(K);
    const int start = g * TPW * CH;
    // load i covers ids start + (i*NT + tid)*VEC .. +VEC  (tile i / RR_NV)
#define RR_ID(i, e) (start + ((i) * RR_NT + tid) * VEC + (e))

    u32x4 raw[NL];
    rr_load<BF16, NL>(raw, row, al, start, V, tid);
    if (tid == 0) { s_cnt = 0; s_ties = 0; }

    // pass 1: thread maximum (padding is -inf)
    float tm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
#pragma unroll
        for (int e = 0; e < VEC; e += 2) tm = fmaxf(tm, fmaxf(RR_X(raw[i], e), RR_X(raw[i], e + 1)));
    }
    // wave maximum and the candidate threshold: the K-th largest lane maximum
    // (exact, bit by bit; bf16 codes differ only in their top 16 bits) bounds
    // the workgroup's K-th largest element from below
    const uint32_t lo = tm > -INFINITY ? ord_f32(tm) : 0u;
    const uint32_t wmax = wave_max_u32(lo);
    uint32_t tau = 0u;
    for (int bit = 31; bit >= (BF16 ? 16 : 0); --bit) {
        const uint32_t cand = tau | (1u << bit);
        if (__popcll(__ballot(lo >= cand)) >= (unsigned)K) tau = cand;
    }
    if (lane == 0) { s_wmax[wid] = wmax; s_wtau[wid] = tau; }
    __syncthreads();
    uint32_t bmax = s_wmax[0], bt = s_wtau[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        bmax = s_wmax[w] > bmax ? s_wmax[w] : bmax;
        bt = s_wtau[w] > bt ? s_wtau[w] : bt;
    }
    if (bmax == 0u) {                                          // chunk range holds no element
        if (tid < 2 + 2 * K) out[tid] = tid == 0 ? __float_as_uint(-INFINITY) : 0u;
        return;
    }
    const float M = unord_f32(bmax);
    const float tauf = bt ? unord_f32(bt) : -INFINITY;
    const float ML = M * DDT_LOG2E;

    // pass 2: sum of exp(x - M) over every element
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
#pragma unroll
        for (int e = 0; e < VEC; e += 2) {
            s0 += exp2f(fmaf(RR_X(raw[i], e), DDT_LOG2E, -ML));
            s1 += exp2f(fmaf(RR_X(raw[i], e + 1), DDT_LOG2E, -ML));
        }
    }
    float s = s0 + s1;
    if (tm == M) {
        // this thread holds the maximum: redo its sum without those elements
        // (summing 1.0 into small terms would cost them precision) and count them
        s = 0.f;
        int c = 0;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float x = RR_X(raw[i], e);
                c += x == M;
                s += x == M ? 0.f : exp2f(fmaf(x, DDT_LOG2E, -ML));
            }
        }
        atomicAdd(&s_ties, c);
    }
    if (tm >= tauf) {
        // candidates at or above the threshold go to the LDS list
#pragma unroll
        for (int i = 0; i < NL; ++i) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float x = RR_X(raw[i], e);
                if (x >= tauf && RR_ID(i, e) < V) {
                    const int slot = atomicAdd(&s_cnt, 1);
                    if (slot < RR_CAP) s_list[slot] = vkey(x, RR_ID(i, e));
                }
            }
        }
    }
    s = wave_sumf(s);
    if (lane == 0) s_wsum[wid] = s;
    __syncthreads();
    const int cnt = s_cnt;
    uint64_t* okeys = (uint64_t*)(out + 2);
    if (cnt <= RR_CAP) {
        // rank counting: keys are unique, so rank < K places the key exactly
        for (int p = tid; p < cnt; p += RR_NT) {
            const uint64_t k = s_list[p];
            int rank = 0;
            for (int q = 0; q < cnt; ++q) rank += s_list[q] > k;
            if (rank < K) okeys[rank] = k;
        }
        for (int k = cnt + tid; k < K; k += RR_NT) okeys[k] = 0ull;
    } else {
        // list overflow (massive ties): exact K rounds over the registers
        uint64_t prev = ~0ull;
        for (int k = 0; k < K; ++k) {
            uint64_t best = 0ull;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    if (RR_ID(i, e) < V) {
                        const uint64_t v = vkey(RR_X(raw[i], e), RR_ID(i, e));
                        if (v < prev && v > best) best = v;
                    }
                }
            }
            best = wave_max_key(best);
            __syncthreads();
            if (lane == 0) s_list[wid] = best;
            __syncthreads();
            best = s_list[0];
#pragma unroll
            for (int w = 1; w < NW; ++w) best = s_list[w] > best ? s_list[w] : best;
            if (tid == 0) okeys[k] = best;
            prev = best;
        }
    }
    if (tid == 0) {
        float st = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) st += s_wsum[w];
        out[0] = __float_as_uint(M);
        out[1] = __float_as_uint(st + (float)(s_ties - 1));
    }
#undef RR_ID
}

// Merge the group partials of one row; all 64 lanes of a wave call it.
// Returns the row max M and sigma' (same value in every lane); lane k < K
// receives the row's k-th best key (0 if the row has fewer than k+1 elements).
__device__ __forceinline__ uint64_t merge_row_wave(const uint32_t* __restrict__ p, int groups, int K,
                                                   float& M, float& Sp) {
    constexpr int MR = 8;                              // keys held in registers per lane
    const int lane = threadIdx.x & (DDT_WAVE - 1);
    const int PS = rr_ps(K);
    float mc = -INFINITY, sc = 0.f;
    if (lane < groups) {
        mc = __uint_as_float(p[lane * PS]);
        sc = __uint_as_float(p[lane * PS + 1]);
    }
    M = unord_f32(wave_max_u32(lane < groups ? ord_f32(mc) : 0u));
    const int cstar = (int)wave_min_u32((lane < groups && mc == M) ? (uint32_t)lane : 0xFFFFFFFFu);
    float contrib = 0.f;
    if (lane < groups && mc > -INFINITY) {
        const float e = exp2f((mc - M) * DDT_LOG2E);
        contrib = sc * e + (lane != cstar ? e : 0.f);
    }
    Sp = wave_sumf(contrib);
    const int total = groups * K;
    const bool fits = total <= MR * DDT_WAVE;
    uint64_t kk[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        const int q = lane + r * DDT_WAVE;
        kk[r] = 0ull;
        if (fits && q < total) {
            const int c = q / K, e = q - c * K;
            kk[r] = *(const uint64_t*)(p + c * PS + 2 + 2 * e);
        }
    }
    uint64_t prev = ~0ull, mine = 0ull;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0ull;
        if (fits) {
#pragma unroll
            for (int r = 0; r < MR; ++r)
                if (kk[r] < prev && kk[r] > best) best = kk[r];
        } else {
            for (int q = lane; q < total; q += DDT_WAVE) {
                const int c = q / K, e = q - c * K;
                const uint64_t v = *(const uint64_t*)(p + c * PS + 2 + 2 * e);
                if (v < prev && v > best) best = v;
            }
        }
        best = wave_max_key(best);
        if (lane == k) mine = best;
        prev = best;
    }
    return mine;
}
