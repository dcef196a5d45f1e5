// Vocabulary-wide row reduction: max, sigma' and top-K of logit rows.
//
// One workgroup reduces one fixed-size chunk of one row, streaming it from HBM
// once with 16-byte non-temporal loads held in registers, and writes a partial
// (chunk max, chunk sigma', chunk top-K keys).  Consumers merge the partials of
// a row with merge_row_wave.  The statistics feed the log confidence
// log c = (l - max) - log1p(sigma') of a draft token, the confidence being the
// draft softmax probability (EAGLE-2 explainer, section on confidence as an
// acceptance proxy; Graft review step 1 keeps it as a summed log-prob).
#pragma once
#include "ddt_device.hpp"

#define RR_NT 256           // threads per workgroup
#define RR_NV 4             // 16-byte loads per thread
#define RR_CAP 512          // LDS candidate list

template <bool BF16> struct RRShape {
    static constexpr int VEC = BF16 ? 8 : 4;          // elements per 16-byte load
    static constexpr int EPT = VEC * RR_NV;           // elements per thread
    static constexpr int CH = RR_NT * EPT;            // elements per chunk
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

// Partial layout per (row, chunk): PS = 2 + 2K words: [0] max, [1] sigma',
// [2 + 2k .. 3 + 2k] candidate key k (uint64, key 0 = none).
__host__ __device__ __forceinline__ int rr_ps(int K) { return 2 + 2 * K; }

template <bool BF16>
__global__ __launch_bounds__(RR_NT) void k_row_partial(RowSrc rs, int V, int chunks, int K,
                                                       uint32_t* __restrict__ part) {
    using SH = RRShape<BF16>;
    constexpr int VEC = SH::VEC, EPT = SH::EPT, CH = SH::CH;
    __shared__ uint64_t s_wkey[RR_NT / DDT_WAVE];
    __shared__ float s_wsum[RR_NT / DDT_WAVE];
    __shared__ uint32_t s_wtau[RR_NT / DDT_WAVE];
    __shared__ int s_cnt;
    __shared__ uint64_t s_list[RR_CAP];

    const int chunk = blockIdx.x % chunks;
    const int rowg = blockIdx.x / chunks;
    const int i0 = rowg / rs.n1, i1 = rowg - i0 * rs.n1;
    if (rs.count != nullptr && i1 >= rs.count[i0] + rs.count_add) return;   // block-uniform
    const int tid = threadIdx.x, lane = tid & (DDT_WAVE - 1), wid = tid / DDT_WAVE;
    const int64_t off = (int64_t)i0 * rs.s0 + (int64_t)i1 * rs.s1;
    const int start = chunk * CH;
    uint32_t* out = part + ((size_t)rowg * chunks + chunk) * rr_ps(K);

    // element j of this thread has id start + ((j / VEC) * NT + tid) * VEC + j % VEC
    float x[EPT];
    if constexpr (BF16) {
        const uint16_t* row = (const uint16_t*)rs.base + off;
        const bool al = (((uintptr_t)row) & 15u) == 0;
#pragma unroll
        for (int i = 0; i < RR_NV; ++i) {
            const int e0 = start + (i * RR_NT + tid) * VEC;
            if (al && e0 + VEC <= V) {
                const u32x4 v = __builtin_nontemporal_load((const u32x4*)(row + e0));
                x[i * 8 + 0] = __uint_as_float(v.x << 16);
                x[i * 8 + 1] = __uint_as_float(v.x & 0xFFFF0000u);
                x[i * 8 + 2] = __uint_as_float(v.y << 16);
                x[i * 8 + 3] = __uint_as_float(v.y & 0xFFFF0000u);
                x[i * 8 + 4] = __uint_as_float(v.z << 16);
                x[i * 8 + 5] = __uint_as_float(v.z & 0xFFFF0000u);
                x[i * 8 + 6] = __uint_as_float(v.w << 16);
                x[i * 8 + 7] = __uint_as_float(v.w & 0xFFFF0000u);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int id = e0 + e;
                    x[i * VEC + e] = id < V ? __uint_as_float((uint32_t)row[id] << 16) : -INFINITY;
                }
            }
        }
    } else {
        const float* row = (const float*)rs.base + off;
        const bool al = (((uintptr_t)row) & 15u) == 0;
#pragma unroll
        for (int i = 0; i < RR_NV; ++i) {
            const int e0 = start + (i * RR_NT + tid) * VEC;
            if (al && e0 + VEC <= V) {
                const u32x4 v = __builtin_nontemporal_load((const u32x4*)(row + e0));
                x[i * 4 + 0] = __uint_as_float(v.x);
                x[i * 4 + 1] = __uint_as_float(v.y);
                x[i * 4 + 2] = __uint_as_float(v.z);
                x[i * 4 + 3] = __uint_as_float(v.w);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int id = e0 + e;
                    x[i * VEC + e] = id < V ? row[id] : -INFINITY;
                }
            }
        }
    }
#define RR_ID(j) (start + (((j) / VEC) * RR_NT + tid) * VEC + ((j) % VEC))

    // thread max, first occurrence (ids grow with j)
    float tm = -INFINITY;
    int tj = -1;
#pragma unroll
    for (int j = 0; j < EPT; ++j)
        if (x[j] > tm) { tm = x[j]; tj = j; }
    const uint64_t tkey = tj >= 0 ? vkey(tm, RR_ID(tj)) : 0ull;

    // chunk max: largest key = (max value, lowest id)
    uint64_t wk = wave_max_u64(tkey);
    if (lane == 0) s_wkey[wid] = wk;
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    uint64_t bk = s_wkey[0];
#pragma unroll
    for (int w = 1; w < RR_NT / DDT_WAVE; ++w) bk = s_wkey[w] > bk ? s_wkey[w] : bk;
    if (bk == 0ull) {                                         // chunk holds no element
        if (tid < 2 + 2 * K) out[tid] = tid == 0 ? __float_as_uint(-INFINITY) : 0u;
        return;
    }
    const float M = vkey_val(bk);
    const int own = (tkey == bk) ? tj : -1;                   // exactly one thread owns the max

    // sigma' relative to the chunk max, the max element itself left out
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const float e = exp_neg(x[j] - M);
        s += (j == own) ? 0.f : e;
    }
    s = wave_sum_f32(s);

    // wave threshold: K-th largest lane maximum (by bits, exact); any K lane
    // maxima are K distinct elements, so the chunk's K-th largest is >= it
    const uint32_t lo = (uint32_t)(tkey >> 32);
    uint32_t tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tau | (1u << bit);
        if (__popcll(__ballot(lo >= cand)) >= (unsigned)K) tau = cand;
    }
    if (lane == 0) { s_wsum[wid] = s; s_wtau[wid] = tau; }
    __syncthreads();
    uint32_t btau = s_wtau[0];
#pragma unroll
    for (int w = 1; w < RR_NT / DDT_WAVE; ++w) btau = s_wtau[w] > btau ? s_wtau[w] : btau;
    const float tauf = btau ? unord_f32(btau) : -INFINITY;

    // candidates at or above the threshold go to LDS
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (x[j] >= tauf && (btau != 0u || RR_ID(j) < V)) {
            const int slot = atomicAdd(&s_cnt, 1);
            if (slot < RR_CAP) s_list[slot] = vkey(x[j], RR_ID(j));
        }
    }
    __syncthreads();
    const int cnt = s_cnt;
    uint64_t* okeys = (uint64_t*)(out + 2);
    if (cnt <= DDT_WAVE) {
        if (wid == 0) {
            // one wave sorts up to 64 candidate keys descending (bitonic over lanes)
            uint64_t k = lane < cnt ? s_list[lane] : 0ull;
#pragma unroll
            for (int size = 2; size <= DDT_WAVE; size <<= 1) {
#pragma unroll
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    const uint64_t o = __shfl_xor(k, stride);
                    const uint64_t hi = o > k ? o : k, lw = o > k ? k : o;
                    const bool lower = (lane & stride) == 0;
                    const bool up = (lane & size) == 0;
                    k = (lower == up) ? hi : lw;
                }
            }
            if (lane < K) okeys[lane] = k;
        }
    } else if (cnt <= RR_CAP) {
        if (wid == 0) {
            uint64_t prev = ~0ull;
            for (int k = 0; k < K; ++k) {
                uint64_t best = 0ull;
                for (int p = lane; p < cnt; p += DDT_WAVE) {
                    const uint64_t v = s_list[p];
                    if (v < prev && v > best) best = v;
                }
                best = wave_max_u64(best);
                if (lane == 0) okeys[k] = best;
                prev = best;
            }
        }
    } else {
        // list overflow (massive ties): exact K rounds over the registers
        uint64_t prev = ~0ull;
        for (int k = 0; k < K; ++k) {
            uint64_t best = 0ull;
#pragma unroll
            for (int j = 0; j < EPT; ++j) {
                if (RR_ID(j) < V) {
                    const uint64_t v = vkey(x[j], RR_ID(j));
                    if (v < prev && v > best) best = v;
                }
            }
            best = wave_max_u64(best);
            __syncthreads();
            if (lane == 0) s_wkey[wid] = best;
            __syncthreads();
            best = s_wkey[0];
#pragma unroll
            for (int w = 1; w < RR_NT / DDT_WAVE; ++w) best = s_wkey[w] > best ? s_wkey[w] : best;
            if (tid == 0) okeys[k] = best;
            prev = best;
        }
    }
    if (tid == 0) {
        float st = 0.f;
#pragma unroll
        for (int w = 0; w < RR_NT / DDT_WAVE; ++w) st += s_wsum[w];
        out[0] = __float_as_uint(M);
        out[1] = __float_as_uint(st);
    }
#undef RR_ID
}

// Merge the chunk partials of one row; all 64 lanes of a wave call it.
// Returns the row max M and sigma' (same value in every lane); lane k < K
// receives the row's k-th best key (0 if the row has fewer than k+1 elements).
__device__ __forceinline__ uint64_t merge_row_wave(const uint32_t* __restrict__ p, int chunks, int K,
                                                   float& M, float& Sp) {
    const int lane = threadIdx.x & (DDT_WAVE - 1);
    const int PS = rr_ps(K);
    float mc = -INFINITY, sc = 0.f;
    if (lane < chunks) {
        mc = __uint_as_float(p[lane * PS]);
        sc = __uint_as_float(p[lane * PS + 1]);
    }
    M = wave_max_f32(mc);
    const int cstar = wave_min_i32((lane < chunks && mc == M) ? lane : DDT_WAVE);
    float contrib = 0.f;
    if (lane < chunks && mc > -INFINITY) {
        const float e = exp_neg(mc - M);
        contrib = sc * e + (lane != cstar ? e : 0.f);
    }
    Sp = wave_sum_f32(contrib);
    const int total = chunks * K;
    uint64_t prev = ~0ull, mine = 0ull;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0ull;
        for (int q = lane; q < total; q += DDT_WAVE) {
            const int c = q / K, e = q - c * K;
            const uint64_t v = *(const uint64_t*)(p + c * PS + 2 + 2 * e);
            if (v < prev && v > best) best = v;
        }
        best = wave_max_u64(best);
        if (lane == k) mine = best;
        prev = best;
    }
    return mine;
}
