// Device helpers shared by the draft-tree kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define DDT_WAVE 64
#define DDT_LOG2E 1.4426950408889634f
#define DDT_LOG2E_D 1.4426950408889634074

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Monotone map float -> uint32 (larger float, larger code); -0 folds onto +0
// so that equal floats get equal codes.
__device__ __forceinline__ uint32_t ord_f32(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __uint_as_float(u);
}

// Candidate key: larger = better under (value desc, id asc).  Key 0 = none;
// its id decodes to -1.
__device__ __forceinline__ uint64_t vkey(float x, int id) {
    return ((uint64_t)ord_f32(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int vkey_id(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }
__device__ __forceinline__ float vkey_val(uint64_t k) { return unord_f32((uint32_t)(k >> 32)); }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = __shfl_xor(v, m);
        v = o > v ? o : v;
    }
    return v;
}
__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Rank counts split over lanes: n items, nt threads; item c is counted by the
// S aligned lanes c*S .. c*S + S - 1, each over a slice of the items.  S is
// the largest power of two <= 16 with S * n <= nt (1 when n > nt / 2).
__device__ __forceinline__ int split_lanes(int n, int nt) {
    int S = 1;
    while (S < 16 && 2 * S * n <= nt) S <<= 1;
    return S;
}
// Sum of v over each aligned group of S lanes (S = 1, 2, 4, 8 or 16), by DPP
// inside rows of 16: swap neighbours, swap pairs, mirror halves, mirror the
// row.  Every lane of the wave must take part.
__device__ __forceinline__ int group_sum(int v, int S) {
    if (S >= 2) v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
    if (S >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
    if (S >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
    if (S >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
    return v;
}
// v from lane l (l wave-uniform), through scalar registers.
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// exp(d) for d <= 0 via the hardware exp2.
__device__ __forceinline__ float exp_neg(float d) { return exp2f(d * DDT_LOG2E); }

// Sort key of a tree node: ascending (~ord(S), key) = (S desc, key asc).
struct NodeKey {
    uint32_t s;   // ~ord(S)
    uint64_t k;   // canonical key
};
__device__ __forceinline__ bool nk_greater(uint32_t sa, uint64_t ka, uint32_t sb, uint64_t kb) {
    return sa > sb || (sa == sb && ka > kb);
}

// In-LDS bitonic sort, ascending by (sa, sb), carrying si.  n2 is a power of
// two; every thread of the block must call it.
template <int NT>
__device__ void bitonic_sort_lds(uint32_t* sa, uint64_t* sb, int32_t* si, int n2) {
    for (int k = 2; k <= n2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int t = threadIdx.x; t < (n2 >> 1); t += NT) {
                const int i = ((t / j) * (j << 1)) + (t % j);
                const int l = i + j;
                const bool up = (i & k) == 0;
                const bool gt = nk_greater(sa[i], sb[i], sa[l], sb[l]);
                if (gt == up) {
                    uint32_t a = sa[i]; sa[i] = sa[l]; sa[l] = a;
                    uint64_t c = sb[i]; sb[i] = sb[l]; sb[l] = c;
                    int32_t d = si[i]; si[i] = si[l]; si[l] = d;
                }
            }
            __syncthreads();
        }
    }
}

__host__ __device__ __forceinline__ int next_pow2(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// Canonical key layout (see ddt.h).
#define KEY_DEPTH_SHIFT 59
#define KEY_SRC_SHIFT 58
#define KEY_RANK_BITS 5

__device__ __forceinline__ uint64_t key_child(uint64_t pkey, int pdepth, int rank, int src) {
    const int d = pdepth + 1;
    uint64_t path = pkey & ((1ull << KEY_SRC_SHIFT) - 1ull);
    path |= (uint64_t)rank << (KEY_SRC_SHIFT - KEY_RANK_BITS * d);
    const uint64_t srcbit = ((uint64_t)src << KEY_SRC_SHIFT) | (pkey & (1ull << KEY_SRC_SHIFT));
    return ((uint64_t)d << KEY_DEPTH_SHIFT) | srcbit | path;
}
