// Vocabulary-wide row reduction: max, sigma' and top-K of logit rows.
//
// One workgroup of 256 threads reduces one fixed-size chunk of one row (8192
// bf16 or 4096 fp32 logits): every thread issues its four 16-byte
// non-temporal loads up front and keeps them in registers.  Pass 1 takes the
// thread maximum; a bit-by-bit ballot search gives each wave the K-th largest
// lane maximum, and the largest of those over the waves is a lower bound for
// the chunk's K-th largest element (the candidate threshold).  Pass 2 sums
// exp(x - M) over the elements below the chunk maximum M (only the wave that
// holds M tests for it).  The few lanes whose maximum reaches the threshold
// stage their words in LDS, the wave tests those elements one per lane, and
// the chunk's top K is placed by rank counting over the resulting list.  The
// workgroup writes one partial (max, sigma', top-K keys); consumers merge the
// partials of a row (merge_row_wave).
//
// The statistics give the log confidence log c = (l - max) - log1p(sigma') of
// a draft token, the confidence being the draft softmax probability (EAGLE-2
// explainer, section on confidence as an acceptance proxy; the Graft review's
// step 1 keeps it as a summed log-prob).
#pragma once
#include "ddt_device.hpp"

#define RR_NT 256           // threads per workgroup
#define RR_NV 4             // 16-byte loads per thread per chunk (small launches)
#define RR_NV_WIDE 8        // the same for launches of RR_WIDE_ROWS rows or more
#define RR_WIDE_ROWS 256
#define RR_WIDE_FLAT_ROWS 512
#define RR_CAP 1024         // LDS candidate list
#define RR_SW 64            // words per wave staged at a time

// Chunk shape for NL 16-byte loads per thread.  Wide chunks (8 loads, 64 bf16
// per thread) halve the per-wave fixed work per element, which is what bounds
// a launch that fills the chip; small launches keep 4 loads, so that each
// workgroup's latency stays short.
template <bool BF16, int NL = RR_NV> struct RRShape {
    static constexpr int VEC = BF16 ? 8 : 4;          // elements per 16-byte load
    static constexpr int EPT = VEC * NL;              // elements per thread per chunk
    static constexpr int CH = RR_NT * EPT;            // elements per chunk
};

// Rows (i0, i1) with i0 < n0 (grid-derived) and i1 < n1; row base at
// base + i0*s0 + i1*s1 elements.  Rows with i1 >= count[i0] + count_add are
// skipped when count is given.  When sum_if is given, rows with
// !(sum_if[i0] > 0) need only the max and the top K: sigma' is not summed and
// reads 0 (greedy verify rows, whose temperature is 0, use only the argmax).
struct RowSrc {
    const void* base;
    int64_t s0, s1;
    int n1;
    const int32_t* count;
    int count_add;
    const float* sum_if;
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

// Inclusive prefix sum of v over the 64 lanes (DPP: shifts by 1, 2, 4, 8
// inside each row of 16, then the totals of earlier rows by broadcast).
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, true);
    return v;
}

// Padding of a ragged bf16 chunk.  Wide chunks pad with -2^121, the smallest
// bf16 value that pass 1's packed fp16 reading orders (it reads as fp16
// -inf), so that their ragged chunks (one in eight of a row's chunks) stay on
// the packed path; -inf padding reads as NaN and would send every wave of the
// chunk to the fp32 reading.  A lane maximum equal to -2^121 is ambiguous and
// takes the fp32 reading, which first restores -inf past V; on the packed path
// the padding lies below the maximum, adds exp(-2^121 - M) = 0 to sigma' and
// never reaches the (finite) threshold.  Short chunks keep -inf: there the
// ragged chunk is one in sixteen and the extra code costs more than it saves.
template <bool BF16, int NL> struct RRPad {
    static constexpr bool low = BF16 && NL >= RR_NV_WIDE;
    static constexpr uint32_t pad16 = low ? 0xFC00u : 0xFF80u;
};

template <bool BF16, int NL>
__device__ __forceinline__ void rr_load(u32x4 (&raw)[NL], const void* row, bool al, int start,
                                        int V, int tid) {
    using SH = RRShape<BF16, NL>;
    constexpr uint32_t pad16 = RRPad<BF16, NL>::pad16;
    if (al && start + SH::CH <= V) {
        // the whole chunk lies inside the row (every chunk but a ragged
        // last one): a uniform base plus a 32-bit per-lane offset, one add
        // per load instead of a range test and a 64-bit address each
        const char* base = (const char*)row + (size_t)start * (BF16 ? 2 : 4);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            // (opaque to the compiler, so that the address stays a scalar
            // base plus a 32-bit vector offset rather than a 64-bit sum)
            uint32_t off = (uint32_t)((i * RR_NT + tid) * 16);
            asm volatile("" : "+v"(off));
            raw[i] = __builtin_nontemporal_load((const u32x4*)(base + off));
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int e0 = start + (i * RR_NT + tid) * SH::VEC;
        if (al && e0 + SH::VEC <= V) {
            raw[i] = __builtin_nontemporal_load(
                (const u32x4*)((const char*)row + (size_t)e0 * (BF16 ? 2 : 4)));
        } else {
            // ragged tail or unaligned row: element-wise, padding past V
            uint32_t w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if constexpr (BF16) {
                    const int a = e0 + 2 * q, b = a + 1;
                    const uint32_t lo = a < V ? (uint32_t)((const uint16_t*)row)[a] : pad16;
                    const uint32_t hi = b < V ? (uint32_t)((const uint16_t*)row)[b] : pad16;
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

// Make one wave's LDS writes visible to its own later LDS reads (no
// workgroup barrier: the wave only talks to itself).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// max of three floats in one instruction (the operands are plain values
// decoded from bf16/fp32 bits; no NaN canonicalisation is wanted)
__device__ __forceinline__ float rr_max3(float a, float b, float c) {
    float r;
    asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Packed maximum of bf16 bit patterns read as fp16.  The reading is monotone
// (sign, then exponent and mantissa bits in order) for every pattern whose
// fp16 exponent field is not all ones, i.e. every bf16 value of magnitude
// below 2^121 and the value 2^121 itself (read as fp16 infinity); larger
// magnitudes, bf16 infinities and NaNs read as fp16 NaN, which the IEEE
// maximum3 propagates, so a NaN result flags the one case that needs the
// fp32 reading.  fp16 denormals are preserved (the kernels' default mode), so
// tiny values compare exactly.
//   rr_pkmax3:   lo = max(a.lo, b.lo, c.lo), hi = max(a.hi, b.hi, c.hi)
//   rr_pkmax3_x: lo = max(a.lo, b.hi, c.hi), hi = max(a.hi, b.lo, c.lo)
// (each one v_pk_maximum3_f16, the swap folded into its operand selects)
typedef _Float16 rr_h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t rr_pkmax3(uint32_t a, uint32_t b, uint32_t c) {
    const rr_h2 x = __builtin_bit_cast(rr_h2, a), y = __builtin_bit_cast(rr_h2, b),
                z = __builtin_bit_cast(rr_h2, c);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z));
}
__device__ __forceinline__ uint32_t rr_pkmax3_x(uint32_t a, uint32_t b, uint32_t c) {
    const rr_h2 x = __builtin_bit_cast(rr_h2, a), y = __builtin_bit_cast(rr_h2, b),
                z = __builtin_bit_cast(rr_h2, c);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(x, __builtin_shufflevector(y, y, 1, 0)), __builtin_shufflevector(z, z, 1, 0)));
}
__device__ __forceinline__ bool rr_nan16(uint32_t t) {
    return __builtin_isnan(__builtin_bit_cast(_Float16, (uint16_t)t));
}

// element e of 16-byte word vector r
#define RR_X(r, e) (BF16 ? __uint_as_float(((e) & 1) ? ((r)[(e) >> 1] & 0xFFFF0000u) : ((r)[(e) >> 1] << 16)) \
                         : __uint_as_float((r)[(e)]))

// The partial record's stores are device-coherent (agent-scope atomic
// stores write through to the level every compute unit reads), so a
// workgroup of the same kernel can read them once the writer's stores have
// completed, with no cache write-back.
__device__ __forceinline__ void rr_st32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void rr_st64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads of values another workgroup of the same kernel stored that way
// (COH) read the coherent level too; plain loads otherwise.
template <bool COH> __device__ __forceinline__ uint32_t rr_ld32(const uint32_t* p) {
    if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}
template <bool COH> __device__ __forceinline__ uint64_t rr_ld64(const uint64_t* p) {
    if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}

// LDS of one chunk reduction (one workgroup of RR_NT threads).
struct RRLds {
    uint32_t wmax[RR_NT / DDT_WAVE], wtau[RR_NT / DDT_WAVE];
    float wsum[RR_NT / DDT_WAVE];
    int cnt, ties, amin;
    uint64_t list[RR_CAP];
    u32x4 stage[(RR_NT / DDT_WAVE) * RR_SW];
    int sid[(RR_NT / DDT_WAVE) * RR_SW];
};

typedef unsigned long long rr_u64x2 __attribute__((ext_vector_type(2)));

// Ranks of the first cnt keys of the candidate list (unique, nonzero; the
// list is zero past them up to RR_NT entries) by counting the larger keys:
// candidate c = tid / S is counted by the S adjacent lanes c*S .. c*S + S - 1,
// lane part over the contiguous slice [part * NC/S, (part + 1) * NC/S) of the
// first NC = RR_NT / S entries, read 16 bytes at a time (the slice address
// depends on the lane's part only, so a wave's reads are broadcasts).  cnt
// <= NC.  Rank < K puts the key at out[rank].
template <int S>
__device__ __forceinline__ void rr_rank_fixed(const uint64_t* s_list, int cnt, int K,
                                              uint64_t* __restrict__ out) {
    constexpr int NC = RR_NT / S, SLICE = NC / S;
    const int tid = threadIdx.x, c = tid / S, part = tid % S;
    const uint64_t k = s_list[c];
    const rr_u64x2* sl = (const rr_u64x2*)(s_list + part * SLICE);
    int r = 0;
#pragma unroll 8
    for (int j = 0; j < SLICE / 2; ++j) {
        const rr_u64x2 w = sl[j];
        r += (w.x > k ? 1 : 0) + (w.y > k ? 1 : 0);
    }
    r = group_sum(r, S);
    if (part == 0 && c < cnt && r < K) rr_st64(out + r, k);
}

// One workgroup reduces chunk g of one row (base `row`, V elements) and
// writes its partial record to `out`.  Every thread of the workgroup calls
// it and every thread returns (no early exit), so a caller can go on after
// it.
template <bool BF16, int NL>
__device__ __forceinline__ void rr_chunk(const void* row, int V, int g, int K, bool sums,
                                         uint32_t* __restrict__ out, RRLds& L) {
    using SH = RRShape<BF16, NL>;
    constexpr int VEC = SH::VEC, CH = SH::CH, NW = RR_NT / DDT_WAVE;
    uint32_t* s_wmax = L.wmax;
    uint32_t* s_wtau = L.wtau;
    float* s_wsum = L.wsum;
    int& s_cnt = L.cnt;
    int& s_ties = L.ties;
    int& s_amin = L.amin;
    uint64_t* s_list = L.list;
    u32x4* s_stage = L.stage;
    int* s_sid = L.sid;
    const int tid = threadIdx.x, lane = tid & (DDT_WAVE - 1), wid = tid / DDT_WAVE;
    const bool al = (((uintptr_t)row) & 15u) == 0;
    const int start = g * CH;
    // load i covers ids start + (i*NT + tid)*VEC .. +VEC
#define RR_ID(i, e) (start + ((i) * RR_NT + tid) * VEC + (e))

    u32x4 raw[NL];
    rr_load<BF16, NL>(raw, row, al, start, V, tid);
    if (tid == 0) { s_cnt = 0; s_ties = 0; s_amin = 0x7FFFFFFF; }
    // the candidate list's first RR_NT entries start at 0 (key 0 is no
    // element and never outranks one), so that the ranking can read a
    // zero-padded list with fixed trip counts
    if (K > 1) s_list[tid] = 0ull;

    // pass 1: the thread maximum (padding is -inf, or -2^121: RRPad).  bf16
    // words take the packed fp16 maximum, two 32-bit registers per
    // instruction; a wave in which some lane's result is NaN (a value of
    // magnitude above 2^121, an infinity or a NaN) takes the fp32 reading
    // instead.
    bool pk = false;                                           // wave-uniform
    float tm = -INFINITY;
    float wm[NL];                                              // word maxima (when needed)
    // word i's maximum in both halves: three packed maxima
    auto pk_word = [&](int i) -> uint32_t {
        const uint32_t m = rr_pkmax3(raw[i][0], raw[i][1], raw[i][2]);
        const uint32_t h = rr_pkmax3_x(m, m, raw[i][3]);      // lo: all but d3.lo; hi: all but d3.hi
        return rr_pkmax3_x(h, h, h);
    };
    static_assert(!BF16 || NL % 2 == 0, "the packed pass pairs the words");
    if constexpr (BF16) {
        // independent packed maxima, three operands each, level by level
        // (a dependent chain would wait on every result)
        uint32_t a[NL];
        if (K > 1) {
            // every word's maximum (the staging needs them), then the thread's
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                a[i] = pk_word(i);
                wm[i] = __uint_as_float(a[i] << 16);
            }
        } else {
            // each word reduced to a packed pair, the fourth registers of odd
            // words folded into their even neighbours
#pragma unroll
            for (int i = 0; i < NL; ++i) a[i] = rr_pkmax3(raw[i][0], raw[i][1], raw[i][2]);
#pragma unroll
            for (int i = 0; i + 1 < NL; i += 2) {
                a[i] = rr_pkmax3(a[i], raw[i][3], raw[i + 1][3]);
            }
        }
        int n = NL;
#pragma unroll
        for (int lvl = 0; lvl < 4; ++lvl) {
            if (n > 1) {
                int m = 0;
#pragma unroll
                for (int j = 0; j < NL; j += 3) {
                    if (j < n) {
                        const uint32_t b = a[j], c = j + 1 < n ? a[j + 1] : b, d = j + 2 < n ? a[j + 2] : c;
                        a[m++] = rr_pkmax3(b, c, d);
                    }
                }
                n = m;
            }
        }
        const uint32_t t = K > 1 ? a[0] : rr_pkmax3_x(a[0], a[0], a[0]);
        pk = __ballot(rr_nan16(t) | (RRPad<BF16, NL>::low && (t & 0xFFFFu) == 0xFC00u)) == 0ull;
        tm = __uint_as_float(t << 16);
    }
    if (!pk) {
        // the fp32 reading: every word's maximum, then the thread's (a ragged
        // chunk's -2^121 padding set to -inf first)
        if (RRPad<BF16, NL>::low && start + CH > V) {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int a = RR_ID(i, 2 * q);
                    uint32_t x = raw[i][q];
                    if (a >= V) x = (x & 0xFFFF0000u) | 0xFF80u;
                    if (a + 1 >= V) x = (x & 0x0000FFFFu) | 0xFF800000u;
                    raw[i][q] = x;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            float x = rr_max3(RR_X(raw[i], 0), RR_X(raw[i], 1), RR_X(raw[i], 2));
#pragma unroll
            for (int e = 3; e < VEC; e += 2) x = rr_max3(x, RR_X(raw[i], e), RR_X(raw[i], e + 1 < VEC ? e + 1 : e));
            wm[i] = x;
        }
        tm = wm[0];
#pragma unroll
        for (int i = 1; i < NL; i += 2) tm = rr_max3(tm, wm[i], wm[i + 1 < NL ? i + 1 : i]);
    }
    // wave maximum and the candidate threshold: the K-th largest lane maximum
    // (exact, bit by bit; bf16 codes differ only in their top 16 bits) bounds
    // the workgroup's K-th largest element from below
    const uint32_t lo = tm > -INFINITY ? ord_f32(tm) : 0u;
    const uint32_t wmax = wave_max_u32(lo);
    uint32_t tau = wmax;                                       // K = 1: the wave maximum
    if (K > 1) {
        tau = 0u;
        for (int bit = 31; bit >= (BF16 ? 16 : 0); --bit) {
            const uint32_t cand = tau | (1u << bit);
            if (__popcll(__ballot(lo >= cand)) >= (unsigned)K) tau = cand;
        }
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
        if (tid < 2 + 2 * K) rr_st32(out + tid, tid == 0 ? __float_as_uint(-INFINITY) : 0u);
        __syncthreads();                                       // LDS free for the caller
        return;
    }
    const float M = unord_f32(bmax);
    const float tauf = bt ? unord_f32(bt) : -INFINITY;
    const float ML = M * DDT_LOG2E;
    // a wave holding the maximum tests for it, word by word, in the words
    // whose maximum is M
    const bool mwave = __ballot(tm == M) != 0ull;
    if (pk && K == 1 && mwave) {
#pragma unroll
        for (int i = 0; i < NL; ++i) wm[i] = __uint_as_float(pk_word(i) << 16);
    }
    // pass 2 unpacks the raw words again: no unpacked copies live across the
    // passes (registers, not instructions, would bound the wide chunks)
#pragma unroll
    for (int i = 0; i < NL; ++i) asm volatile("" : "+v"(raw[i]));

    // pass 2: sum of exp(x - M) over the elements below M and the count of
    // elements equal to M (sigma' leaves out exactly one of them; the others
    // add exp(0) = 1 each, put back below).  The raw exp2 flushes results
    // below 2^-126 to zero, far below the sum's precision.
    float s0 = 0.f, s1 = 0.f;
    int ties = 0;
    if (!sums) {
        // max and top K only
    } else if (!mwave) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
#pragma unroll
            for (int e = 0; e < VEC; e += 2) {
                s0 += __builtin_amdgcn_exp2f(fmaf(RR_X(raw[i], e), DDT_LOG2E, -ML));
                s1 += __builtin_amdgcn_exp2f(fmaf(RR_X(raw[i], e + 1), DDT_LOG2E, -ML));
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            if (__ballot(wm[i] == M)) {
#pragma unroll
                for (int e = 0; e < VEC; e += 2) {
                    const float x0 = RR_X(raw[i], e), x1 = RR_X(raw[i], e + 1);
                    ties += (x0 == M) + (x1 == M);
                    s0 += x0 == M ? 0.f : __builtin_amdgcn_exp2f(fmaf(x0, DDT_LOG2E, -ML));
                    s1 += x1 == M ? 0.f : __builtin_amdgcn_exp2f(fmaf(x1, DDT_LOG2E, -ML));
                }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; e += 2) {
                    s0 += __builtin_amdgcn_exp2f(fmaf(RR_X(raw[i], e), DDT_LOG2E, -ML));
                    s1 += __builtin_amdgcn_exp2f(fmaf(RR_X(raw[i], e + 1), DDT_LOG2E, -ML));
                }
            }
        }
    }
    float s = s0 + s1;
    if (ties) atomicAdd(&s_ties, ties);
    if (K == 1) {
        // argmax: the smallest id holding M (a lane's ids grow with (i, e))
        if (tm == M) {
            int idm = 0x7FFFFFFF;
#pragma unroll
            for (int i = NL - 1; i >= 0; --i) {
                if (wm[i] == M) {
#pragma unroll
                    for (int e = VEC - 1; e >= 0; --e)
                        if (RR_X(raw[i], e) == M) idm = RR_ID(i, e);
                }
            }
            atomicMin(&s_amin, idm);
        }
    } else {
        // candidates at or above the threshold go to the LDS list.  The lanes
        // of a wave whose maximum reaches the threshold (usually a few) stage
        // their loaded words in LDS; the whole wave then tests those elements,
        // one per lane, and appends the ones that qualify.  Ids need checking
        // only in a ragged chunk or when the threshold is -inf (padding
        // qualifies only against a threshold of -inf).
        const bool chk = !(tauf > -INFINITY) || start + CH > V;
        const uint64_t pm = __ballot(tm >= tauf);
        if (pm) {
            u32x4* st = s_stage + wid * RR_SW;
            int* sid = s_sid + wid * RR_SW;
            // the words whose maximum reaches the threshold, in (word, lane)
            // order, RR_SW at a time
            int nw = 0;                                  // words holding a candidate
            for (int b0 = 0; b0 == 0 || b0 < nw; b0 += RR_SW) {
                int c = 0;
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    const bool h = wm[i] >= tauf;
                    const uint64_t m = __ballot(h);
                    const int pos = c - b0 + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    if (h && pos >= 0 && pos < RR_SW) {
                        st[pos] = raw[i];
                        sid[pos] = start + (i * RR_NT + tid) * VEC;
                    }
                    c += __popcll(m);
                }
                nw = c;
                wave_lds_sync();
                // one staged word (VEC elements) per lane; a wave prefix of the
                // hit counts places the hits in the list
                const int nq = min(RR_SW, nw - b0);
                for (int q0 = 0; q0 < nq; q0 += DDT_WAVE) {
                    const int q = q0 + lane;
                    uint32_t hit = 0u;
                    u32x4 w = u32x4{0u, 0u, 0u, 0u};
                    int id0 = 0;
                    if (q < nq) {
                        w = st[q];
                        id0 = sid[q];
                        if (!chk) {                      // (block-uniform)
#pragma unroll
                            for (int e = 0; e < VEC; ++e) hit |= (uint32_t)(RR_X(w, e) >= tauf) << e;
                        } else {
#pragma unroll
                            for (int e = 0; e < VEC; ++e)
                                hit |= (uint32_t)((RR_X(w, e) >= tauf) & (id0 + e < V)) << e;
                        }
                    }
                    const int nh = __popc(hit);
                    const int incl = wave_incl_scan_i32(nh);
                    const int tot = __builtin_amdgcn_readlane(incl, DDT_WAVE - 1);
                    int base = 0;
                    if (lane == 0) base = atomicAdd(&s_cnt, tot);
                    base = __builtin_amdgcn_readfirstlane(base);
                    int slot = base + incl - nh;
                    while (hit) {
                        const int e = __ffs(hit) - 1;
                        hit &= hit - 1;
                        if (slot < RR_CAP) s_list[slot] = vkey(RR_X(w, e), id0 + e);
                        ++slot;
                    }
                }
                wave_lds_sync();                         // before the next batch is staged
            }
        }
    }
    s = wave_sumf(s);
    if (lane == 0) s_wsum[wid] = s;
    __syncthreads();
    const int cnt = s_cnt;
    uint64_t* okeys = (uint64_t*)(out + 2);
    if (K == 1) {
        if (tid == 0) rr_st64(okeys, vkey(M, s_amin));
    } else if (cnt <= RR_NT) {
        // the usual case (a few dozen candidates): fixed trip counts over the
        // zero-padded list, no remainder loops
        if (cnt <= RR_NT / 4) rr_rank_fixed<4>(s_list, cnt, K, okeys);
        else if (cnt <= RR_NT / 2) rr_rank_fixed<2>(s_list, cnt, K, okeys);
        else rr_rank_fixed<1>(s_list, cnt, K, okeys);
        for (int k = cnt + tid; k < K; k += RR_NT) rr_st64(okeys + k, 0ull);
    } else if (cnt <= RR_CAP) {
        // rank counting, each rank counted by S lanes: keys are unique, so
        // rank < K places the key exactly
        const int SL = split_lanes(cnt, RR_NT);
        const int lg = __ffs(SL) - 1;
        for (int cb = 0; cb < cnt; cb += RR_NT >> lg) {
            const int c = cb + (tid >> lg), part = tid & (SL - 1);
            uint64_t k = 0ull;
            int rank = 0;
            if (c < cnt) {
                k = s_list[c];
#pragma unroll 8
                for (int q = part; q < cnt; q += SL) rank += s_list[q] > k ? 1 : 0;
            }
            rank = group_sum(rank, SL);
            if (part == 0 && c < cnt && rank < K) rr_st64(okeys + rank, k);
        }
        for (int k = cnt + tid; k < K; k += RR_NT) rr_st64(okeys + k, 0ull);
    } else {
        // list overflow (massive ties): exact K rounds, each reading the
        // chunk again one 16-byte word at a time (keeping every element's key
        // in registers would set the register budget of the whole kernel)
        uint64_t prev = ~0ull;
        for (int k = 0; k < K; ++k) {
            uint64_t best = 0ull;
#pragma unroll 1
            for (int i = 0; i < NL; ++i) {
                u32x4 rw[1];
                rr_load<BF16, 1>(rw, row, al, start + i * RR_NT * VEC, V, tid);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    if (RR_ID(i, e) < V) {
                        const uint64_t v = vkey(RR_X(rw[0], e), RR_ID(i, e));
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
            if (tid == 0) rr_st64(okeys + k, best);
            prev = best;
        }
    }
    if (tid == 0) {
        float st = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) st += s_wsum[w];
        rr_st32(out, __float_as_uint(M));
        rr_st32(out + 1, __float_as_uint(sums ? st + (float)(s_ties - 1) : 0.f));
    }
    __syncthreads();                                           // LDS free for the caller
#undef RR_ID
}

// One workgroup reduces one chunk of one row.  Seven workgroups per compute
// unit (72 VGPRs) keep the wide chunks' waves resident seven to a SIMD; the
// register allocator would otherwise take a few more and leave six.
template <bool BF16, int NL>
__global__ __launch_bounds__(RR_NT, 7) void k_row_partial(RowSrc rs, int V, int groups, int K,
                                                       uint32_t* __restrict__ part) {
    __shared__ RRLds L;
    const int g = blockIdx.x % groups;
    const int rowg = blockIdx.x / groups;
    const int i0 = rowg / rs.n1, i1 = rowg - i0 * rs.n1;
    if (rs.count != nullptr && i1 >= rs.count[i0] + rs.count_add) return;   // block-uniform
    const bool sums = rs.sum_if == nullptr || rs.sum_if[i0] > 0.f;        // block-uniform
    const int64_t off = (int64_t)i0 * rs.s0 + (int64_t)i1 * rs.s1;
    const void* row = (const char*)rs.base + off * (BF16 ? 2 : 4);
    rr_chunk<BF16, NL>(row, V, g, K, sums, part + ((size_t)rowg * groups + g) * rr_ps(K), L);
}

#define MRG_CAP 128                      // candidate list per wave
#define MRG_SCR (MRG_CAP + 32)           // u64 LDS entries per wave: candidates + output


// Merge the `groups` partials of one row with one wave: row max M, sigma'
// (partials' sums rescaled to M, the excluded element taken from the first
// group holding M), and the row's top-K keys, lane k holding the k-th (key 0
// past the row's length).  scr: MRG_SCR entries of LDS private to the wave.
//
// Top-K: with j = ceil(K / groups), the j best keys of every group are
// groups * j >= K distinct keys of the row; T, the K-th largest value code
// among them, is at most the value code of the row's K-th best key, so every
// key of the row's top K has a value code of at least T.  The keys passing
// that test (typically little more than K of the groups * K) are ranked by
// counting.  When more than MRG_CAP pass (long runs of equal values) the top K
// is taken in K max-extraction rounds.
//
// The merge is split in two so that a kernel can request the partials of its
// rows together with its other inputs: merge_issue only issues the loads,
// merge_finish waits for them and merges.  live = false (a slot whose
// partials are not current): the wave returns M = -inf, sigma' = 0, no keys.
#define MRG_MR 4                         // keys held in registers per lane

struct MergeIn {
    float mc, sc;                        // group max and sigma' (lane < groups)
    uint32_t hv;                         // sampled value code (K > 1)
    uint64_t kk[MRG_MR];                 // keys lane + 64 r, when they fit
};

// q / d for 0 <= q < 2^12 and 1 <= d <= 64, given rd = 1/d to within two
// ulp: q * rd is then within 2^-11 of q/d (exact for d = 1), and a quotient
// that is not an integer is at least 1/d >= 2^-6 below the next one, so
// adding 2^-10 before truncating gives floor(q / d) exactly.  Three
// instructions instead of an integer division's fifteen or so.
__device__ __forceinline__ int small_div(int q, float rd) {
    return (int)fmaf((float)q, rd, 0x1p-10f);
}

// Every lane loads, from a clamped address inside the row's partials, so that
// the loads are straight-line code: a load under a branch ends in a register
// copy that waits for it.  merge_finish masks the lanes past the data.
template <bool COH = false>
__device__ __forceinline__ void merge_issue(const uint32_t* __restrict__ p, int groups, int K,
                                            MergeIn& in) {
    const int lane = threadIdx.x & (DDT_WAVE - 1);
    const int PS = rr_ps(K);
    const int jth = (K + groups - 1) / groups;         // 1 <= jth <= K (wave-uniform)
    const int total = groups * K;
    // (the hardware reciprocal: within one ulp, which small_div allows)
    const float rK = __builtin_amdgcn_rcpf((float)K), rj = __builtin_amdgcn_rcpf((float)jth);
    const int gl = lane < groups ? lane : 0;
    in.mc = __uint_as_float(rr_ld32<COH>(p + gl * PS));
    in.sc = __uint_as_float(rr_ld32<COH>(p + gl * PS + 1));
    // sample: the jth best keys of every group (groups * jth <= 64 lanes)
    const int hl = lane < groups * jth ? lane : 0;
    const int hc = small_div(hl, rj), he = hl - hc * jth;
    in.hv = rr_ld32<COH>(p + hc * PS + 2 + 2 * he + 1);   // high word (value code)
#pragma unroll
    for (int r = 0; r < MRG_MR; ++r) {
        const int q = lane + r * DDT_WAVE;
        const int qc = q < total ? q : 0;
        const int c = small_div(qc, rK), e = qc - c * K;
        in.kk[r] = rr_ld64<COH>((const uint64_t*)(p + c * PS + 2 + 2 * e));
    }
}

template <bool COH = false>
__device__ __forceinline__ uint64_t merge_finish(MergeIn& in, const uint32_t* __restrict__ p,
                                                 int groups, int K, float& M, float& Sp,
                                                 uint64_t* scr, bool live) {
    const int lane = threadIdx.x & (DDT_WAVE - 1);
    const int PS = rr_ps(K);
    const int jth = (K + groups - 1) / groups;
    const int total = groups * K;
    const bool fits = total <= MRG_MR * DDT_WAVE;
    // the loads stay ahead of this point (no sinking into the branch below)
    asm volatile("" : "+v"(in.mc), "+v"(in.sc), "+v"(in.hv));
#pragma unroll
    for (int r = 0; r < MRG_MR; ++r) asm volatile("" : "+v"(in.kk[r]));
    if (!live) {
        M = -INFINITY;
        Sp = 0.f;
        return 0ull;
    }
    const float mc = lane < groups ? in.mc : -INFINITY;
    const float sc = lane < groups ? in.sc : 0.f;
    const uint32_t hv = K > 1 && lane < groups * jth ? in.hv : 0u;
    constexpr int MR = MRG_MR;
    uint64_t kk[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) kk[r] = fits && lane + r * DDT_WAVE < total ? in.kk[r] : 0ull;
    M = unord_f32(wave_max_u32(lane < groups ? ord_f32(mc) : 0u));
    // T: the K-th largest sampled value code, bit by bit over the top 16 bits
    // (a lower T only admits a few more candidates); K = 1 needs none.  With
    // exactly K samples (groups * jth = K) it is the smallest sample's top 16
    // bits, the same value the search finds.
    uint32_t T = 0u;
    if (K > 1 && groups * jth == K) {
        T = wave_min_u32(lane < K ? hv : 0xFFFFFFFFu) & 0xFFFF0000u;
    } else {
        for (int bit = 31; K > 1 && bit >= 16; --bit) {
            const uint32_t cand = T | (1u << bit);
            if (__popcll(__ballot(hv >= cand)) >= (unsigned)K) T = cand;
        }
    }
    const uint64_t mm = __ballot(lane < groups && mc == M);
    const int cstar = mm ? __ffsll((unsigned long long)mm) - 1 : -1;
    float contrib = 0.f;
    if (lane < groups && mc > -INFINITY) {
        const float e = exp2f((mc - M) * DDT_LOG2E);
        contrib = sc * e + (lane != cstar ? e : 0.f);
    }
    Sp = wave_sumf(contrib);
    if (K == 1) {                                      // the best group head
        const uint64_t best = wave_max_key(kk[0]);
        return lane == 0 ? best : 0ull;
    }

    if (fits) {
        int nc = 0;
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const bool f = kk[r] != 0ull && (uint32_t)(kk[r] >> 32) >= T;
            const uint64_t m = __ballot(f);
            const int pos = nc + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (f && pos < MRG_CAP) scr[pos] = kk[r];
            nc += __popcll(m);
        }
        if (nc <= MRG_CAP) {
            if (lane < K) scr[MRG_CAP + lane] = 0ull;
            wave_lds_sync();
            if (nc <= DDT_WAVE) {
                // one candidate per lane, the others read through scalar registers
                const uint64_t x = lane < nc ? scr[lane] : 0ull;
                int r = 0;
                for (int q = 0; q < nc; ++q) r += readlane_u64(x, q) > x ? 1 : 0;
                if (lane < nc && r < K) scr[MRG_CAP + r] = x;
            } else {
                for (int i = lane; i < nc; i += DDT_WAVE) {
                    const uint64_t x = scr[i];
                    int r = 0;
#pragma unroll 4
                    for (int q = 0; q < nc; ++q) r += scr[q] > x ? 1 : 0;
                    if (r < K) scr[MRG_CAP + r] = x;
                }
            }
            wave_lds_sync();
            const uint64_t mine = lane < K ? scr[MRG_CAP + lane] : 0ull;
            wave_lds_sync();
            return mine;
        }
    }
    // K max-extraction rounds
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
                const uint64_t v = rr_ld64<COH>((const uint64_t*)(p + c * PS + 2 + 2 * e));
                if (v < prev && v > best) best = v;
            }
        }
        best = wave_max_key(best);
        if (lane == k) mine = best;
        prev = best;
    }
    return mine;
}

// K = 1 (argmax rows): the group maxima, sums and head keys only.
struct MergeIn1 {
    float mc, sc;
    uint64_t k0;
};

// Straight-line loads from clamped addresses, as in merge_issue.
__device__ __forceinline__ void merge1_issue(const uint32_t* __restrict__ p, int groups, MergeIn1& in) {
    const int lane = threadIdx.x & (DDT_WAVE - 1);
    constexpr int PS = 2 + 2 * 1;
    const int gl = lane < groups ? lane : 0;
    in.mc = __uint_as_float(p[gl * PS]);
    in.sc = __uint_as_float(p[gl * PS + 1]);
    in.k0 = *(const uint64_t*)(p + gl * PS + 2);
}

// The K = 1 merge_finish: lane 0 returns the row's best key; with stats =
// false (a greedy row: only its argmax is read) M and sigma' are not formed
// and read -inf and 0.
__device__ __forceinline__ uint64_t merge1_finish(const MergeIn1& in, int groups, float& M, float& Sp,
                                                  bool stats = true) {
    const int lane = threadIdx.x & (DDT_WAVE - 1);
    const bool on = lane < groups;
    if (!stats) {
        M = -INFINITY;
        Sp = 0.f;
        const uint64_t best = wave_max_key(on ? in.k0 : 0ull);
        return lane == 0 ? best : 0ull;
    }
    const float mc = on ? in.mc : -INFINITY;
    M = unord_f32(wave_max_u32(on ? ord_f32(mc) : 0u));
    const uint64_t mm = __ballot(on && mc == M);
    const int cstar = mm ? __ffsll((unsigned long long)mm) - 1 : -1;
    float contrib = 0.f;
    if (on && mc > -INFINITY) {
        const float e = exp2f((mc - M) * DDT_LOG2E);
        contrib = in.sc * e + (lane != cstar ? e : 0.f);
    }
    Sp = wave_sumf(contrib);
    const uint64_t best = wave_max_key(on ? in.k0 : 0ull);
    return lane == 0 ? best : 0ull;
}

__device__ __forceinline__ uint64_t merge_row_wave(const uint32_t* __restrict__ p, int groups, int K,
                                                   float& M, float& Sp, uint64_t* scr,
                                                   bool live = true) {
    MergeIn in;
    merge_issue(p, groups, K, in);
    return merge_finish(in, p, groups, K, M, Sp, scr, live);
}
