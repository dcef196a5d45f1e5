// Tree kernels: CAST's width/depth decision (run by the draft layer kernel),
// rerank, retrieval graft, flatten + mask, the select (rerank and flatten in
// one launch), accept walk, successor refresh.  One workgroup per batch row
// unless noted; every index derived from device state is bounded by the
// capacities passed in, so corrupt state cannot push an access out of range.
#pragma once
#include "ddt_device.hpp"
#include "ddt_rowreduce.hpp"
#include "../../include/ddt.h"

// ---------------------------------------------------------------------------
// CAST width and depth for the whole batch
// ---------------------------------------------------------------------------
//
// CAST notes, key design 2: width n_i = anchor scan of the batch-averaged
// cumulative utility u_k of the layer's sorted values e^S against the cost
// c_k = S_D[sel(ctx)][k] / S_T[sel(ctx)][1] and threshold C1[i].  Key design
// 3: FIFO A of the last R gain ratios u_n(i)/u_n(i-1), initially {1}; grow
// another layer iff mean(A) * u_n / c_n >= C2 (and the depth cap allows).
// Key design 1: select(c) = min(floor(c/L), M-1) (the printed max is read as
// min).  State lives in t.cast_state: [0..7] FIFO, [8] length, [9] previous
// u_n, [10] context (tree tokens fed so far).

__device__ __forceinline__ int cast_sel_row(long long c, int L, int M) {
    long long r = c / L;
    return (int)(r < M - 1 ? r : M - 1);
}

// Anchor scan over cumulative utility u[1..kmax] and cost c[1..kmax] (LDS):
// keep 1, then for k = 2..kmax move the anchor a to k when the average
// marginal (u_k - u_a) / (c_k - c_a) reaches C; a non-increasing cost step
// counts as an infinite marginal when utility grows.  The test is written
// u_k - u_a >= C (c_k - c_a), which differs from the quotient only at a
// rounding boundary.  One wave: a run of moves to adjacent items is found
// with one ballot over (k-1, k) pairs, a search from a fixed anchor with one
// ballot per 64 items, so a typical scan takes a handful of steps.  Every
// lane returns the same count.
__device__ __forceinline__ bool anchor_moves(const double* u, const double* c, double C, int a, int k) {
    const double du = u[k] - u[a], dc = c[k] - c[a];
    return dc > 0.0 ? du >= C * dc : du > 0.0;
}

__device__ int anchor_scan_wave(const double* u, const double* c, double C, int kmax) {
    if (kmax <= 0) return 0;
    const int lane = threadIdx.x & (DDT_WAVE - 1);
    int a = 1, k0 = 2;                       // items below k0 are settled
    while (k0 <= kmax) {
        int hit = -1;
        if (a == k0 - 1) {
            // walk: first k >= k0 whose adjacent step does not move
            for (int base = k0; base <= kmax && hit < 0; base += DDT_WAVE) {
                const int k = base + lane;
                const uint64_t m = __ballot(k <= kmax && !anchor_moves(u, c, C, k - 1, k));
                if (m) hit = base + __ffsll((unsigned long long)m) - 1;
            }
            if (hit < 0) return kmax;
            a = hit - 1;
            k0 = hit + 1;
        } else {
            // fixed anchor: first k >= k0 it moves to
            for (int base = k0; base <= kmax && hit < 0; base += DDT_WAVE) {
                const int k = base + lane;
                const uint64_t m = __ballot(k <= kmax && anchor_moves(u, c, C, a, k));
                if (m) hit = base + __ffsll((unsigned long long)m) - 1;
            }
            if (hit < 0) return a;
            a = hit;
            k0 = hit + 1;
        }
    }
    return a;
}

// CAST's batch rule runs in the last workgroup of a layer, on inputs staged
// in LDS: the rows' frontier values, the per-round state and the width costs
// of the layer's context row.  Cost tables hold at most DDT_CAST_MAX_M rows.
#define DDT_CAST_MAX_M 64

struct CastView {
    double* st;       // [16] state: FIFO [0..7], length, previous u_n, context; [11] C1 of
                      // the layer, [12] 1/B
    double* c;        // [R_max] width costs c_k = S_D[sel(ctx)][k] / S_T[sel(ctx)][1], k = 1..
};

// Wave-level helpers for the batch rule (wave 0, all 64 lanes active).
// x from lane l (l wave-uniform), through scalar registers.
__device__ __forceinline__ double readlane_f64(double x, int l) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// DPP move of a double (both halves); lanes without a source, and rows
// outside RM, read 0.
template <int CTRL, int RM>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, RM, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, RM, 0xF, true);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// row of 16, then the totals of earlier rows by broadcast.
__device__ __forceinline__ double wave_incl_scan_f64(double x) {
    x += dpp_f64<0x111, 0xF>(x);
    x += dpp_f64<0x112, 0xF>(x);
    x += dpp_f64<0x114, 0xF>(x);
    x += dpp_f64<0x118, 0xF>(x);
    x += dpp_f64<0x142, 0xA>(x);
    x += dpp_f64<0x143, 0xC>(x);
    return x;
}

// Anchor scan with item k (1-based, k <= kmax <= 64) in lane k - 1: u = u_k,
// c = c_k.  Keeps 1, moves the anchor a to k when u_k - u_a >= C (c_k - c_a)
// (a non-increasing cost step moves it when utility grows); same walk as
// anchor_scan_wave, on ballot masks instead of LDS.  Returns the anchor
// (0 when kmax = 0); every lane gets it.
__device__ __forceinline__ int anchor_scan_regs(double u, double c, double C, int kmax) {
    const int lane = threadIdx.x & (DDT_WAVE - 1);
    const bool item = lane < kmax;
    const double up = __shfl_up(u, 1), cpv = __shfl_up(c, 1);
    const bool adj_moves = (c - cpv) > 0.0 ? (u - up) >= C * (c - cpv) : (u - up) > 0.0;
    // bit k-1 set: items k-1 -> k is a step the anchor does not take
    const uint64_t stop_adj = __ballot(lane >= 1 && item && !adj_moves);
    if (kmax <= 0) return 0;
    int a = 1, k0 = 2;
    while (k0 <= kmax) {
        if (a == k0 - 1) {
            const uint64_t m = stop_adj & (~0ull << (k0 - 1));
            if (!m) return kmax;
            const int hit = __ffsll((unsigned long long)m);          // lane + 1 = item
            a = hit - 1;
            k0 = hit + 1;
        } else {
            const double ua = readlane_f64(u, a - 1), ca = readlane_f64(c, a - 1);
            const double du = u - ua, dc = c - ca;
            const bool mv = dc > 0.0 ? du >= C * dc : du > 0.0;
            const uint64_t m = __ballot(item && lane + 1 >= k0 && mv);
            if (!m) return a;
            a = __ffsll((unsigned long long)m);
            k0 = a + 1;
        }
    }
    return a;
}

// The batch rule, run by wave 0 of the layer's last workgroup with mean (lane
// k - 1) = the batch average of e^S over every row's k-th frontier node (k <=
// kcap <= 32): width by the anchor scan on the batch-averaged cumulative utility,
// then the depth gate with the gain FIFO; every row's n_front gets the
// result.  Item k (1-based) lives in lane k - 1: u_k, c_k in registers; the
// anchor scan works on ballot masks and the FIFO on lanes 0..7.
//
// The depth gate is evaluated in every lane as if the width were n = lane + 1
// (push the gain ratio u_n / prev, drop the oldest entry when the FIFO then
// holds more than R, score = mean(FIFO) * u_n / c_n): the same operations, in
// the same order, as for the chosen n alone, but independent of the anchor
// scan, so that its divisions overlap the scan instead of following it; the
// chosen lane's values are then read.
__device__ void cast_decide(const CastView& L, const ddt_tree& t, const ddt_cast& cp, int layer, int kcap,
                            double mean) {
    const int lane = threadIdx.x & (DDT_WAVE - 1), B = t.B;
    if (layer == 1 && lane < t.D_max) t.widths[lane] = 0;
    // state (FIFO entries 0..7 one per lane, oldest first; length; previous
    // u_n, negative before the first layer's; context), C1, costs
    const double f = lane < 8 ? L.st[lane] : 0.0;
    const int len = (int)L.st[8];
    const double prev = L.st[9];
    const int ctx = (int)L.st[10];
    const double C1 = L.st[11];
    const bool item = lane < kcap;
    const double c = item ? L.c[lane] : 0.0;
    // column means of e^S (lane k - 1: item k), prefix-summed across lanes
    const double u = wave_incl_scan_f64(mean);
    // FIFO after the push: the entries kept (len <= R always, so a push drops
    // the oldest exactly when len == R) and their sum, oldest first; the new
    // ratio is added last
    const bool push = prev >= 0.0;
    const int drop = push && len >= cp.R ? 1 : 0;
    const int len2 = len + (push ? 1 : 0) - drop;
    double base = 0.0;
    for (int i = drop; i < len; ++i) base += readlane_f64(f, i);
    const double phi_l = push && prev > 0.0 ? u / prev : 0.0;
    const double fm_l = (push ? base + phi_l : base) / (double)len2;
    const double sc_l = fm_l * u / c;
    const int n = anchor_scan_regs(u, c, C1, kcap);
    const double un = n > 0 ? readlane_f64(u, n - 1) : 0.0;
    const double score = n > 0 ? readlane_f64(sc_l, n - 1) : 0.0;
    const double phi = n > 0 ? readlane_f64(phi_l, n - 1) : 0.0;    // 0 / prev = 0 for n = 0
    const bool stop = (layer >= t.D_max) || !(score >= (double)cp.C2);
    // the new FIFO: entries shifted down by one when the oldest is dropped
    // (lane i takes lane i + 1, within the first row of 16 lanes), the new
    // ratio in entry len2 - 1
    const double fsh = dpp_f64<0x101, 0xF>(f);
    double fn = drop ? fsh : f;
    if (push && lane == len2 - 1) fn = phi;
    double* st = t.cast_state;
    if (lane < 8) st[lane] = fn;
    if (lane == 8) st[8] = (double)len2;
    if (lane == 9) st[9] = un;
    if (lane == 10) st[10] = (double)(ctx + n);
    if (lane == 0) {
        t.widths[layer - 1] = n;
        t.cont[0] = stop ? 0 : 1;
    }
    // the frontier width goes out device-coherent: the requests' own stage
    // of the same launch stored it that way before
    if (lane < B) __hip_atomic_store(t.n_front + lane, stop ? 0 : n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// the draft layer (reduction, children, frontier, CAST) is k_expand_layer in
// ddt_layer.hpp; AT_SORT bounds the nodes one layer of a request creates
// ---------------------------------------------------------------------------
#define AT_SORT 1024

// ---------------------------------------------------------------------------
// rerank: top-m of all non-root nodes by (S desc, key asc)
// ---------------------------------------------------------------------------
//
// EAGLE-2 explainer, reranking section: every candidate node is ranked by
// value, the top m are verified; a child never outranks its parent and equal
// values go to the shallower node, so the set is a connected subtree.  CAST
// key design 4: m per row by the anchor scan of the sorted cumulative values
// against the verify cost.  Graft: m = the row's k_draft.
//
// Only the first m_max positions are needed.  A four-pass byte-wise radix
// select over the value codes finds T, the code of the m_max-th largest value;
// the nodes above T and the ties at T (up to RK_CAND in all) are ordered by
// rank counting on (value code, canonical key).  Rows with more ties at T than
// that fall back to a full bitonic sort of the row.

struct RerankArgs {
    ddt_tree t;
    ddt_cast c;
    int cast_on, use_k_draft, m_max;
    int32_t* sel;
    int32_t* m_out;
};

#define RK_NT 1024
#define RK_PER (DDT_MAX_NODES / RK_NT)   // nodes per thread
#define RK_SORT DDT_MAX_NODES
#define RK_CAND 1024
#define RK_SMALL 256                     // rows of at most this many nodes skip the select

// In-LDS bitonic sort of n2 (power of two) 64-bit keys, ascending.
template <int NT>
__device__ void bitonic_sort_u64(uint64_t* v, int n2) {
    for (int k = 2; k <= n2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            const int lj = __ffs(j) - 1;                     // j is a power of two
            for (int t = threadIdx.x; t < (n2 >> 1); t += NT) {
                const int i = ((t >> lj) << (lj + 1)) + (t & (j - 1));
                const int l = i + j;
                const uint64_t x = v[i], y = v[l];
                if ((x > y) == ((i & k) == 0)) { v[i] = y; v[l] = x; }
            }
            __syncthreads();
        }
    }
}

// Runs of equal value in sv[0 .. N) (sorted by (~code, node)) re-ordered by
// canonical key, one thread per run (runs are rare outside degenerate rows).
template <int NT>
__device__ void rerank_fix_ties(const uint64_t* key, int N, uint64_t* sv) {
    const int tid = threadIdx.x;
    for (int q = tid; q < N; q += NT) {
        const uint32_t hv = (uint32_t)(sv[q] >> 32);
        if ((q > 0 && (uint32_t)(sv[q - 1] >> 32) == hv) || q + 1 >= N ||
            (uint32_t)(sv[q + 1] >> 32) != hv)
            continue;
        int e = q + 1;
        while (e < N && (uint32_t)(sv[e] >> 32) == hv) ++e;
        for (int i = q + 1; i < e; ++i) {           // insertion sort by key
            const uint64_t x = sv[i];
            const uint64_t kx = key[(uint32_t)x];
            int j = i - 1;
            while (j >= q && key[(uint32_t)sv[j]] > kx) { sv[j + 1] = sv[j]; --j; }
            sv[j + 1] = x;
        }
    }
    __syncthreads();
}

// Fallback: full sort of the row's N non-root nodes by (~code, node), runs of
// equal value re-ordered by canonical key; writes the first kmax nodes to
// out_node in order.
template <int NT>
__device__ void rerank_sort_all(const float* S, const uint64_t* key, int N, int kmax, uint64_t* sv,
                                int32_t* out_node) {
    const int tid = threadIdx.x;
    const int n2 = next_pow2(N > 0 ? N : 1);
    for (int q = tid; q < n2; q += NT)
        sv[q] = q < N ? ((uint64_t)~ord_f32(S[1 + q]) << 32) | (uint32_t)(1 + q) : ~0ull;
    __syncthreads();
    bitonic_sort_u64<NT>(sv, n2);
    rerank_fix_ties<NT>(key, N, sv);
    for (int k = tid; k < kmax; k += NT) out_node[k] = (int32_t)(uint32_t)sv[k];
    __syncthreads();
}

// Node records of a small row (at most RK_SMALL nodes besides the root), left
// in LDS by the rerank for the flat layout of the same workgroup; indexed by
// node id.
struct NodeRecs {
    const uint64_t* key;
    const int32_t *tok, *par, *dep;
    bool ok;                             // the row was small: the tables are filled
};

// Request blockIdx.x's selection (one workgroup of RK_NT threads): writes sel
// and m_out, and leaves the selected nodes in rank order in LDS
// (*nodes_lds[k] for k < m).  Returns m.
__device__ int rerank_row(const RerankArgs& a, const int32_t** nodes_lds, NodeRecs* recs) {
    const ddt_tree& t = a.t;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    __shared__ int s_hist[256];
    __shared__ int s_bin, s_need, s_ngt, s_ntie, s_slot, s_m;
    __shared__ uint32_t s_T;
    __shared__ uint32_t s_ca[RK_CAND];
    __shared__ uint64_t s_ck[RK_CAND];
    __shared__ int32_t s_cn[RK_CAND];
    __shared__ int32_t s_node[DDT_MAX_VERIFY];
    __shared__ float s_sv[DDT_MAX_VERIFY];
    __shared__ double s_u[DDT_MAX_VERIFY + 1], s_c[DDT_MAX_VERIFY + 1];
    __shared__ uint64_t s_sort[RK_SORT];
    __shared__ uint64_t s_nkey[RK_SMALL + 1];
    __shared__ int32_t s_ntok[RK_SMALL + 1], s_npar[RK_SMALL + 1], s_ndep[RK_SMALL + 1];
    const int nn = min(max(t.n_nodes[b], 1), t.cap);
    const int N = nn - 1;
    const int kmax = min(a.m_max, N);
    const float* S = t.S + (size_t)b * t.cap;
    const uint64_t* key = t.key + (size_t)b * t.cap;

    // one round of loads: values and keys of this thread's nodes, verify costs.
    // Straight-line loads from clamped addresses (a load under a branch ends in
    // a register copy that waits for it); the values past the data are masked
    // after the loads.  The addresses are clamped to the row's capacity, not
    // to its node count, so that the loads go out together with the count's
    // instead of after it.
    const int cap1 = t.cap - 1;
    uint32_t o[RK_PER];
    uint64_t kk[RK_PER];
    float sraw[RK_PER];
#pragma unroll
    for (int i = 0; i < RK_PER; ++i) {
        const int q = tid + i * RK_NT;
        const int qc = q < cap1 ? q : 0;
        sraw[i] = S[1 + qc];
        kk[i] = key[1 + qc];
    }
    // records of node tid (root included) for the flat layout of a small row
    const int rn = tid <= cap1 ? tid : 0;
    const uint64_t r_key = key[rn];
    const int32_t r_tok = t.token[(size_t)b * t.cap + rn], r_par = t.parent[(size_t)b * t.cap + rn],
                  r_dep = t.depth[(size_t)b * t.cap + rn];
    // every value of a small row in each lane set lane + 64 j (wave 0's
    // threshold search), requested with the rest
    float s_all[RK_SMALL / DDT_WAVE];
#pragma unroll
    for (int j = 0; j < RK_SMALL / DDT_WAVE; ++j) {
        const int q = lane + j * DDT_WAVE;
        s_all[j] = S[1 + (q < cap1 ? q : 0)];
    }
    // verify costs c_k = S_T[row][k] / S_T[row][1] for k = tid + 1 (without
    // CAST the loads read the row's own values and are not used)
    const int kc = tid < min(a.m_max, cap1) ? tid : 0;             // (kmax <= both)
    const float* ST = S;
    if (a.cast_on) ST = a.c.S_T + (size_t)cast_sel_row(a.c.ctx_verify, a.c.L, a.c.M) * (a.c.N + 1);
    const float c_num = ST[kc + 1], c_den = ST[1];
    const float C3 = a.cast_on ? a.c.C3[b] : 0.f;       // requested with the rest
#pragma unroll
    for (int i = 0; i < RK_PER; ++i) {
        const int q = tid + i * RK_NT;
        o[i] = q < N ? ord_f32(sraw[i]) : 0u;
        kk[i] = q < N ? kk[i] : 0ull;
    }
    if (a.cast_on && tid < kmax) s_c[tid + 1] = (double)c_num / (double)c_den;
    if (tid == 0) { s_need = kmax; s_ngt = 0; s_ntie = 0; s_slot = 0; }

    // radix select: T = code of the kmax-th largest value (0 when every node
    // is kept; sorting mid-sized rows whole measured slower: a barrier of the
    // 1024-thread workgroup costs about 0.2 us, and a bitonic sort of 512
    // nodes takes 45 of them).  Small rows take a lower bound instead: wave 0
    // holds all their codes (four per lane) and finds, bit by bit over the top
    // 16 bits, the largest 16-bit prefix p with at least kmax codes >= p << 16;
    // then T' = p << 16 <= T (T's own prefix qualifies, and a larger T' would
    // leave fewer than kmax codes above T), and the few codes below T in T's
    // 16-bit bucket join the candidates.  Ranking every node of a 150-node row
    // cost 2.2 us against about 0.3 us for the search.
    const bool small = N <= RK_SMALL;
    if (small && tid <= N) { s_nkey[tid] = r_key; s_ntok[tid] = r_tok; s_npar[tid] = r_par; s_ndep[tid] = r_dep; }
    recs->key = s_nkey; recs->tok = s_ntok; recs->par = s_npar; recs->dep = s_ndep; recs->ok = small;
    uint32_t T = 0u;
    if (small) {
        // (the barrier also orders the counters' initialisation before the
        // listing's atomics)
        if (wid == 0) {
            uint32_t p = 0u;
            if (kmax > 0 && kmax < N) {
                uint32_t oc[RK_SMALL / DDT_WAVE];
#pragma unroll
                for (int j = 0; j < RK_SMALL / DDT_WAVE; ++j)
                    oc[j] = lane + j * DDT_WAVE < N ? ord_f32(s_all[j]) : 0u;
                for (int bit = 31; bit >= 16; --bit) {
                    const uint32_t cand = p | (1u << bit);
                    int c = 0;
#pragma unroll
                    for (int j = 0; j < RK_SMALL / DDT_WAVE; ++j) c += __popcll(__ballot(oc[j] >= cand));
                    if (c >= kmax) p = cand;
                }
            }
            if (lane == 0) s_T = p;
        }
        __syncthreads();
        T = s_T;
    } else if (kmax > 0 && kmax < N) {
        uint32_t prefix = 0u, pmask = 0u;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            if (tid < 256) s_hist[tid] = 0;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < RK_PER; ++i) {
                const int q = tid + i * RK_NT;
                const bool act = q < N && (o[i] & pmask) == prefix;
                const int bin = (int)((o[i] >> shift) & 255u);
                // the wave's most common bins first, one atomic each (many
                // nodes share the top byte of their code, and atomics on one
                // LDS word serialize); the rest one by one
                uint64_t pend = __ballot(act);
                for (int rd = 0; rd < 2 && pend; ++rd) {
                    const int leader = __ffsll((unsigned long long)pend) - 1;
                    const int lb = __builtin_amdgcn_readlane(bin, leader);
                    const uint64_t same = __ballot(act && bin == lb) & pend;
                    if (lane == leader) atomicAdd(&s_hist[lb], (int)__popcll(same));
                    pend &= ~same;
                }
                if ((pend >> lane) & 1ull) atomicAdd(&s_hist[bin], 1);
            }
            __syncthreads();
            if (wid == 0) {
                // lane l holds bins 255-4l .. 252-4l (descending)
                const int need = s_need;
                int h[4], loc = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) { h[i] = s_hist[255 - 4 * lane - i]; loc += h[i]; }
                const int incl = wave_incl_scan_i32(loc);
                int ex = incl - loc;
                if (ex < need && need <= incl) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (ex < need && need <= ex + h[i]) { s_bin = 255 - 4 * lane - i; s_need = need - ex; }
                        ex += h[i];
                    }
                }
            }
            __syncthreads();
            prefix |= (uint32_t)s_bin << shift;
            pmask |= 0xFFu << shift;
        }
        T = prefix;
    }
    // candidates: every node strictly above T, and the ties at T (counted
    // per wave: one LDS atomic per wave, since atomics on one LDS word from
    // every thread serialize).  Small rows skip the count: all their nodes
    // fit the candidate list, and the listing's slot counter gives nc.
    if (!small) {
        int ngt = 0, ntie = 0;
#pragma unroll
        for (int i = 0; i < RK_PER; ++i) {
            const int q = tid + i * RK_NT;
            ngt += (q < N) & (o[i] > T);
            ntie += (q < N) & (o[i] == T);
        }
        const int wgt = __builtin_amdgcn_readlane(wave_incl_scan_i32(ngt), DDT_WAVE - 1);
        const int wtie = __builtin_amdgcn_readlane(wave_incl_scan_i32(ntie), DDT_WAVE - 1);
        if (lane == 0 && wgt) atomicAdd(&s_ngt, wgt);
        if (lane == 0 && wtie) atomicAdd(&s_ntie, wtie);
        __syncthreads();
    }
    int nc = small ? 0 : s_ngt + s_ntie;
    int32_t* sel = a.sel + (size_t)b * (a.m_max + 1);
    if (kmax == 0) {
        // nothing to rank
    } else if (small || nc <= RK_CAND) {
        int mine = 0;
#pragma unroll
        for (int i = 0; i < RK_PER; ++i) mine += (tid + i * RK_NT < N) & (o[i] >= T);
        // slots: a wave prefix of the counts and one LDS atomic per wave
        const int incl = wave_incl_scan_i32(mine);
        const int wtot = __builtin_amdgcn_readlane(incl, DDT_WAVE - 1);
        int wbase = 0;
        if (lane == 0 && wtot) wbase = atomicAdd(&s_slot, wtot);
        int slot = __builtin_amdgcn_readfirstlane(wbase) + incl - mine;
#pragma unroll
        for (int i = 0; i < RK_PER; ++i) {
            const int q = tid + i * RK_NT;
            if (q < N && o[i] >= T) { s_ca[slot] = ~o[i]; s_ck[slot] = kk[i]; s_cn[slot] = 1 + q; ++slot; }
        }
        __syncthreads();
        if (small) nc = s_slot;
        // rank of candidate c, counted by S lanes (nc <= RK_CAND = RK_NT)
        const int SL = split_lanes(nc, RK_NT);
        const int lg = __ffs(SL) - 1;
        const int c = tid >> lg, part = tid & (SL - 1);
        uint32_t ca = 0u;
        uint64_t ck = 0ull;
        int r = 0;
        if (c < nc) {
            ca = s_ca[c];
            ck = s_ck[c];
            // branch-free: equal value codes are common (bf16 logits repeat),
            // and a branch per tie measured slower than the second load
#pragma unroll 4
            for (int p = part; p < nc; p += SL) {
                const uint32_t pa = s_ca[p];
                r += (int)(pa < ca) | ((int)(pa == ca) & (int)(s_ck[p] < ck));
            }
        }
        r = group_sum(r, SL);
        if (part == 0 && c < nc && r < kmax) {
            s_node[r] = s_cn[c];
            s_sv[r] = unord_f32(~ca);
        }
        __syncthreads();
    } else {
        rerank_sort_all<RK_NT>(S, key, N, kmax, s_sort, s_node);
        for (int k = tid; k < kmax; k += RK_NT) s_sv[k] = S[s_node[k]];
        __syncthreads();
    }
    // verify count
    if (a.cast_on && kmax <= DDT_WAVE) {
        // item k in lane k - 1: cumulative values and costs in registers
        if (wid == 0) {
            const bool item = lane < kmax;
            const double v = item ? (double)expf(s_sv[lane]) : 0.0;
            const double u = wave_incl_scan_f64(v);
            const double c = item ? s_c[lane + 1] : 0.0;
            const int m = anchor_scan_regs(u, c, (double)C3, kmax);
            if (lane == 0) s_m = m;
        }
    } else if (a.cast_on) {
        for (int k = tid; k < kmax; k += RK_NT) s_u[k + 1] = (double)expf(s_sv[k]);
        __syncthreads();
        if (wid == 0) {
            // prefix sums: four consecutive items per lane, then across lanes
            double loc[4], run = 0.0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = 4 * lane + i + 1;
                run += k <= kmax ? s_u[k] : 0.0;
                loc[i] = run;
            }
            double incl = run;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const double v = __shfl_up(incl, d);
                if (lane >= d) incl += v;
            }
            const double ex = incl - run;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = 4 * lane + i + 1;
                if (k <= kmax) s_u[k] = ex + loc[i];
            }
            if (lane == 0) { s_u[0] = 0.0; s_c[0] = 0.0; }
            wave_lds_sync();
            const int m = anchor_scan_wave(s_u, s_c, (double)C3, kmax);
            if (lane == 0) s_m = m;
        }
    } else if (tid == 0) {
        s_m = a.use_k_draft ? min(max(t.k_draft[b], 0), kmax) : kmax;
    }
    __syncthreads();
    const int m = s_m;
    for (int k = tid; k <= a.m_max; k += RK_NT)
        sel[k] = k == 0 ? 0 : (k <= m ? s_node[k - 1] : -1);
    if (tid == 0) a.m_out[b] = m;
    *nodes_lds = s_node;
    return m;
}

__global__ __launch_bounds__(RK_NT) void k_rerank(RerankArgs a) {
    const int32_t* nodes;
    NodeRecs recs;
    rerank_row(a, &nodes, &recs);
}

// ---------------------------------------------------------------------------
// Graft retrieval graft: template envelope by successor-matrix row lookups
// ---------------------------------------------------------------------------
//
// Graft review step 2: root-centred retrieval, x_u = M[x_parent(u), r_u].
// Template (reading of "depth x width"): `width` chains under the anchor (the
// root; or, for the tail-only graft of the Fig. 2 comparison, the tail of the
// selected draft tree); chain c starts with successor c of the anchor's token
// and continues with successor 0 of its own last token; level-major order,
// the first K_ret = K_max - m kept; no level past the canonical key's depth.

struct GatherArgs {
    ddt_tree t;
    const int32_t* M;
    int64_t M_bstride;
    int V, k_succ, depth, width, K_max, m_cap, anchor;
    int32_t* sel;
    int32_t* m_out;
};

__global__ __launch_bounds__(64) void k_succ_gather(GatherArgs a) {
    const ddt_tree& t = a.t;
    const int b = blockIdx.x, c = threadIdx.x;
    __shared__ int s_kret, s_base, s_m, s_anc, s_lv;
    const size_t o = (size_t)b * t.cap;
    int32_t* sel = a.sel + (size_t)b * (a.m_cap + 1);
    const int m = min(max(a.m_out[b], 0), a.K_max);
    // the anchor: the root, or the deepest selected node (ties: higher S,
    // then smaller key), each lane over its share of sel[1 .. m], then the wave
    int anc = 0;
    if (a.anchor == 1) {
        int bd = -1;
        float bS = -INFINITY;
        uint64_t bk = ~0ull;
        for (int q = 1 + c; q <= m; q += 64) {
            const int nd = sel[q];
            if (nd < 1 || nd >= t.cap) continue;
            const int d = t.depth[o + nd];
            const float S = t.S[o + nd];
            const uint64_t k = t.key[o + nd];
            if (d > bd || (d == bd && (S > bS || (S == bS && k < bk)))) { bd = d; bS = S; bk = k; anc = nd; }
        }
#pragma unroll
        for (int w = 32; w >= 1; w >>= 1) {
            const int od = __shfl_xor(bd, w);
            const float oS = __shfl_xor(bS, w);
            const uint64_t ok = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(bk >> 32), w) << 32) |
                                (uint32_t)__shfl_xor((int)(uint32_t)bk, w);
            const int oa = __shfl_xor(anc, w);
            if (od > bd || (od == bd && (oS > bS || (oS == bS && ok < bk)))) { bd = od; bS = oS; bk = ok; anc = oa; }
        }
    }
    if (c == 0) {
        int kret = a.K_max - m;
        const int base = min(max(t.n_nodes[b], 1), t.cap);
        const int ad = min(max(t.depth[o + anc], 0), DDT_MAX_DEPTH);
        const int lv = min(a.depth, DDT_MAX_DEPTH - ad);
        kret = min(kret, min(t.cap - base, lv * a.width));
        s_kret = max(kret, 0); s_base = base; s_m = m; s_anc = anc; s_lv = lv;
    }
    __syncthreads();
    const int kret = s_kret, base = s_base, lv = s_lv;
    const int32_t* Mb = a.M + (size_t)b * a.M_bstride;
    if (c < a.width) {
        int prev = s_anc;                          // parent node (the anchor for level 1)
        int ptok = t.token[o + prev];
        for (int lvl = 1; lvl <= lv; ++lvl) {
            const int idx = (lvl - 1) * a.width + c;
            if (idx >= kret) break;
            const int r = lvl == 1 ? c : 0;
            const int pt = min(max(ptok, 0), a.V - 1);
            const int tk = Mb[(size_t)pt * a.k_succ + r];
            const int node = base + idx;
            const int pd = t.depth[o + prev];
            t.token[o + node] = tk;
            t.parent[o + node] = prev;
            t.depth[o + node] = pd + 1;
            t.eslot[o + node] = -1;
            t.key[o + node] = key_child(t.key[o + prev], pd, r, 1);
            t.S[o + node] = -INFINITY;
            t.logc[o + node] = -INFINITY;
            if (1 + m + idx <= a.m_cap) sel[1 + m + idx] = node;
            prev = node;
            ptok = tk;
        }
    }
    __syncthreads();
    if (c == 0) {
        t.n_nodes[b] = base + kret;
        a.m_out[b] = min(m + kret, a.m_cap);
    }
}

// ---------------------------------------------------------------------------
// flatten + ancestor mask + position ids + retrieve paths
// ---------------------------------------------------------------------------
//
// EAGLE-2 explainer, reranking section (flatten to a 1-D list, mask by the
// tree) and engineering difficulty one (mask by parent relation, never by
// linear position); Graft review step 3 (tree position ids, ancestor mask,
// candidate path indices).  Flat order: ascending canonical key.

struct MaskArgs {
    ddt_tree t;
    ddt_flat f;
    const int32_t* sel;
    const int32_t* m;
    int prefix;
    uint8_t* dense;
};

#define MK_NT 256

// Request blockIdx.x's flat layout by one workgroup of NT >= MK_NT threads,
// P <= MK_NT.  The selection comes from sel (global) or, when nodes_lds is
// given, from the rerank of the same workgroup (node of selection index k >= 1
// at nodes_lds[k - 1], m given).  One round of global loads for the selected
// nodes' key, token, parent and depth; flat indices by rank counting on the
// keys; a node -> flat index table in LDS gives each node's flat parent;
// leaves are numbered by a ballot prefix sum.
template <int NT>
__device__ void mask_row(const MaskArgs& a, int m_in, const int32_t* nodes_lds) {
    const ddt_tree& t = a.t;
    const ddt_flat& f = a.f;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int P = f.P, W = f.W, Dp = f.Dp, cap = t.cap;
    __shared__ uint64_t s_key[MK_NT];
    __shared__ int32_t s_node[MK_NT], s_tok[MK_NT], s_par[MK_NT], s_dep[MK_NT];
    __shared__ int32_t s_fnode[MK_NT], s_ftok[MK_NT], s_fpn[MK_NT], s_fdep[MK_NT];
    __shared__ int s_fp[MK_NT], s_hc[MK_NT], s_lidx[MK_NT];
    __shared__ int16_t s_inv[DDT_MAX_NODES];
    __shared__ int s_woff[NT / 64];
    const int m = min(max(m_in, 0), P - 1);
    const int n = m + 1;
    const size_t o = (size_t)b * cap;
    const int32_t* sel = a.sel + (size_t)b * P;
    // the selection (issued with the count), then the selected nodes' records:
    // straight-line loads from clamped addresses, masked afterwards (a load
    // under a branch ends in a register copy that waits for it)
    for (int q = tid; q < P; q += NT) {
        const int raw = nodes_lds == nullptr ? sel[q] : (q == 0 ? 0 : nodes_lds[q - 1]);
        int node = q <= m ? raw : -1;
        if (node < 0 || node >= cap) node = -1;
        const int nc = node >= 0 ? node : 0;
        const uint64_t kv = t.key[o + nc];
        const int32_t tv = t.token[o + nc], pv = t.parent[o + nc], dv = t.depth[o + nc];
        s_node[q] = node;
        s_key[q] = node >= 0 ? kv : ~0ull;
        s_tok[q] = node >= 0 ? tv : -1;
        s_par[q] = node >= 0 ? pv : -1;
        s_dep[q] = node >= 0 ? dv : 0;
        s_hc[q] = 0;
    }
    for (int i = tid; i < cap; i += NT) s_inv[i] = -1;
    __syncthreads();
    // flat index = rank of the key among the selected keys (keys are unique)
    for (int q = tid; q < n; q += NT) {
        const uint64_t k = s_key[q];
        int r = 0;
#pragma unroll 8
        for (int p = 0; p < n; ++p) r += s_key[p] < k ? 1 : 0;
        s_fnode[r] = s_node[q]; s_ftok[r] = s_tok[q]; s_fpn[r] = s_par[q]; s_fdep[r] = s_dep[q];
        if (s_node[q] >= 0) s_inv[s_node[q]] = (int16_t)r;
    }
    __syncthreads();
    const size_t fo = (size_t)b * P;
    for (int i = tid; i < P; i += NT) {
        int node = -1, tk = -1, fp = -1, d = 0;
        if (i < n && s_fnode[i] >= 0) {
            node = s_fnode[i];
            tk = s_ftok[i];
            const int pn = s_fpn[i];
            fp = (pn >= 0 && pn < cap) ? (int)s_inv[pn] : -1;
            d = s_fdep[i];
        }
        f.node[fo + i] = node;
        f.token[fo + i] = tk;
        f.parent[fo + i] = fp;
        f.pos[fo + i] = a.prefix + d;
        s_fp[i] = fp; s_fdep[i] = d;
        if (i >= 1 && i < n && fp >= 0) s_hc[fp] = 1;
    }
    __syncthreads();
    // leaves (no selected child), numbered in flat order
    {
        const bool leaf = tid < n && !s_hc[tid];
        const uint64_t bal = __ballot(leaf);
        if (lane == 0) s_woff[wid] = __popcll(bal);
        __syncthreads();
        int off = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) { off += w < wid ? s_woff[w] : 0; tot += s_woff[w]; }
        if (tid < P)
            s_lidx[tid] = leaf ? off + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u)) : -1;
        if (tid == 0) { f.n_leaves[b] = tot; f.m[b] = m; }
        __syncthreads();
    }
    // ancestor mask: one thread per (row, word), walking the parent chain
    const int cols = a.prefix + P;
    for (int q = tid; q < P * W; q += NT) {
        const int i = q / W, k = q - i * W;
        uint32_t word = 0u;
        int j = i, guard = 0;
        while (j >= 0 && guard++ <= DDT_MAX_DEPTH + 1) {
            if ((j >> 5) == k) word |= 1u << (j & 31);
            j = (i < n) ? s_fp[j] : -1;
        }
        f.mask[(fo + i) * W + k] = word;
        if (a.dense != nullptr) {
            uint8_t* dr = a.dense + ((size_t)b * P + i) * cols;
            if (k == 0)
                for (int col = 0; col < a.prefix; ++col) dr[col] = 1;
            for (int e = 0; e < 32 && k * 32 + e < P; ++e)
                dr[a.prefix + k * 32 + e] = (uint8_t)((word >> e) & 1u);
        }
    }
    const int L = f.L;
    int32_t* ret = f.retrieve + (size_t)b * L * (Dp + 1);
    int nl = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) nl += s_woff[w];
    for (int i = tid; i < n; i += NT) {
        const int li = s_lidx[i];
        if (li < 0 || li >= L) continue;
        int32_t* row = ret + (size_t)li * (Dp + 1);
        const int d = min(s_fdep[i], Dp);
        for (int s2 = d + 1; s2 <= Dp; ++s2) row[s2] = -1;
        int j = i;
        for (int s2 = d; s2 >= 0; --s2) {
            row[s2] = j;
            j = j >= 0 ? s_fp[j] : -1;
        }
    }
    for (int q = nl * (Dp + 1) + tid; q < L * (Dp + 1); q += NT) ret[q] = -1;
}

__global__ __launch_bounds__(MK_NT) void k_build_mask(MaskArgs a) {
    mask_row<MK_NT>(a, a.m[blockIdx.x], nullptr);
}

// The flat layout of a small selection (m + 1 <= P <= 64 positions, no dense
// mask) by wave 0 alone, from the rerank's LDS: the node records were loaded
// with the values, so no second round of global loads.  Lane q holds
// selection row q, then lane i flat row i.  Same outputs as mask_row: flat
// index = rank of the canonical key among the selected keys; parents through
// a node -> flat index table; the ancestor sets (mask rows) by pointer
// doubling over the flat parents (six steps reach depth 63); leaves by ballot;
// a leaf's retrieve row lists its ancestor set's flat indices in ascending
// order (a parent precedes its children in key order).
__device__ void flat_small(const MaskArgs& a, int m_in, const int32_t* nodes_lds, const NodeRecs& r,
                           int N) {
    const ddt_flat& f = a.f;
    const int b = blockIdx.x, lane = threadIdx.x & 63;
    const int P = f.P, W = f.W, Dp = f.Dp, L = f.L;
    __shared__ int32_t s_fnode[DDT_WAVE], s_ftok[DDT_WAVE], s_fpn[DDT_WAVE], s_fdep[DDT_WAVE];
    __shared__ int s_hc[DDT_WAVE];
    __shared__ uint64_t s_selk[DDT_WAVE];
    __shared__ int16_t s_inv[RK_SMALL + 1];
    const int m = min(max(m_in, 0), P - 1);
    const int n = m + 1;
    // selection row q = lane: its node (row 0 the root) and key
    const int nq = lane == 0 ? 0 : (lane < n ? nodes_lds[lane - 1] : 0);
    const int nqc = nq >= 0 && nq <= N ? nq : 0;
    const uint64_t kq = lane < n ? r.key[nqc] : ~0ull;
    // flat index: the number of selected keys below this row's (broadcast
    // LDS reads, eight in flight)
    s_selk[lane] = kq;
    for (int i = lane; i <= N; i += DDT_WAVE) s_inv[i] = -1;
    s_hc[lane] = 0;
    wave_lds_sync();
    int rk = 0;
#pragma unroll 8
    for (int p = 0; p < n; ++p) rk += s_selk[p] < kq ? 1 : 0;
    if (lane < n) {
        s_fnode[rk] = nq; s_ftok[rk] = r.tok[nqc]; s_fpn[rk] = r.par[nqc]; s_fdep[rk] = r.dep[nqc];
        if (nq >= 0 && nq <= N) s_inv[nq] = (int16_t)rk;
    }
    wave_lds_sync();
    // flat row i = lane
    const int i = lane;
    int node = -1, tk = -1, fp = -1, d = 0;
    if (i < n) {
        node = s_fnode[i];
        tk = s_ftok[i];
        const int pn = s_fpn[i];
        fp = (pn >= 0 && pn <= N) ? (int)s_inv[pn] : -1;
        d = s_fdep[i];
    }
    const size_t fo = (size_t)b * P;
    if (i < P) {
        f.node[fo + i] = node;
        f.token[fo + i] = tk;
        f.parent[fo + i] = fp;
        f.pos[fo + i] = a.prefix + d;
    }
    if (i >= 1 && i < n && fp >= 0) s_hc[fp] = 1;
    // ancestor sets: M_i = {i} and the ancestors within 2^k - 1 steps,
    // anc = the ancestor 2^k steps up (-1 past the root); 2^steps exceeds the
    // deepest selected row's depth (a chain of selected rows is at most that
    // long: a parent precedes its child in flat order)
    uint64_t M = 1ull << i;
    int anc = (i < n && fp >= 0 && fp < i) ? fp : -1;
    const int dmax = (int)wave_max_u32(i < n ? (uint32_t)max(d, 0) : 0u);
    const int steps = dmax > 0 ? min(32 - __clz(dmax), 6) : 0;
    for (int k = 0; k < steps; ++k) {
        const int src = anc >= 0 ? anc : lane;
        const uint64_t Ma = ((uint64_t)(uint32_t)__shfl((int)(uint32_t)(M >> 32), src) << 32) |
                            (uint32_t)__shfl((int)(uint32_t)M, src);
        const int aa = __shfl(anc, src);
        if (anc >= 0) { M |= Ma; anc = aa; }
    }
    if (i < P)
        for (int k = 0; k < W; ++k) f.mask[(fo + i) * W + k] = (uint32_t)(M >> (32 * k));
    wave_lds_sync();
    // leaves (no selected child), numbered in flat order
    const bool leaf = i < n && !s_hc[i];
    const uint64_t bal = __ballot(leaf);
    const int nl = (int)__popcll(bal);
    if (lane == 0) { f.n_leaves[b] = nl; f.m[b] = m; }
    int32_t* ret = f.retrieve + (size_t)b * L * (Dp + 1);
    const int li = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (leaf && li < L) {
        int32_t* row = ret + (size_t)li * (Dp + 1);
        const int dd = min(d, Dp);
        uint64_t x = M;
        for (int s2 = Dp; s2 >= 0; --s2) {
            int v = -1;
            if (s2 <= dd && x) {
                v = 63 - __clzll((long long)x);
                x &= ~(1ull << v);
            }
            row[s2] = v;
        }
    }
    for (int q = nl * (Dp + 1) + lane; q < L * (Dp + 1); q += DDT_WAVE) ret[q] = -1;
}

// rerank and flat layout of one request in one workgroup (no Graft template
// between them): the selection stays in LDS
__global__ __launch_bounds__(RK_NT) void k_select(RerankArgs ra, MaskArgs ma) {
    const int32_t* nodes;
    NodeRecs recs;
    const int m = rerank_row(ra, &nodes, &recs);
    if (recs.ok && ma.f.P <= DDT_WAVE && ma.dense == nullptr) {
        if (threadIdx.x < DDT_WAVE) {
            const int N = min(max(ra.t.n_nodes[blockIdx.x], 1), ra.t.cap) - 1;
            flat_small(ma, m, nodes, recs, N);
        }
        return;
    }
    mask_row<RK_NT>(ma, m, nodes);
}

// ---------------------------------------------------------------------------
// accept walk
// ---------------------------------------------------------------------------
//
// EAGLE-2 explainer: at T = 0 acceptance is an argmax match along candidate
// paths (losslessness section); at T > 0 a drafted token x is accepted with
// probability min(1, p(x)/q(x)) and a rejection resamples from
// norm(max(0, p - q)) (ledger section), q being the distribution x was
// proposed from.  Tree reading: siblings are tried in flat order with the
// residual carried between them.  Point-mass proposals (every child in the
// point mode, Graft retrieval children always) take q = delta_x: accept with
// probability p_k(x), a rejection removes x from the residual; the draft
// rows are then not read.

struct VerifyArgs {
    ddt_tree t;
    int G;                 // workgroups per request
    int point;             // 1: every child is a point-mass proposal
    unsigned spin_limit;   // bound of the cross-workgroup wait (polls)

    ddt_flat f;
    const uint32_t* part;
    int chunks, Kp;
    const void* tgt;
    int bf16, V;
    int64_t ts0, ts1;
    const void* drf;
    int64_t dl, ds0, ds1;
    const float* temperature;
    const float* U;
    int k_top;
    int32_t* row_topk;
    int32_t* row_argmax;
    int32_t* accept_len;
    int32_t* accept_path;
    int32_t* next_token;
};

#define VF_NT 1024
#define VF_RET 3072           // candidate-path entries staged in LDS
#define VF_TILE 256            // one wave x 4 elements
#define VF_MAXTILES 2048       // V <= 524288

// 4 consecutive logits starting at v0 (a multiple of 4); -inf past V
__device__ __forceinline__ void ld4(const void* row, bool bf16, bool al, int V, int v0, float (&x)[4]) {
    if (bf16) {
        const uint16_t* r = (const uint16_t*)row;
        if (al && v0 + 4 <= V) {
            const uint2 w = *(const uint2*)(r + v0);
            x[0] = __uint_as_float(w.x << 16);
            x[1] = __uint_as_float(w.x & 0xFFFF0000u);
            x[2] = __uint_as_float(w.y << 16);
            x[3] = __uint_as_float(w.y & 0xFFFF0000u);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = v0 + e < V ? __uint_as_float((uint32_t)r[v0 + e] << 16) : -INFINITY;
        }
    } else {
        const float* r = (const float*)row;
        if (al && v0 + 4 <= V) {
            const u32x4 w = *(const u32x4*)(r + v0);
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] = __uint_as_float(w[q]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = v0 + e < V ? r[v0 + e] : -INFINITY;
        }
    }
}

__device__ __forceinline__ float ld_logit(const void* row, bool bf16, int v) {
    return bf16 ? __uint_as_float((uint32_t)((const uint16_t*)row)[v] << 16) : ((const float*)row)[v];
}

// The walk at one node: p(v) = 2^((t_v - Mt) kT - lzt) is the target softmax at
// temperature T (kT = log2(e) / T, lzt = log2 of its normaliser), q(v) likewise
// from the draft row.  After k rejections the residual is
// p_k = max(0, p - a_k q) / b_k with a_0 = 0, b_0 = 1, a_{k+1} = a_k + b_k and
// b_{k+1} = F(a_{k+1}) = sum_v max(0, p(v) - a_{k+1} q(v)): the repeated
// norm(max(0, p_k - q)) written out (an all-zero residual leaves p_k as it
// was), so each rejection costs one pass over the two rows and no division.
// Per-element values are fp64: b_k can be small when target and draft are
// close, and the error of p - a q is amplified by 1 / b_k.
// 2^x in fp64 for x <= 0 by Tang's table method: x = k/64 + r with
// |r| <= 1/128, 2^x = 2^(k>>6) * 2^((k&63)/64) * e^(r ln2).  The 64 table
// entries come from the library exp2 at kernel start; e^z for |z| < 0.0055 is
// a degree-5 Taylor polynomial (truncation below 4e-17).  Results below
// 2^-1100 are 0.
__device__ __forceinline__ double exp2_tab(double x, const double* tab) {
    x = fmax(x, -1100.0);
    const double k = rint(x * 64.0);
    const int ki = (int)k;
    const double r = fma(k, -0.015625, x);             // exact
    const double z = r * 0.6931471805599453094;
    double pz = fma(z, 1.0 / 120.0, 1.0 / 24.0);
    pz = fma(z, pz, 1.0 / 6.0);
    pz = fma(z, pz, 0.5);
    pz = fma(z, pz, 1.0);
    pz = fma(z, pz, 1.0);
    return ldexp(tab[ki & 63] * pz, ki >> 6);
}

struct WalkRows {
    const void* trow;
    const void* drow;
    const double* tab;                                 // 2^(j/64), j < 64 (LDS)
    bool bf16, alt, ald;
    double kT, Mt, Md, lzt, lzd;
};

__device__ __forceinline__ double walk_p(const WalkRows& w, float t) {
    return exp2_tab(((double)t - w.Mt) * w.kT - w.lzt, w.tab);
}
__device__ __forceinline__ double walk_q(const WalkRows& w, float d) {
    return exp2_tab(((double)d - w.Md) * w.kT - w.lzd, w.tab);
}

// A request's T > 0 walk may run on G workgroups, each over its own slice of
// the vocabulary (whole tiles).  Every workgroup takes the same decisions from
// the same totals; a pass's totals are combined through global memory:
// thread 0 stores the workgroup's sums in the pass's slot (two slots,
// alternating), releases, counts itself in, and spins (bounded) until all G
// have arrived.  A workgroup reaches pass k + 2's store only after all G
// arrived at pass k + 1, i.e. after every workgroup read pass k's slot.
// The wait is bounded (spin_limit polls).  A workgroup whose wait runs out
// leaves the walk; workgroup 0 then redoes that pass, and every later one,
// alone over the whole vocabulary, so the request still completes with the
// same decisions.
#define WALK_SPIN_LIMIT (1u << 22)

struct RowSync {
    double* buf;         // [2][G][2] pass sums
    double* tiles;       // [VF_MAXTILES] tile sums
    uint32_t* cnt;       // [0] arrivals (k + 1) * G after pass k, [1] exits
    unsigned limit;      // polls before the wait gives up
    int G, g, k;         // workgroups taking part (1 once alone), this one, passes so far
    int lo, hi;          // vocabulary slice [lo, hi)
    int t_lo, t_hi;      // the same slice in tiles
};

// The end of a pass: thread 0 adds the waves' sums (s_red: nw values, then
// nw more when two sums are taken), combines the two totals over the
// request's workgroups and broadcasts them through s_bc; every thread
// returns them.  Two barriers: one before thread 0 reads s_red (all waves
// have written it), one before the others read s_bc.  A later pass writes
// s_red only after the second barrier (thread 0 has read it) and s_bc only
// after its own first barrier (every thread has read it), so no further
// barrier is needed.  s_err is set on a timed-out wait.
__device__ void pass_end(RowSync& rs, const double* s_red, int nw, bool two, double& x0, double& x1,
                         double* s_bc, int* s_err) {
    __syncthreads();
    if (threadIdx.x == 0) {
        double a0 = 0.0, a1 = 0.0;
        for (int q = 0; q < nw; ++q) a0 += s_red[q];
        if (two)
            for (int q = 0; q < nw; ++q) a1 += s_red[nw + q];
        if (rs.G > 1) {
            // this workgroup's totals go to the pass's slot; release, count in,
            // and wait (bounded) for all G before reading every slot
            double* slot = rs.buf + (size_t)(rs.k & 1) * rs.G * 2;
            slot[2 * rs.g] = a0;
            slot[2 * rs.g + 1] = a1;
            __threadfence();
            atomicAdd(rs.cnt, 1u);
            const uint32_t target = (uint32_t)(rs.k + 1) * (uint32_t)rs.G;
            unsigned spins = 0;
            while (!*s_err &&
                   __hip_atomic_load(rs.cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                if (++spins > rs.limit) { *s_err = 1; break; }
                __builtin_amdgcn_s_sleep(2);
            }
            __threadfence();
            a0 = 0.0; a1 = 0.0;
            for (int q = 0; q < rs.G; ++q) {
                a0 += __hip_atomic_load(slot + 2 * q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                a1 += __hip_atomic_load(slot + 2 * q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        s_bc[0] = a0; s_bc[1] = a1;
    }
    __syncthreads();
    x0 = s_bc[0]; x1 = s_bc[1];
    if (rs.G > 1) rs.k++;
}

// block-wide sum over the slice of fn(t_v, d_v) in fp64, combined over the
// request's workgroups; when only the target row is needed (UseD false) the
// draft row is not read
template <bool UseD, class Fn>
__device__ double walk_pass(const WalkRows& w, RowSync& rs, double* s_red, double* s_bc, int* s_err,
                            int V, Fn fn) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    double acc = 0.0;
    for (int v0 = rs.lo + tid * 4; v0 < rs.hi; v0 += VF_NT * 4) {
        float tx[4], dx[4];
        ld4(w.trow, w.bf16, w.alt, V, v0, tx);
        if (UseD) ld4(w.drow, w.bf16, w.ald, V, v0, dx);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += fn(tx[e], UseD ? dx[e] : 0.f);
    }
    const double d = wave_sum_f64(acc);
    if (lane == 0) s_red[wid] = d;
    double tot, zero;
    pass_end(rs, s_red, VF_NT / 64, false, tot, zero, s_bc, s_err);
    return tot;
}

// both softmax normalisers of a node in one sweep over its two rows
__device__ void walk_norms(const WalkRows& w, RowSync& rs, double* s_red, double* s_bc, int* s_err,
                           int V, double& Zt, double& Zd) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    double at = 0.0, ad = 0.0;
    for (int v0 = rs.lo + tid * 4; v0 < rs.hi; v0 += VF_NT * 4) {
        float tx[4], dx[4];
        ld4(w.trow, w.bf16, w.alt, V, v0, tx);
        ld4(w.drow, w.bf16, w.ald, V, v0, dx);
#pragma unroll
        for (int e = 0; e < 4; ++e) { at += walk_p(w, tx[e]); ad += walk_q(w, dx[e]); }
    }
    at = wave_sum_f64(at);
    ad = wave_sum_f64(ad);
    if (lane == 0) { s_red[wid] = at; s_red[VF_NT / 64 + wid] = ad; }
    pass_end(rs, s_red, VF_NT / 64, true, Zt, Zd, s_bc, s_err);
}

// Per-tile sums (256 ids, one wave per tile) of the weights max(0, p - aa q)
// (p alone without q) over the slice, into s_tile and, with several
// workgroups, rs.tiles; returns the request's total.
__device__ double walk_tiles(const WalkRows& w, RowSync& rs, double* s_red, double* s_bc, int* s_err,
                             int V, bool useq, double aa, double* s_tile) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    double mine = 0.0;
    for (int tile = rs.t_lo + wid; tile < rs.t_hi; tile += VF_NT / 64) {
        float tx[4], dx[4];
        const int v0 = tile * VF_TILE + lane * 4;
        ld4(w.trow, w.bf16, w.alt, V, v0, tx);
        if (useq) ld4(w.drow, w.bf16, w.ald, V, v0, dx);
        double ls = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ls += useq ? fmax(0.0, walk_p(w, tx[e]) - aa * walk_q(w, dx[e])) : walk_p(w, tx[e]);
        const double ws = wave_sum_f64(ls);
        if (lane == 0) {
            s_tile[tile] = ws;
            if (rs.G > 1) rs.tiles[tile] = ws;
        }
        mine += ws;
    }
    // the tile sums this wave stored for the other workgroups are complete
    // (device scope) before the barrier that precedes the arrival count
    if (rs.G > 1) __threadfence();
    if (lane == 0) s_red[wid] = mine;
    double tot, zero;
    pass_end(rs, s_red, VF_NT / 64, false, tot, zero, s_bc, s_err);
    return tot;
}

// Inverse CDF over the tile sums in s_tile (all tiles of the request): the
// smallest id whose running sum (ascending ids) exceeds u * total, else the
// last id with mass.  The nz ids in zx carry no weight (the caller has taken
// them out of their tiles' sums).  Wave 0 finds the tile by a lane scan over the tile
// sums, then the id inside it.  Returns the id in every thread.
__device__ int walk_pick(const WalkRows& w, int V, bool useq, double aa, double u, double tot,
                         const double* s_tile, int* s_out, const int* zx, int nz) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int ntiles = (V + VF_TILE - 1) / VF_TILE;
    if (wid == 0) {
        const double thr = u * tot;
        const int tpl = (ntiles + 63) / 64;            // tiles per lane
        const int t0 = lane * tpl;
        double loc = 0.0;
        int lastpos_t = -1;
        for (int i = 0; i < tpl; ++i) {
            const int tt = t0 + i;
            if (tt < ntiles) {
                loc += s_tile[tt];
                if (s_tile[tt] > 0.0) lastpos_t = tt;
            }
        }
        double incl = loc;
        for (int d = 1; d < 64; d <<= 1) {
            const double o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        const double ex = incl - loc;
        const uint64_t m = __ballot(incl > thr);
        int ts = -1;
        double base = 0.0;
        if (m) {
            const int L = __ffsll((unsigned long long)m) - 1;
            if (lane == L) {
                double acc = ex;
                for (int i = 0; i < tpl && ts < 0; ++i) {
                    const int tt = t0 + i;
                    if (tt >= ntiles) break;
                    if (acc + s_tile[tt] > thr) { ts = tt; base = acc; }
                    else acc += s_tile[tt];
                }
                if (ts < 0) { ts = lastpos_t >= 0 ? lastpos_t : t0; base = acc; }
            }
            ts = __shfl(ts, L);
            base = __shfl(base, L);
        } else {
            // rounding at the top end: the last tile with mass
            int lt = lastpos_t;
            for (int d = 32; d >= 1; d >>= 1) lt = max(lt, __shfl_xor(lt, d));
            if (lt < 0) lt = 0;
            const int L = lt / tpl;
            if (lane == L) {
                double acc = ex;
                for (int tt = t0; tt < lt; ++tt) acc += s_tile[tt];
                base = acc;
            }
            ts = lt;
            base = __shfl(base, L);
        }
        float tx[4], dx[4];
        const int v0 = ts * VF_TILE + lane * 4;
        ld4(w.trow, w.bf16, w.alt, V, v0, tx);
        if (useq) ld4(w.drow, w.bf16, w.ald, V, v0, dx);
        double pv[4];
        double ls = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pv[e] = useq ? fmax(0.0, walk_p(w, tx[e]) - aa * walk_q(w, dx[e])) : walk_p(w, tx[e]);
            for (int z = 0; z < nz; ++z)
                if (v0 + e == zx[z]) pv[e] = 0.0;
            ls += pv[e];
        }
        double in2 = ls;
        for (int d = 1; d < 64; d <<= 1) {
            const double o = __shfl_up(in2, d);
            if (lane >= d) in2 += o;
        }
        double run = base + (in2 - ls);
        int hit = 0x7FFFFFFF, lastpos = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int v = v0 + e;
            run += pv[e];
            if (v < V && pv[e] > 0.0) {
                if (run > thr && hit == 0x7FFFFFFF) hit = v;
                lastpos = v;
            }
        }
        hit = wave_min_i32(hit);
        int lp = lastpos;
        for (int d = 32; d >= 1; d >>= 1) lp = max(lp, __shfl_xor(lp, d));
        if (lane == 0) *s_out = hit != 0x7FFFFFFF ? hit : (lp >= 0 ? lp : 0);
    }
    __syncthreads();
    return *s_out;
}

__global__ __launch_bounds__(VF_NT) void k_verify(VerifyArgs a) {
    const ddt_tree& t = a.t;
    const ddt_flat& f = a.f;
    const int G = a.G;                                 // workgroups per request (T > 0 walk)
    const int b = blockIdx.x / G, g = blockIdx.x - (blockIdx.x / G) * G;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int P = f.P, Dp = f.Dp;
    __shared__ int s_am[MK_NT];
    __shared__ float s_M[MK_NT], s_S[MK_NT];
    __shared__ int s_fp[MK_NT], s_ft[MK_NT];
    __shared__ double s_tile[VF_MAXTILES];
    __shared__ double s_red[2 * (VF_NT / 64)];
    __shared__ double s_e2t[64];
    __shared__ int s_path[DDT_MAX_DEPTH + 2];
    __shared__ int s_ch[MK_NT];
    // T > 0 walk, per flat position i: draft slot and depth of its node, the
    // reduction statistics of the draft row it expanded, and the target and
    // draft logits of its token under its parent's rows
    __shared__ int s_wslot[MK_NT], s_wdep[MK_NT];
    __shared__ float s_wrm[MK_NT], s_wrs[MK_NT], s_wtl[MK_NT], s_wdl[MK_NT];
    // retrieval positions (point-mass proposals), and the positions of the
    // current node's rejected retrieval children (their tokens leave p)
    __shared__ int s_wret[MK_NT], s_zc[MK_NT];
    __shared__ int s_nz;
    __shared__ int s_wcnt[MK_NT / 64];
    __shared__ int s_nch, s_u, s_len, s_acc, s_next;
    __shared__ unsigned long long s_best;
    __shared__ uint64_t s_mscr[VF_NT / 64][MRG_SCR];
    __shared__ int32_t s_ret[VF_RET];
    __shared__ double s_bc[2];
    __shared__ int s_err;
    const int m = min(max(f.m[b], 0), P - 1);
    const int n = m + 1;
    const size_t fo = (size_t)b * P;
    const float T = a.temperature[b];
    if (!(T > 0.f) && g != 0) return;                  // greedy rows: one workgroup
    const int Lr = min(max(f.n_leaves[b], 0), f.L);
    const bool ret_lds = Lr * (Dp + 1) <= VF_RET;
    const bool greedy = !(T > 0.f);
    // second load trip: the candidate paths (greedy), the flat parents and tokens and
    // the first batch of argmax merges are requested before anything waits
    // (straight-line loads from clamped addresses: a load under a branch ends
    // in a register copy that waits for it)
    // (clamped to the arrays' capacities rather than to m and the leaf count,
    // so that these loads go out together with the first trip's; everything
    // past the data is masked below)
    const int32_t* ret = f.retrieve + (size_t)b * f.L * (Dp + 1);
    const int nret = greedy && ret_lds ? Lr * (Dp + 1) : 0;
    const int ret_cap = f.L * (Dp + 1);
    int32_t r_ret[VF_RET / VF_NT];
#pragma unroll
    for (int k = 0; k < VF_RET / VF_NT; ++k) {
        const int q = tid + k * VF_NT;
        r_ret[k] = ret[q < ret_cap ? q : 0];
    }
    const int tn = tid < P ? tid : 0;                  // P <= MK_NT <= VF_NT
    const int r_fp = f.parent[fo + tn], r_ft = f.token[fo + tn];
    const bool k1 = a.Kp == 1;
    constexpr int VB = 4, NWV = VF_NT / 64;           // rows per wave per batch, waves
    MergeIn1 in1[VB];
    if (k1) {
#pragma unroll
        for (int r = 0; r < VB; ++r) {
            const int i = min(wid + r * NWV, P - 1);
            merge1_issue(a.part + ((size_t)(b * P + i) * a.chunks) * rr_ps(1), a.chunks, in1[r]);
        }
    }
    // LDS staging from registers
#pragma unroll
    for (int k = 0; k < VF_RET / VF_NT; ++k) {
        const int q = tid + k * VF_NT;
        if (q < nret) s_ret[q] = r_ret[k];
    }
    if (tid < P) {
        s_fp[tid] = tid < n ? r_fp : -1;
        s_ft[tid] = tid < n ? r_ft : -1;
        if (tid >= n && g == 0) {                      // padding positions carry -1
            if (a.row_argmax) a.row_argmax[fo + tid] = -1;
            for (int k = 0; a.row_topk && k < a.k_top; ++k) a.row_topk[(fo + tid) * a.k_top + k] = -1;
        }
    }
    // merges: wave w takes rows w, w + 16, ...; argmax rows in batches of VB
    // whose loads go out together
    if (k1) {
        for (int i0 = wid; i0 < n; i0 += VB * NWV) {
            if (i0 != wid) {
#pragma unroll
                for (int r = 0; r < VB; ++r) {
                    const int i = min(i0 + r * NWV, n - 1);
                    merge1_issue(a.part + ((size_t)(b * P + i) * a.chunks) * rr_ps(1), a.chunks, in1[r]);
                }
            }
#pragma unroll
            for (int r = 0; r < VB; ++r) {
                const int i = i0 + r * NWV;
                if (i >= n) break;
                float M, Sp;
                const uint64_t mine = merge1_finish(in1[r], a.chunks, M, Sp, T > 0.f);
                if (lane == 0) {
                    const int am = vkey_id(mine);
                    s_am[i] = am; s_M[i] = M; s_S[i] = Sp;
                    if (a.row_argmax && g == 0) a.row_argmax[fo + i] = am;
                    if (a.row_topk && g == 0 && a.k_top > 0) a.row_topk[(fo + i) * a.k_top] = am;
                }
            }
        }
    } else {
        for (int i = wid; i < n; i += NWV) {
            float M, Sp;
            const uint32_t* p = a.part + ((size_t)(b * P + i) * a.chunks) * rr_ps(a.Kp);
            const uint64_t mine = merge_row_wave(p, a.chunks, a.Kp, M, Sp, s_mscr[wid]);
            const int am = __shfl(vkey_id(mine), 0);
            if (lane == 0) {
                s_am[i] = am; s_M[i] = M; s_S[i] = Sp;
                if (a.row_argmax && g == 0) a.row_argmax[fo + i] = am;
            }
            if (a.row_topk && g == 0 && lane < a.k_top) a.row_topk[(fo + i) * a.k_top + lane] = vkey_id(mine);
        }
    }
    if (tid == 0) s_best = 0ull;
    __syncthreads();
    int32_t* apath = a.accept_path + (size_t)b * (Dp + 1);

    if (!(T > 0.f)) {
        // greedy: longest matching prefix over the candidate paths
        const int L = Lr;
        const int32_t* ret = f.retrieve + (size_t)b * f.L * (Dp + 1);
        unsigned long long best = 0ull;
        for (int l = tid; l < L; l += VF_NT) {
            const int32_t* path = ret_lds ? s_ret + l * (Dp + 1) : ret + (size_t)l * (Dp + 1);
            int len = 0;
            for (int s = 1; s <= Dp; ++s) {
                const int j = path[s], pj = path[s - 1];
                if (j < 0 || j >= n || pj < 0 || pj >= n) break;
                if (s_ft[j] == s_am[pj]) len = s;
                else break;
            }
            const unsigned long long k = ((unsigned long long)len << 32) | (unsigned)(0x7FFFFFFF - l);
            best = k > best ? k : best;
        }
        best = wave_max_u64(best);
        if (lane == 0) atomicMax(&s_best, best);
        __syncthreads();
        if (tid == 0) {
            if (s_best == 0ull) {                      // no candidate path: root only
                for (int s = 0; s <= Dp; ++s) apath[s] = s == 0 ? 0 : -1;
                a.accept_len[b] = 0;
                a.next_token[b] = s_am[0];
            } else {
                const int len = (int)(s_best >> 32);
                const int l = 0x7FFFFFFF - (int)(s_best & 0xFFFFFFFFu);
                const int32_t* path = ret_lds ? s_ret + l * (Dp + 1) : ret + (size_t)l * (Dp + 1);
                for (int s = 0; s <= Dp; ++s) apath[s] = s <= len ? path[s] : -1;
                a.accept_len[b] = len;
                a.next_token[b] = s_am[path[len]];
            }
        }
        return;
    }

    // T > 0: sibling walk with residual resampling
    const double kT = (double)DDT_LOG2E_D / (double)T;
    const float* Ub = a.U + fo * 2;
    const int ntiles = (a.V + VF_TILE - 1) / VF_TILE;
    RowSync rs;
    rs.buf = t.walk_buf + (size_t)b * DDT_WALK_STRIDE;
    rs.tiles = rs.buf + 4 * 32;
    rs.cnt = t.walk_sync + 2 * (size_t)b;
    rs.limit = a.spin_limit;
    rs.G = G; rs.g = g; rs.k = 0;
    {
        const int tpw = (ntiles + G - 1) / G;
        rs.t_lo = min(g * tpw, ntiles);
        rs.t_hi = min(rs.t_lo + tpw, ntiles);
        rs.lo = rs.t_lo * VF_TILE;
        rs.hi = min(a.V, rs.t_hi * VF_TILE);
    }
    // After a pass whose wait ran out (s_err set): workgroup 0 leaves the
    // exchange, takes the whole vocabulary and asks for the pass again
    // (true); any other workgroup leaves the walk (false, s_err stays set and
    // it never counts itself in again).  Alone, no wait can run out.
    auto alone_again = [&]() -> bool {
        if (!s_err || g != 0) return false;
        rs.G = 1; rs.t_lo = 0; rs.t_hi = ntiles; rs.lo = 0; rs.hi = a.V;
        __syncthreads();                               // every thread has read s_err
        if (tid == 0) s_err = 0;
        __syncthreads();
        return true;
    };
    if (tid == 0) { s_u = 0; s_len = 0; s_path[0] = 0; s_err = 0; s_next = 0; }
    if (tid < 64) s_e2t[tid] = exp2((double)tid / 64.0);
    // every position's draft slot, depth and row statistics (a chain of three
    // loads, once), then its logits under its parent's rows (one more round):
    // the walk's steps read LDS only
    const size_t es = a.bf16 ? 2 : 4;
    const bool use_draft = a.drf != nullptr && !a.point;
    auto drow_of = [&](int slot, int dep) -> const char* {
        const int64_t doff = (int64_t)dep * a.dl + (int64_t)b * a.ds0 + (int64_t)slot * a.ds1;
        return (const char*)a.drf + (size_t)doff * es;
    };
    if (tid < n) {
        const int node = f.node[fo + tid];
        const bool ok = node >= 0 && node < t.cap;
        const int nc = ok ? node : 0;
        int slot = t.eslot[(size_t)b * t.cap + nc];
        const int dep = t.depth[(size_t)b * t.cap + nc];
        if (!ok || !use_draft || dep < 0 || dep >= t.D_max || slot >= t.R_max) slot = -1;
        const size_t ri = ((size_t)b * t.D_max + (slot >= 0 ? dep : 0)) * t.R_max + (slot >= 0 ? slot : 0);
        const float rm = t.rmax[ri], rsv = t.rsp[ri];
        const uint64_t key = t.key[(size_t)b * t.cap + nc];
        s_wret[tid] = ok && ((key >> KEY_SRC_SHIFT) & 1ull) ? 1 : 0;
        s_wslot[tid] = slot;
        s_wdep[tid] = ok ? dep : 0;
        s_wrm[tid] = rm;
        s_wrs[tid] = rsv;
    }
    __syncthreads();
    if (tid < n) {
        const int pa = min(max(s_fp[tid], 0), n - 1);
        const int x = min(max(s_ft[tid], 0), a.V - 1);
        const char* trow = (const char*)a.tgt + (size_t)(b * a.ts0 + pa * a.ts1) * es;
        const int ps = s_wslot[pa];
        const char* drow = ps >= 0 ? drow_of(ps, s_wdep[pa]) : trow;
        s_wtl[tid] = ld_logit(trow, a.bf16 != 0, x);
        s_wdl[tid] = ld_logit(drow, a.bf16 != 0, x);
    }
    __syncthreads();
    while (!s_err) {
        const int u = s_u;
        // children of u in flat order: ballots over the positions, then each
        // wave's offset from the counts of the waves before it
        {
            const bool is_ch = tid < n && tid > u && s_fp[tid] == u;
            const uint64_t bm = __ballot(is_ch);
            if (lane == 0 && wid < MK_NT / 64) s_wcnt[wid] = __popcll(bm);
            __syncthreads();
            if (is_ch) {
                int off = 0;
                for (int w2 = 0; w2 < wid; ++w2) off += s_wcnt[w2];
                s_ch[off + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u))] = tid;
            }
            if (tid == 0) {
                int c = 0;
                for (int w2 = 0; w2 < MK_NT / 64; ++w2) c += s_wcnt[w2];
                s_nch = c;
            }
        }
        __syncthreads();
        const int nch = s_nch;
        const int uslot = s_wslot[u];
        const int udep = s_wdep[u];
        // u's draft row proposes its draft children; its retrieval children
        // (and every child in the point mode, or of a node without a draft
        // row) get point-mass proposals q = delta_x: accepted with
        // probability p_k(x), and a rejection removes x from the residual.
        // Draft children come first in flat order, so the excluded tokens
        // never meet a draft pass.
        const bool has_q = nch > 0 && uslot >= 0;
        WalkRows w;
        w.tab = s_e2t;
        w.bf16 = a.bf16 != 0;
        w.trow = (const char*)a.tgt + (size_t)(b * a.ts0 + u * a.ts1) * es;
        w.drow = has_q ? drow_of(uslot, udep) : w.trow;
        const uintptr_t amask = w.bf16 ? 7u : 15u;     // 4-element vector loads
        w.alt = (((uintptr_t)w.trow) & amask) == 0;
        w.ald = (((uintptr_t)w.drow) & amask) == 0;
        w.kT = kT;
        w.Mt = s_M[u];
        w.Md = has_q ? (double)s_wrm[u] : w.Mt;
        w.lzt = 0.0;
        w.lzd = 0.0;
        bool tiles_ready = false;                       // s_tile holds the emission weights
        bool tiles_unnorm = false;                      // ... as unnormalised p (lzt = 0)
        double tiles_tot = 0.0;
        // Normalisers.  The accept tests at T = 1 use the rows' own statistics
        // (the reduction's fp32 sigma', relative error ~1e-6, well inside the
        // accept-test margin); the fp64 sums are taken only once a rejection
        // needs a residual.  With point-mass children only, that one pass over
        // the target row also leaves the emission weights per tile.
        bool zexact = false;
        auto exact_norms = [&]() {
            if (has_q) {
                w.lzt = 0.0;                           // sums of the unnormalised rows
                w.lzd = 0.0;
                double Zt, Zd;
                do walk_norms(w, rs, s_red, s_bc, &s_err, a.V, Zt, Zd); while (alone_again());
                w.lzt = log2(Zt);
                w.lzd = log2(Zd);
            } else {
                WalkRows w0 = w;
                w0.lzt = 0.0;
                double Z;
                do Z = walk_tiles(w0, rs, s_red, s_bc, &s_err, a.V, false, 0.0, s_tile);
                while (alone_again());
                w.lzt = log2(Z);                       // Z >= 1: the maximum weighs 1
                tiles_ready = true;
                tiles_unnorm = true;
                tiles_tot = Z;
            }
            zexact = true;
        };
        if (nch > 0) {
            if (T == 1.f) {
                w.lzt = log2(1.0 + (double)s_S[u]);
                w.lzd = has_q ? log2(1.0 + (double)s_wrs[u]) : 0.0;
            } else {
                exact_norms();
            }
        }
        double ra = 0.0, rb = 1.0;                      // residual p_k = max(0, p - ra q) / rb, minus excluded tokens
        int accepted = -1;
        if (tid == 0) s_nz = 0;
        __syncthreads();
        // the unnormalised residual weight of child c's token
        auto wres = [&](int c) {
            const double px = walk_p(w, s_wtl[c]);
            const double qx = has_q ? walk_q(w, s_wdl[c]) : 0.0;
            double wx = fmax(0.0, px - ra * qx);
            for (int z = 0; z < s_nz; ++z)
                if (s_ft[s_zc[z]] == s_ft[c]) wx = 0.0;
            return wx;
        };
        for (int ci = 0; ci < nch && !s_err; ++ci) {
            const int c = s_ch[ci];
            if (s_wret[c] || !has_q) {
                if (tid == 0) s_acc = ((double)Ub[2 * c] < wres(c) / rb) ? 1 : 0;
                __syncthreads();
                if (s_acc) { accepted = c; break; }
                if (!zexact) {
                    exact_norms();
                    if (s_err) break;
                }
                const double wx = wres(c);              // every thread, exact normalisers
                __syncthreads();                        // s_nz read by all before it grows
                // a token already removed (a duplicate sibling) weighs 0 and is
                // not listed again; an all-zero residual keeps p as it was
                if (wx > 0.0 && rb - wx > 0.0) {
                    rb -= wx;
                    if (tid == 0) s_zc[s_nz++] = c;
                }
                __syncthreads();
                continue;
            }
            if (tid == 0) {
                const double px = walk_p(w, s_wtl[c]);
                const double qx = walk_q(w, s_wdl[c]);
                const double pk = fmax(0.0, px - ra * qx) / rb;
                const double ratio = qx > 0.0 ? pk / qx : INFINITY;
                s_acc = ((double)Ub[2 * c] < ratio) ? 1 : 0;
            }
            __syncthreads();
            if (s_acc) { accepted = c; break; }
            if (!zexact) {
                exact_norms();
                if (s_err) break;
            }
            // rejection: b' = F(a + b); after the last sibling the same
            // pass leaves the emission weights per tile
            const double an = ra + rb;
            double F;
            if (ci == nch - 1) {
                do F = walk_tiles(w, rs, s_red, s_bc, &s_err, a.V, true, an, s_tile);
                while (alone_again());
                tiles_ready = F > 0.0;
                tiles_unnorm = false;
                tiles_tot = F;
            } else {
                do F = walk_pass<true>(w, rs, s_red, s_bc, &s_err, a.V, [&](float tv, float dv) {
                    return fmax(0.0, walk_p(w, tv) - an * walk_q(w, dv));
                });
                while (alone_again());
            }
            if (s_err) break;
            if (F > 0.0) { ra = an; rb = F; }
        }
        if (s_err) break;
        if (accepted >= 0) {
            if (tid == 0) { s_u = accepted; s_path[++s_len] = accepted; }
            __syncthreads();
            continue;
        }
        // emission from the current residual by inverse CDF with U[u][1] over
        // the unnormalised weights max(0, p - a q) (p at a leaf); the threshold
        // scales with their total
        if (!tiles_ready) {
            do tiles_tot = walk_tiles(w, rs, s_red, s_bc, &s_err, a.V, has_q, ra, s_tile);
            while (alone_again());
            tiles_unnorm = false;
        }
        if (s_err) break;
        if (g == 0) {
            WalkRows we = w;                           // the units the tiles were summed in
            if (tiles_unnorm) we.lzt = 0.0;
            if (rs.G > 1)                              // the other workgroups' tiles
                for (int q = tid; q < ntiles; q += VF_NT)
                    s_tile[q] = __hip_atomic_load(rs.tiles + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            // rejected point-mass tokens carry no weight: out of their tiles'
            // sums and the total here, out of the element scan in walk_pick
            const int nz = s_nz;
            if (tid == 0) {
                for (int z = 0; z < nz; ++z) {
                    const int c = s_zc[z];
                    const double wx = fmax(0.0, walk_p(we, s_wtl[c]) - ra * (has_q ? walk_q(we, s_wdl[c]) : 0.0));
                    const int tt = min(max(s_ft[c], 0), a.V - 1) / VF_TILE;
                    s_tile[tt] = fmax(0.0, s_tile[tt] - wx);
                    s_zc[z] = s_ft[c];                 // from here on: the excluded tokens
                }
            }
            __syncthreads();
            if (nz > 0) {
                double tot = 0.0;
                for (int q = 0; q < ntiles; ++q) tot += s_tile[q];
                tiles_tot = tot;
            }
            walk_pick(we, a.V, has_q, ra, (double)Ub[2 * u + 1], tiles_tot, s_tile, &s_next, s_zc, nz);
        }
        break;
    }
    // workgroup 0 never ends with s_err set (a wait that ran out sent it on
    // alone), so every request gets its outcome
    if (g == 0 && tid == 0) {
        const int len = s_len;
        for (int s2 = 0; s2 <= Dp; ++s2) apath[s2] = s2 <= len ? s_path[s2] : -1;
        a.accept_len[b] = len;
        a.next_token[b] = s_next;
    }
    if (G > 1 && tid == 0) {
        // the last workgroup of the request to leave returns the counters to 0
        __threadfence();
        if (atomicAdd(rs.cnt + 1, 1u) == (uint32_t)G - 1) {
            atomicExch(rs.cnt, 0u);
            atomicExch(rs.cnt + 1, 0u);
        }
    }
}

// ---------------------------------------------------------------------------
// successor-matrix refresh
// ---------------------------------------------------------------------------
//
// Graft review step 3: every verified token's row of M is replaced by the
// top-k of the target's next-token distribution at that position; the later
// flat position wins on duplicate tokens (reading).  With a shared matrix
// (M_bstride = 0) one workgroup handles the whole batch so the winner is the
// last (row, position) pair.

struct UpdateArgs {
    ddt_flat f;
    int32_t* M;
    int64_t M_bstride;
    int V, k_succ, k_top, B, shared;
    const int32_t* row_topk;     // [B][P][k_top], or NULL to merge partials
    const uint32_t* part;
    int chunks, Kp;
};

#define UP_NT 256

__global__ __launch_bounds__(UP_NT) void k_succ_update(UpdateArgs a) {
    const ddt_flat& f = a.f;
    const int P = f.P;
    const int b0 = a.shared ? 0 : blockIdx.x, b1 = a.shared ? a.B : blockIdx.x + 1;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    __shared__ uint64_t s_mscr[UP_NT / 64][MRG_SCR];
    for (int b = b0; b < b1; ++b) {
        const int m = min(max(f.m[b], 0), P - 1);
        const size_t fo = (size_t)b * P;
        int32_t* Mb = a.M + (size_t)b * a.M_bstride;
        if (a.row_topk != nullptr) {
            for (int i = 1 + tid; i <= m; i += UP_NT) {
                const int tk = f.token[fo + i];
                if (tk < 0 || tk >= a.V) continue;
                bool last = true;
                for (int j = i + 1; j <= m && last; ++j) last = f.token[fo + j] != tk;
                for (int bb = b + 1; a.shared && bb < a.B && last; ++bb) {
                    const int mm = min(max(f.m[bb], 0), P - 1);
                    for (int j = 1; j <= mm && last; ++j) last = f.token[(size_t)bb * P + j] != tk;
                }
                if (!last) continue;
                for (int c = 0; c < a.k_succ; ++c)
                    Mb[(size_t)tk * a.k_succ + c] = a.row_topk[(fo + i) * a.k_top + c];
            }
        } else {
            for (int i = 1 + wid; i <= m; i += UP_NT / 64) {
                const int tk = f.token[fo + i];
                if (tk < 0 || tk >= a.V) continue;
                bool last = true;
                for (int j = i + 1; j <= m && last; ++j) last = f.token[fo + j] != tk;
                for (int bb = b + 1; a.shared && bb < a.B && last; ++bb) {
                    const int mm = min(max(f.m[bb], 0), P - 1);
                    for (int j = 1; j <= mm && last; ++j) last = f.token[(size_t)bb * P + j] != tk;
                }
                float M, Sp;
                const uint32_t* p = a.part + ((size_t)(b * P + i) * a.chunks) * rr_ps(a.Kp);
                const uint64_t mine = merge_row_wave(p, a.chunks, a.Kp, M, Sp, s_mscr[wid]);
                if (last && lane < a.k_succ) Mb[(size_t)tk * a.k_succ + lane] = vkey_id(mine);
            }
        }
        if (a.shared) __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// standalone row top-k: merge partials into ids / log confidences
// ---------------------------------------------------------------------------

struct RowFinishArgs {
    const uint32_t* part;
    int rows, chunks, K;
    int32_t* ids;
    float* logc;
    float* rmax;
    float* rsp;
};

__global__ __launch_bounds__(256) void k_row_finish(RowFinishArgs a) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows) return;
    float M, Sp;
    const uint32_t* p = a.part + (size_t)row * a.chunks * rr_ps(a.K);
    __shared__ uint64_t s_mscr[4][MRG_SCR];
    const uint64_t mine = merge_row_wave(p, a.chunks, a.K, M, Sp, s_mscr[threadIdx.x >> 6]);
    if (lane < a.K) {
        if (a.ids) a.ids[(size_t)row * a.K + lane] = vkey_id(mine);
        if (a.logc)
            a.logc[(size_t)row * a.K + lane] = mine ? (vkey_val(mine) - M) - log1pf(Sp) : -INFINITY;
    }
    if (lane == 0) {
        if (a.rmax) a.rmax[row] = M;
        if (a.rsp) a.rsp[row] = Sp;
    }
}
