// One draft layer in one kernel: vocabulary reduction, row merge, children,
// frontier and CAST's batch rule.
//
// EAGLE-2 explainer, expansion section: every expanded node gets its draft
// row's top-K_n tokens as children, value(child) = value(parent) x
// confidence(child), kept here as S_child = S_parent + log c in fp32 (Graft
// review step 1, S_{d,j} recursion); the next frontier is the best K_e of the
// newest layer by value (ties: canonical key).  Graft review step 1: at a
// checkpoint depth a request stops unless exp(max S of the layer) > tau.
// CAST notes, key designs 2 and 3: the width and depth rule over the whole
// batch.
//
// Grid: one 256-thread workgroup per (request b, frontier slot j, vocabulary
// chunk g); workgroups of slots past the request's frontier width leave at
// once.  Launches of many rows, which fill the device many times over, run
// the plain reduction (k_row_partial) and then k_expand_finish, one
// 1024-thread workgroup per request whose waves merge the request's rows in
// parallel (a chunk workgroup that waits for its ticket holds a slot the next
// chunk could use, and the merges and frontier then need no coherent
// handoffs).  Nothing waits: each stage is run by the last workgroup to arrive on
// a device-scope counter ("ticket"), which then resets it.
//   A. every workgroup reduces its chunk to a partial record;
//   B. the last chunk of row (b, j) merges the row's partials (one wave)
//      and writes its K_n children into the tree, and their sort keys (S,
//      canonical order) over the row's partials, which are no longer needed;
//   C. the last row of request b ranks the layer's sort keys of b into the
//      next frontier and closes b's layer (node count, frontier width,
//      Graft gate); a request with one row skips this ticket and keeps the
//      sort keys in LDS;
//   D. with CAST, the last request runs the batch rule.
// Every value one workgroup hands to another within the launch (partial
// records, the new nodes' values, the frontier values and counts, the
// frontier width) is written with device-coherent stores and read with
// device-coherent loads (agent-scope atomic accesses, which bypass the
// caches that are not coherent across the chip), so no cache write-back or
// invalidation is needed.  Before counting itself in, every wave waits for
// its stores to complete (a workgroup barrier alone does not wait for other
// waves' stores).  Values read only by later kernels use plain stores; no
// address is written by two workgroups of one launch with plain stores.
#pragma once
#include "ddt_device.hpp"
#include "ddt_rowreduce.hpp"
#include "ddt_tree_kernels.hpp"

struct LayerArgs {
    ddt_tree t;
    ddt_cast c;
    const void* base;            // logits row (b, j) at base + b*s0 + j*s1 elements
    int64_t s0, s1;
    uint32_t* part;              // [B*R][groups][2 + 2 K_n] chunk partials
    const int32_t* root_tok;     // [B], layer 1
    int V, groups, K_n, K_e, R, layer;
    int ck, kd_ck, K_max, gate_on, cast_on;   // ck: this layer is a Graft checkpoint
    float tau;
};

// Every wave waits for its device-coherent stores to complete, then thread 0
// counts the workgroup in on *ctr.  Returns true, in every thread, for the
// last of n arrivals, which resets the counter; its later loads are issued
// after the count, so its coherent loads see every arrival's stores.
__device__ __forceinline__ bool ticket_last(uint32_t* ctr, uint32_t n, int& s_flag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = atomicAdd(ctr, 1u);
        s_flag = old == n - 1u;
        if (s_flag) atomicExch(ctr, 0u);
    }
    __syncthreads();
    return s_flag != 0;
}

__device__ __forceinline__ void st_coh_f32(float* p, float v) { rr_st32((uint32_t*)p, __float_as_uint(v)); }
__device__ __forceinline__ void st_coh_i32(int32_t* p, int32_t v) { rr_st32((uint32_t*)p, (uint32_t)v); }
__device__ __forceinline__ float ld_coh_f32(const float* p) { return __uint_as_float(rr_ld32<true>((const uint32_t*)p)); }
__device__ __forceinline__ int32_t ld_coh_i32(const int32_t* p) { return (int32_t)rr_ld32<true>((const uint32_t*)p); }

// Dynamic LDS of the layer kernel: the stages run one after another in a
// workgroup, so they share one block sized for the largest.
__host__ __device__ __forceinline__ size_t layer_lds_c(int R_max, int K_n) {
    return ((size_t)R_max * K_n + R_max) * 8;                      // sort keys, parents' keys
}
__host__ __device__ __forceinline__ size_t layer_lds_d(int B, int R_max, int M) {
    (void)B; (void)M;
    return 16 * 8 + (size_t)R_max * 8;
}

// Request b's next frontier from the layer's sort keys s_sk[count] (nrows
// rows of K_n, row-major) and the parents' keys s_pk[nrows] (LDS): rank <
// R_max makes a frontier record and rank 0 closes b's layer (node count,
// frontier width, Graft gate).  The values stage D reads go out
// device-coherent.  Every thread of the workgroup calls it.
//
// One row's children come out of the merge in (value desc, id asc) order
// and S = S_parent + log c keeps that order, so the sort keys of a request
// with one row usually ascend already: then a key's rank is its position
// (each wave checks the order on its own, over the same LDS words, so every
// wave decides alike).  Otherwise each rank is counted over all keys by SL
// lanes.  (A bound from each row's first keys, then ranks among the keys
// below it, measured slower in the 1024-thread finish at 256 keys: its
// sampling and two more barriers cost more than the shorter counting saved.)
template <int NT>
__device__ void layer_frontier(const LayerArgs& a, int b, int base, int count, const uint64_t* s_sk,
                               const uint64_t* s_pk, int nrows) {
    const ddt_tree& t = a.t;
    const int tid = threadIdx.x, lane = tid & (DDT_WAVE - 1), Rm = t.R_max, Kn = a.K_n,
              layer = a.layer, du = layer - 1;
    int32_t* fr = t.frontier + (size_t)b * Rm;
    float* frS = t.front_S + (size_t)b * Rm;
    uint64_t* frK = t.front_key + (size_t)b * Rm;
    auto emit = [&](int q, uint64_t sk, int r) {
        const float Sv = unord_f32(~(uint32_t)(sk >> 32));
        const int jj = q / Kn;
        fr[r] = base + q; st_coh_f32(frS + r, Sv);
        frK[r] = key_child(layer == 1 ? 0ull : s_pk[jj], du, q - jj * Kn, 0);
        if (r == 0) {
            st_coh_i32(t.n_nodes + b, base + count);
            st_coh_i32(t.layer_base + b, base);
            int nf = min(a.K_e, count);
            if (layer >= t.D_max) nf = 0;
            if (layer == 1) {
                t.active[b] = 1;
                t.k_draft[b] = a.gate_on ? a.K_max : 0;
            }
            if (a.ck && !(expf(Sv) > a.tau)) {                // g_d = 1[c_d > tau_d]
                t.active[b] = 0;
                t.k_draft[b] = a.kd_ck;
                nf = 0;
            }
            st_coh_i32(t.n_front + b, nf);
        }
    };
    if (count == 0) {
        if (tid == 0) {
            if (layer == 1) { st_coh_i32(t.n_nodes + b, 1); st_coh_i32(t.layer_base + b, 1); }
            st_coh_i32(t.n_front + b, 0);
        }
        return;
    }
    // one row: each wave checks the order on its own (the same LDS words, so
    // every wave decides alike)
    if (nrows == 1 && count <= DDT_WAVE) {
        const uint64_t x = lane < count ? s_sk[lane] : 0ull, xp = lane >= 1 && lane < count ? s_sk[lane - 1] : 0ull;
        if (__ballot(lane >= 1 && lane < count && !(xp < x)) == 0ull) {
            if (tid < count && tid < Rm) emit(tid, x, tid);
            return;
        }
    }
    const int SL = split_lanes(count, NT);
    const int lg = __ffs(SL) - 1;
    for (int cb = 0; cb < count; cb += NT >> lg) {
        const int q = cb + (tid >> lg), part = tid & (SL - 1);
        uint64_t sk = 0ull;
        int r = 0;
        if (q < count) {
            sk = s_sk[q];
#pragma unroll 4
            for (int p = part; p < count; p += SL) r += s_sk[p] < sk ? 1 : 0;
        }
        r = group_sum(r, SL);
        if (part == 0 && q < count && r < Rm) emit(q, sk, r);
    }
}

// CAST's batch rule (key designs 2 and 3) in the last request of the layer;
// with CAST every request has the same frontier width, so all B take part in
// every layer that runs.  The inputs that do not depend on this layer's
// frontiers (state, the layer's C1, cost-table entries) are staged in
// `region` (LDS) beforehand by threads i0, i0 + stride, ... (cast_stage);
// cast_finish then takes the batch ticket and, in the last request, wave 0
// reads the frontiers (lane k the k-th node of every request) and decides.
__device__ __forceinline__ CastView cast_view(unsigned char* region, int R_max) {
    (void)R_max;
    CastView L;
    L.st = (double*)region;                                      // [16] state, C1, 1/B
    L.c = L.st + 16;                                             // [R_max] width costs
    return L;
}

// The state (layer 1 starts it: FIFO {1}, length 1, no previous u_n,
// context 0), the layer's C1, 1/B, and the width costs of this layer's
// context row, c_k = S_D[sel(ctx)][k] / S_T[sel(ctx)][1] (the context is the
// previous layer's state; each cost thread reads it itself).
__device__ void cast_stage(const LayerArgs& a, unsigned char* region, int i0, int stride) {
    const ddt_tree& t = a.t;
    const ddt_cast& cp = a.c;
    const int Rm = t.R_max, layer = a.layer, N = cp.N;
    const CastView L = cast_view(region, Rm);
    for (int q = i0; q < 16 + Rm; q += stride) {
        if (q < 12) {
            L.st[q] = q == 11 ? (double)cp.C1[layer - 1]
                    : layer > 1 ? t.cast_state[q] : q == 0 ? 1.0 : q == 8 ? 1.0 : q == 9 ? -1.0 : 0.0;
        } else if (q == 12) {
            L.st[12] = 1.0 / (double)t.B;
        } else if (q >= 16) {
            const int k = q - 16;
            const int ctx = layer > 1 ? (int)t.cast_state[10] : 0;
            const float* rowp = cp.S_D + (size_t)cast_sel_row(ctx, cp.L, cp.M) * (N + 1);
            const float* rowt = cp.S_T + (size_t)cast_sel_row(ctx, cp.L, cp.M) * (N + 1);
            L.c[k] = k < N ? (double)rowp[k + 1] / (double)rowt[1] : 0.0;
        }
    }
}

// The same inputs for the one-kernel layer, requested early from registers:
// thread q < 12 the state entry or C1 at the kernel's start; thread
// CAST_CT + k (wave 1, idle while wave 0 merges) the context at the start
// and cost k of its row once the row's merge begins, so that stage D finds
// them in registers instead of waiting on two dependent loads.
#define CAST_CT 64
static_assert(CAST_CT + DDT_MAX_FRONT <= RR_NT, "cost threads inside the workgroup");
struct CastPre {
    double v;         // state entry / C1 (q < 12)
    int ctx;          // context (cost threads)
    float num, den;   // S_D[row][k + 1], S_T[row][1] (cost threads)
};

__device__ __forceinline__ void cast_prefetch(const LayerArgs& a, CastPre& p) {
    const ddt_tree& t = a.t;
    const int q = threadIdx.x, layer = a.layer;
    p.v = 0.0; p.ctx = 0; p.num = 0.f; p.den = 1.f;
    if (q < 12) {
        p.v = q == 11 ? (double)a.c.C1[layer - 1]
            : layer > 1 ? t.cast_state[q] : q == 0 ? 1.0 : q == 8 ? 1.0 : q == 9 ? -1.0 : 0.0;
    } else if (q >= CAST_CT && q < CAST_CT + t.R_max && layer > 1) {
        p.ctx = (int)t.cast_state[10];
    }
}

__device__ __forceinline__ void cast_cost_loads(const LayerArgs& a, CastPre& p) {
    const ddt_cast& cp = a.c;
    const int k = (int)threadIdx.x - CAST_CT, N = cp.N;
    if (k >= 0 && k < a.t.R_max) {
        const size_t row = (size_t)cast_sel_row(p.ctx, cp.L, cp.M) * (N + 1);
        p.num = k < N ? cp.S_D[row + k + 1] : 0.f;
        p.den = cp.S_T[row + 1];
    }
}

// cast_stage from the prefetched registers (every thread of the workgroup)
__device__ __forceinline__ void cast_stage_pre(const LayerArgs& a, unsigned char* region, const CastPre& p) {
    const CastView L = cast_view(region, a.t.R_max);
    const int q = threadIdx.x, k = q - CAST_CT;
    if (q < 12) L.st[q] = p.v;
    else if (q == 12) L.st[12] = 1.0 / (double)a.t.B;
    else if (k >= 0 && k < a.t.R_max) L.c[k] = k < a.c.N ? (double)p.num / (double)p.den : 0.0;
}

template <int NT>
__device__ void cast_finish(const LayerArgs& a, unsigned char* region, int& s_flag) {
    const ddt_tree& t = a.t;
    const int tid = threadIdx.x, lane = tid & (DDT_WAVE - 1), Rm = t.R_max, B = t.B;
    const CastView L = cast_view(region, Rm);
    if (!ticket_last(t.ticket, (uint32_t)B, s_flag)) return;
    if (tid >= DDT_WAVE) return;                                 // wave 0 decides
    // every request's node count and this lane's column of frontier values,
    // requested together (straight-line loads from clamped addresses)
    const int lb = lane < B ? lane : 0, kl = lane < Rm ? lane : 0;
    const int nn = ld_coh_i32(t.n_nodes + lb), lbase = ld_coh_i32(t.layer_base + lb);
    double mean = 0.0;                                           // column sum of e^S, b ascending
    for (int b0 = 0; b0 < B; b0 += 8) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = ld_coh_f32(t.front_S + (size_t)min(b0 + j, B - 1) * Rm + kl);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (b0 + j < B) mean += (double)expf(x[j]);
    }
    const int cnt = lane < B ? max(0, nn - lbase) : 0x7FFFFFFF;
    const int kcap = min(min(a.K_e, Rm), (int)wave_min_u32((uint32_t)cnt));
    cast_decide(L, t, a.c, a.layer, kcap, lane < kcap ? mean * L.st[12] : 0.0);
}

template <bool BF16, int NL>
__global__ __launch_bounds__(RR_NT) void k_expand_layer(LayerArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ int s_flag;
    const ddt_tree& t = a.t;
    const int tid = threadIdx.x, lane = tid & (DDT_WAVE - 1), wid = tid / DDT_WAVE;
    const int g = blockIdx.x % a.groups;
    const int rowg = blockIdx.x / a.groups;
    const int b = rowg / a.R, j = rowg - b * a.R;
    const int layer = a.layer, du = layer - 1;
    const int nrows = layer == 1 ? 1 : min(max(t.n_front[b], 0), a.R);
    if (j >= nrows) return;                                       // block-uniform
    const int Kn = a.K_n, cap = t.cap, Rm = t.R_max;
    const int PS = rr_ps(Kn);
    // the row's parent (frontier slot j of the previous layer; the root at
    // layer 1) and the request's node count, requested now so that they have
    // arrived by stage B (scalar loads; the previous kernel wrote them)
    const int jf = layer == 1 ? 0 : j;
    const int u0 = t.frontier[(size_t)b * Rm + jf];
    const float pS0 = t.front_S[(size_t)b * Rm + jf];
    const uint64_t pk0 = t.front_key[(size_t)b * Rm + jf];
    const int nn0 = t.n_nodes[b];
    // wave 0: the other rows' parents' keys (the layer's key order is
    // (parent key, sibling rank))
    const uint64_t pkl = t.front_key[(size_t)b * Rm + (lane < nrows && layer > 1 ? lane : 0)];
    CastPre cpre;
    if (a.cast_on) cast_prefetch(a, cpre);

    // ---- A: this workgroup's chunk of row (b, j) ----------------------------
    const void* row = (const char*)a.base + ((int64_t)b * a.s0 + (int64_t)j * a.s1) * (BF16 ? 2 : 4);
    uint32_t* prow = a.part + (size_t)rowg * a.groups * PS;
    rr_chunk<BF16, NL>(row, a.V, g, Kn, true, prow + (size_t)g * PS, *reinterpret_cast<RRLds*>(dyn));
    if (!ticket_last(t.layer_sync + rowg, (uint32_t)a.groups, s_flag)) return;

    // ---- B: merge row (b, j), attach its children ----------------------------
    int32_t* tok = t.token + (size_t)b * cap;
    int32_t* par = t.parent + (size_t)b * cap;
    int32_t* dep = t.depth + (size_t)b * cap;
    int32_t* esl = t.eslot + (size_t)b * cap;
    uint64_t* key = t.key + (size_t)b * cap;
    float* S = t.S + (size_t)b * cap;
    float* lc = t.logc + (size_t)b * cap;
    const int base = layer == 1 ? 1 : nn0;
    const bool fits = base >= 1 && base + nrows * Kn <= cap;       // capacity guard
    if (a.cast_on) cast_cost_loads(a, cpre);
    if (wid == 0) {
        MergeIn mi;
        merge_issue<true>(prow, a.groups, Kn, mi);
        float M, Sp;
        const uint64_t mine = merge_finish<true>(mi, prow, a.groups, Kn, M, Sp, (uint64_t*)dyn, true);
        const int u = layer == 1 ? 0 : ((u0 >= 0 && u0 < base) ? u0 : 0);
        const float pS = layer == 1 ? 0.f : pS0;
        const uint64_t pk = layer == 1 ? 0ull : pk0;
        // rank of this row's parent key among the request's parents
        int prk = 0;
        for (int k = 0; k < nrows; ++k) prk += readlane_u64(pkl, k) < pk ? 1 : 0;
        if (fits) {
            if (layer == 1 && lane == 0) {
                tok[0] = a.root_tok[b]; par[0] = -1; dep[0] = 0; key[0] = 0ull;
                S[0] = 0.f; lc[0] = 0.f;
            }
            if (lane < Kn) {
                const float logc = (vkey_val(mine) - M) - log1pf(Sp);
                const float Sv = pS + logc;
                const int node = base + j * Kn + lane;
                tok[node] = vkey_id(mine); par[node] = u; dep[node] = du + 1; esl[node] = -1;
                S[node] = Sv; lc[node] = logc; key[node] = key_child(pk, du, lane, 0);
                // sort key (~code(S), parent's key rank * K_n + r), ascending
                // = (S desc, canonical key asc) within the layer; written over
                // the row's partials, which are no longer needed, or, when the
                // row is the request's only one, kept in LDS (the merge
                // scratch there is no longer needed either)
                const uint64_t sk = ((uint64_t)~ord_f32(Sv) << 32) | (uint32_t)(prk * Kn + lane);
                if (nrows == 1) ((uint64_t*)dyn)[lane] = sk;
                else rr_st64((uint64_t*)prow + lane, sk);
            }
            if (lane == 0) {
                esl[u] = j;
                const size_t ri = ((size_t)b * t.D_max + du) * Rm + j;
                t.rmax[ri] = M;
                t.rsp[ri] = Sp;
            }
        }
    }
    // ---- C: request b's frontier ---------------------------------------------
    // (a request of one row goes on in the same workgroup: its only row's
    // sort keys are in LDS)
    uint64_t* s_sk = (uint64_t*)dyn;                             // [nrows * Kn]
    uint64_t* s_pk = s_sk + (size_t)Rm * Kn;                     // [nrows]
    const int count = fits ? nrows * Kn : 0;
    if (nrows > 1) {
        if (!ticket_last(t.layer_sync + (size_t)t.B * Rm + b, (uint32_t)nrows, s_flag)) return;
        for (int q = tid; q < count; q += RR_NT) {
            const int jj = q / Kn, r = q - jj * Kn;
            s_sk[q] = rr_ld64<true>((const uint64_t*)(a.part + (size_t)(b * a.R + jj) * a.groups * PS) + r);
        }
    }
    if (tid < nrows) s_pk[tid] = pkl;
    __syncthreads();
    layer_frontier<RR_NT>(a, b, base, count, s_sk, s_pk, nrows);
    if (!a.cast_on) return;

    // ---- D: CAST's batch rule --------------------------------------------------
    cast_stage_pre(a, dyn + layer_lds_c(Rm, Kn), cpre);
    cast_finish<RR_NT>(a, dyn + layer_lds_c(Rm, Kn), s_flag);
}

// ---------------------------------------------------------------------------
// the layer of a request after the plain reduction (launches of many rows)
// ---------------------------------------------------------------------------
#define EF_NT 1024
#define EF_NW (EF_NT / DDT_WAVE)

// Dynamic LDS of k_expand_finish: merge scratch per wave, the rows' top keys,
// the layer's sort keys, per-row statistics and parents; the CAST region
// follows (layer_lds_d).
__host__ __device__ __forceinline__ size_t finish_lds(int R_max, int K_n) {
    return (size_t)EF_NW * MRG_SCR * 8 + (size_t)R_max * K_n * 16 + (size_t)R_max * 24;
}

__global__ __launch_bounds__(EF_NT) void k_expand_finish(LayerArgs a) {
    extern __shared__ __align__(16) unsigned char dyn[];
    __shared__ int s_flag;
    const ddt_tree& t = a.t;
    const int tid = threadIdx.x, lane = tid & (DDT_WAVE - 1), wid = tid / DDT_WAVE;
    const int b = blockIdx.x;
    const int layer = a.layer, du = layer - 1;
    const int nrows = layer == 1 ? 1 : min(max(t.n_front[b], 0), a.R);
    if (nrows == 0) return;                                      // a stopped request
    const int Kn = a.K_n, cap = t.cap, Rm = t.R_max;
    const int PS = rr_ps(Kn);
    uint64_t* scr = (uint64_t*)dyn;                              // [EF_NW][MRG_SCR]
    uint64_t* s_key = scr + (size_t)EF_NW * MRG_SCR;             // [R_max * K_n]
    uint64_t* s_sk = s_key + (size_t)Rm * Kn;                    // [R_max * K_n]
    uint64_t* s_pk = s_sk + (size_t)Rm * Kn;                     // [R_max]
    float* s_M = (float*)(s_pk + Rm);
    float* s_Sp = s_M + Rm;
    float* s_pS = s_Sp + Rm;
    int* s_pn = (int*)(s_pS + Rm);
    const int base = layer == 1 ? 1 : t.n_nodes[b];
    const bool fits = base >= 1 && base + nrows * Kn <= cap;
    const int count = fits ? nrows * Kn : 0;
    if (a.cast_on) cast_stage(a, dyn + finish_lds(Rm, Kn), tid, EF_NT);
    if (tid < nrows) {
        const int u0 = t.frontier[(size_t)b * Rm + tid];
        s_pn[tid] = layer == 1 ? 0 : ((u0 >= 0 && u0 < base) ? u0 : 0);
        s_pS[tid] = layer == 1 ? 0.f : t.front_S[(size_t)b * Rm + tid];
        s_pk[tid] = layer == 1 ? 0ull : t.front_key[(size_t)b * Rm + tid];
    }
    // wave w merges rows w, w + 16 (plain loads: the previous kernel wrote the
    // partials)
    for (int jr = wid; jr < nrows; jr += EF_NW) {
        float M, Sp;
        const uint32_t* pr = a.part + (size_t)(b * a.R + jr) * a.groups * PS;
        const uint64_t mine = merge_row_wave(pr, a.groups, Kn, M, Sp, scr + (size_t)wid * MRG_SCR);
        if (lane < Kn) s_key[jr * Kn + lane] = mine;
        if (lane == 0) { s_M[jr] = M; s_Sp[jr] = Sp; }
    }
    __syncthreads();
    int32_t* tok = t.token + (size_t)b * cap;
    int32_t* par = t.parent + (size_t)b * cap;
    int32_t* dep = t.depth + (size_t)b * cap;
    int32_t* esl = t.eslot + (size_t)b * cap;
    uint64_t* key = t.key + (size_t)b * cap;
    float* S = t.S + (size_t)b * cap;
    float* lc = t.logc + (size_t)b * cap;
    if (layer == 1 && tid == 0 && fits) {
        tok[0] = a.root_tok[b]; par[0] = -1; dep[0] = 0; key[0] = 0ull; S[0] = 0.f; lc[0] = 0.f;
    }
    for (int q = tid; q < count; q += EF_NT) {
        const int jj = q / Kn, r = q - jj * Kn;
        const uint64_t kk = s_key[q];
        const float logc = (vkey_val(kk) - s_M[jj]) - log1pf(s_Sp[jj]);
        const float Sv = s_pS[jj] + logc;
        const uint64_t pk = s_pk[jj];
        const int u = s_pn[jj];
        const int node = base + q;
        tok[node] = vkey_id(kk); par[node] = u; dep[node] = du + 1; esl[node] = -1;
        S[node] = Sv; lc[node] = logc; key[node] = key_child(pk, du, r, 0);
        int prk = 0;
        for (int k = 0; k < nrows; ++k) prk += s_pk[k] < pk ? 1 : 0;
        s_sk[q] = ((uint64_t)~ord_f32(Sv) << 32) | (uint32_t)(prk * Kn + r);
        if (r == 0) {
            esl[u] = jj;
            const size_t ri = ((size_t)b * t.D_max + du) * Rm + jj;
            t.rmax[ri] = s_M[jj];
            t.rsp[ri] = s_Sp[jj];
        }
    }
    __syncthreads();
    layer_frontier<EF_NT>(a, b, base, count, s_sk, s_pk, nrows);
    if (!a.cast_on) return;
    cast_finish<EF_NT>(a, dyn + finish_lds(Rm, Kn), s_flag);
}
