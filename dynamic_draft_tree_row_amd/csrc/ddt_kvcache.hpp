// Paged KV cache: committing the accepted path, sharing and release.  The
// candidates' KV is the round's contiguous tree buffer; after the verify, the
// accepted tokens' KV is appended to each request's block-paged context and
// the rest is simply not copied (EAGLE-2 explainer, engineering difficulty
// two, and the decode-step flow's commit / discard steps).
//
// The bookkeeping of a commit (which blocks each request needs, admission
// while the free stack lasts, pops, copy-on-write of a shared partial block,
// holder counts, pushes of blocks left without a holder) is one workgroup of
// 1024 threads, one request per thread, with two block-wide scans; it writes
// a 4-int plan per request.  The data movement is then one workgroup per
// request (16-byte copies).  Fork and release are one workgroup each and take
// their pairs / requests in order, so every outcome is deterministic.
//
// Every block id read from the caller's arrays is range-checked before it
// indexes the pool, the holder counts or the free stack, so a state that
// breaks the documented invariants cannot send an access out of bounds (its
// outcome is then unspecified).
#pragma once
#include "ddt_device.hpp"

#define KV_NT 1024              // bookkeeping threads (one per request)
#define KV_MAXB 1024            // requests per cache
#define KV_MAXBLK 4096          // blocks per table row
#define KV_CT 256               // copy threads per workgroup
#define KV_SPLIT 4              // copy workgroups per request
#define KV_STAGE 4096           // top entries of the free stack staged in LDS

struct KvCache {
    uint16_t* k;                // bf16 [n_blocks][block][Hkv][D]
    uint16_t* v;
    int32_t* table;             // [B][max_blocks]
    int32_t* len;               // [B]
    int32_t* ref;               // [n_blocks]
    int32_t* free_ids;          // [n_blocks]
    int32_t* n_free;            // [1]
    int32_t* plan;              // [B][4]: first token, tokens, copied block, its copy
    int B, max_blocks, n_blocks, block, Hkv, D;
};

struct KvCommitArgs {
    KvCache c;
    const int32_t* accept_len;  // [B]
    const int32_t* accept_path; // [B][Dp+1]
    int Dp;
    const uint16_t* kt;         // bf16 [B][P][Hkv][D]
    const uint16_t* vt;
    int P;
    int32_t* status;            // [B]
};

struct KvForkArgs {
    KvCache c;
    const int32_t* src;
    const int32_t* dst;
    int n;
    int32_t* status;
};

struct KvReleaseArgs {
    KvCache c;
    const int32_t* req;
    int n;
};

// inclusive sum over the 1024 threads of the workgroup (all must call it)
__device__ __forceinline__ int kv_block_scan(int v, int* s_w) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d);
        if (lane >= d) v += t;
    }
    if (lane == 63) s_w[w] = v;
    __syncthreads();
    if (w == 0) {
        int x = lane < KV_NT / 64 ? s_w[lane] : 0;
#pragma unroll
        for (int d = 1; d < KV_NT / 64; d <<= 1) {
            const int t = __shfl_up(x, d);
            if (lane >= d) x += t;
        }
        if (lane < KV_NT / 64) s_w[lane] = x;
    }
    __syncthreads();
    const int r = v + (w > 0 ? s_w[w - 1] : 0);
    __syncthreads();
    return r;
}

// bookkeeping of a commit: thread b plans request b.  Its loads come in three
// rounds: the free count with each request's own inputs, then the top of the
// free stack with the tail block's id, then that block's holder count.
__global__ __launch_bounds__(KV_NT) void k_kv_plan(KvCommitArgs a) {
    __shared__ int s_w[KV_NT / 64];
    __shared__ int s_x[KV_MAXB];                        // old block of each admitted copier, else -1
    __shared__ int s_need[KV_NT];                       // blocks each request needs (0 past B)
    __shared__ int s_red[2];
    __shared__ int s_free[KV_STAGE];                    // free_ids[nf - win .. nf)
    const KvCache& c = a.c;
    const int b = threadIdx.x;
    const int bs = c.block, mb = c.max_blocks;
    const int nf_in = *c.n_free;
    int acc = -1, L0 = 0;
    int pe[DDT_MAX_DEPTH + 1];                          // the path entries (Dp <= DDT_MAX_DEPTH)
    if (b < c.B) {
        acc = a.accept_len[b];
        L0 = c.len[b];
#pragma unroll
        for (int j = 0; j <= DDT_MAX_DEPTH; ++j) pe[j] = a.accept_path[(size_t)b * (a.Dp + 1) + min(j, a.Dp)];
    }
    const int nf = min(max(nf_in, 0), c.n_blocks);
    const int win = min(nf, KV_STAGE);
    int stg[KV_STAGE / KV_NT];
#pragma unroll
    for (int u = 0; u < KV_STAGE / KV_NT; ++u) {
        const int i = b + u * KV_NT;
        stg[u] = i < win ? c.free_ids[nf - win + i] : 0;
    }
    auto pop = [&](int idx) { return idx >= nf - win ? s_free[idx - (nf - win)] : c.free_ids[idx]; };
    int st = 0, n = 0, off = 0, first = 0, last = -1, X = -1, r = 0, need = 0;
    bool live = false;
    if (b < c.B && acc >= 0) {
        n = acc + 1;
        bool bad = n > a.Dp + 1;
#pragma unroll
        for (int j = 0; j <= DDT_MAX_DEPTH; ++j)
            if (j < n && (pe[j] < 0 || pe[j] >= a.P)) bad = true;
        if (bad) {
            st = -3;
        } else if (L0 < 0 || L0 + n > mb * bs) {
            st = -1;
        } else {
            live = true;
            off = L0 % bs;
            first = L0 / bs;
            last = (L0 + n - 1) / bs;
            if (off > 0) {
                X = c.table[(size_t)b * mb + first];
                r = (unsigned)X < (unsigned)c.n_blocks ? c.ref[X] : 0;
            }
            const bool cow = off > 0 && r > 1;
            need = (last - first + 1) - (off > 0 ? 1 : 0) + (cow ? 1 : 0);
            if (!cow) X = -1;
        }
    }
#pragma unroll
    for (int u = 0; u < KV_STAGE / KV_NT; ++u)
        if (b + u * KV_NT < win) s_free[b + u * KV_NT] = stg[u];
    s_need[b] = need;
    if (b == 0) { s_red[0] = 0; s_red[1] = 0; }
    // admission in index order while the free stack lasts
    const int pre = kv_block_scan(need, s_w);
    const bool adm = live && pre <= nf;
    if (live) st = adm ? n : -2;
    // blocks taken: the prefix at the last request whose prefix fits (the
    // prefixes never decrease, so exactly one thread finds itself there, or
    // none when the first request does not fit)
    if (pre <= nf && (b == KV_NT - 1 || pre + s_need[b + 1] > nf)) s_red[0] = pre;
    s_x[b] = adm ? X : -1;
    __syncthreads();
    // copiers of one old block: the lowest-index one settles its holder count
    // and, when no holder is left, pushes it
    int cnt = 0;
    bool lowest = true;
    if (adm && X >= 0) {
        for (int j = 0; j < c.B; ++j)
            if (s_x[j] == X) {
                ++cnt;
                if (j < b) lowest = false;
            }
    }
    const bool frees = adm && X >= 0 && lowest && cnt == r;
    const int prank = kv_block_scan(frees ? 1 : 0, s_w) - (frees ? 1 : 0);
    if (frees) atomicAdd(&s_red[1], 1);
    // pops: request b takes free_ids[top - 1], [top - 2], ... with top = nf
    // minus the blocks of the admitted requests before it
    int cowblk = -1;
    if (adm) {
        int top = nf - (pre - need);
        if (X >= 0) {
            cowblk = pop(--top);
            c.table[(size_t)b * mb + first] = cowblk;
            if ((unsigned)cowblk < (unsigned)c.n_blocks) c.ref[cowblk] = 1;
        }
        for (int t = first + (off > 0 ? 1 : 0); t <= last; ++t) {
            const int nb = pop(--top);
            c.table[(size_t)b * mb + t] = nb;
            if ((unsigned)nb < (unsigned)c.n_blocks) c.ref[nb] = 1;
        }
        c.len[b] = L0 + n;
        if (X >= 0 && lowest) c.ref[X] = r - cnt;
    }
    if (b < c.B) {
        *(int4*)(c.plan + 4 * b) = make_int4(L0, adm ? n : 0, adm ? X : -1, cowblk);
        a.status[b] = st;
    }
    __syncthreads();                                    // every pop has read its id before the pushes reuse the slots
    const int total = s_red[0];
    if (frees && nf - total + prank < c.n_blocks) c.free_ids[nf - total + prank] = X;
    if (b == 0) *c.n_free = nf - total + s_red[1];
}

// data movement of a commit: workgroup b copies request b's shared partial
// block (copy-on-write) and its accepted path.  The rows' source and
// destination offsets are worked out first (one thread per token, into LDS),
// so the copy loop's loads depend on nothing but the loop index.
__global__ __launch_bounds__(KV_CT) void k_kv_copy(KvCommitArgs a) {
    __shared__ size_t s_src[DDT_MAX_DEPTH + 1], s_dst[DDT_MAX_DEPTH + 1];
    const KvCache& c = a.c;
    const int b = blockIdx.x;
    const int j = threadIdx.x;
    const int4 pl = *(const int4*)(c.plan + 4 * b);
    const int p = j <= a.Dp ? a.accept_path[(size_t)b * (a.Dp + 1) + j] : 0;  // with the plan: n <= Dp + 1
    const int L0 = pl.x, n = pl.y, X = pl.z, nbk = pl.w;
    if (n == 0) return;
    const int HD = c.Hkv * c.D;                         // elements per token, a multiple of 8
    const int V8 = HD / 8;                              // 16-byte words per token
    const int bs = c.block;
    if (j < n) {
        const int t = L0 + j;
        const int blk = c.table[(size_t)b * c.max_blocks + t / bs];
        s_src[j] = ((size_t)b * a.P + p) * HD;
        s_dst[j] = (unsigned)blk < (unsigned)c.n_blocks ? ((size_t)blk * bs + t % bs) * HD : ~(size_t)0;
    }
    const int e0 = blockIdx.y * KV_CT + threadIdx.x;   // this workgroup's share: every KV_SPLIT-th run of KV_CT words
    if ((unsigned)X < (unsigned)c.n_blocks && (unsigned)nbk < (unsigned)c.n_blocks) {
        const int off = L0 % bs;
        const size_t so = (size_t)X * bs * HD, dof = (size_t)nbk * bs * HD;
        for (int e = e0; e < off * V8; e += KV_CT * KV_SPLIT) {
            *(u32x4*)(c.k + dof + 8 * (size_t)e) = *(const u32x4*)(c.k + so + 8 * (size_t)e);
            *(u32x4*)(c.v + dof + 8 * (size_t)e) = *(const u32x4*)(c.v + so + 8 * (size_t)e);
        }
    }
    __syncthreads();
    for (int e = e0; e < n * V8; e += KV_CT * KV_SPLIT) {
        const int tok = e / V8, w = e - tok * V8;
        const size_t src = s_src[tok] + 8 * (size_t)w;
        const u32x4 kd = *(const u32x4*)(a.kt + src);   // loads outside the store's guard
        const u32x4 vd = *(const u32x4*)(a.vt + src);
        const size_t dst = s_dst[tok];
        if (dst != ~(size_t)0) {
            *(u32x4*)(c.k + dst + 8 * (size_t)w) = kd;
            *(u32x4*)(c.v + dst + 8 * (size_t)w) = vd;
        }
    }
}

// fork: pairs in order; dst takes src's blocks (one more holder each) and length
__global__ __launch_bounds__(KV_NT) void k_kv_fork(KvForkArgs a) {
    __shared__ int s_ok;
    const KvCache& c = a.c;
    const int mb = c.max_blocks;
    for (int i = 0; i < a.n; ++i) {
        const int s = a.src[i], d = a.dst[i];
        if (threadIdx.x == 0) {
            bool ok = s >= 0 && s < c.B && d >= 0 && d < c.B && s != d;
            if (ok) ok = c.len[d] == 0 && c.table[(size_t)d * mb] == -1;
            for (int j = 0; j < a.n && ok; ++j) ok = a.src[j] != d;
            s_ok = ok;
            a.status[i] = ok ? 0 : -1;
        }
        __syncthreads();
        if (s_ok) {
            for (int t = threadIdx.x; t < mb; t += KV_NT) {
                const int x = c.table[(size_t)s * mb + t];
                c.table[(size_t)d * mb + t] = x;
                if ((unsigned)x < (unsigned)c.n_blocks) atomicAdd(&c.ref[x], 1);
            }
            if (threadIdx.x == 0) c.len[d] = c.len[s];
        }
        __syncthreads();
    }
}

// release: requests in order; blocks left with no holder are pushed in table
// order (thread t handles entries 4t .. 4t + 3, so a scan keeps that order)
__global__ __launch_bounds__(KV_NT) void k_kv_release(KvReleaseArgs a) {
    __shared__ int s_w[KV_NT / 64];
    __shared__ int s_nf;
    const KvCache& c = a.c;
    const int mb = c.max_blocks;
    if (threadIdx.x == 0) s_nf = min(max(*c.n_free, 0), c.n_blocks);
    __syncthreads();
    for (int i = 0; i < a.n; ++i) {
        const int r = a.req[i];
        if (r < 0 || r >= c.B) continue;
        int freed[KV_MAXBLK / KV_NT];
        int nfree = 0;
#pragma unroll
        for (int u = 0; u < KV_MAXBLK / KV_NT; ++u) {
            const int t = threadIdx.x * (KV_MAXBLK / KV_NT) + u;
            freed[u] = -1;
            if (t < mb) {
                const int x = c.table[(size_t)r * mb + t];
                if ((unsigned)x < (unsigned)c.n_blocks) {
                    if (atomicSub(&c.ref[x], 1) == 1) {
                        freed[u] = x;
                        ++nfree;
                    }
                    c.table[(size_t)r * mb + t] = -1;
                }
            }
        }
        const int incl = kv_block_scan(nfree, s_w);
        int pos = s_nf + incl - nfree;
#pragma unroll
        for (int u = 0; u < KV_MAXBLK / KV_NT; ++u)
            if (freed[u] >= 0) {
                if (pos < c.n_blocks) c.free_ids[pos] = freed[u];
                ++pos;
            }
        __syncthreads();                                // every thread has read s_nf
        if (threadIdx.x == KV_NT - 1) s_nf = min(s_nf + incl, c.n_blocks);    // the last inclusive sum is the total
        if (threadIdx.x == 0) c.len[r] = 0;
        __syncthreads();
    }
    if (threadIdx.x == 0) *c.n_free = s_nf;
}
