// C ABI of the draft-tree library: argument checks on the host, then kernel
// launches on the caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <string.h>
#include <algorithm>
#include <mutex>

#include "../../include/ddt.h"
#include "ddt_device.hpp"
#include "ddt_rowreduce.hpp"
#include "ddt_tree_kernels.hpp"
#include "ddt_layer.hpp"
#include "ddt_attention.hpp"
#include "ddt_kvcache.hpp"

// Chunk partials of ddt_row_topk_noalloc: one fixed array per device (each
// device that loads the library holds its own copy until the process ends).
// In host code this name is only a host-side stand-in; kernels and copies
// get the device address taken by hipGetSymbolAddress (scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[DDT_NOALLOC_SCRATCH_BYTES];

namespace {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Launches of RR_WIDE_ROWS rows or more reduce wide chunks; launches over the
// flat verify rows from RR_WIDE_FLAT_ROWS rows on (only each request's first
// m_b + 1 of its P rows are live, so fewer chunks are actually reduced).
inline bool wide_rows(long long rows, bool flat = false) {
    return rows >= (flat ? RR_WIDE_FLAT_ROWS : RR_WIDE_ROWS);
}

inline int chunk_elems(int dtype, bool wide) {
    if (dtype == DDT_BF16) return wide ? RRShape<true, RR_NV_WIDE>::CH : RRShape<true, RR_NV>::CH;
    return wide ? RRShape<false, RR_NV_WIDE>::CH : RRShape<false, RR_NV>::CH;
}

// Chunks per row of the small-launch shape: the most a launch can use (sizes
// workspaces and the capacity check).
inline int chunks_of(int V, int dtype) {
    return (V + chunk_elems(dtype, false) - 1) / chunk_elems(dtype, false);
}

// Partials per row (one per chunk) of a launch over `rows` rows; the producer
// and its consumers call this with the same rows, so they agree.
inline int groups_of(long long rows, int V, int dtype, bool flat = false) {
    const int ch = chunk_elems(dtype, wide_rows(rows, flat));
    return (V + ch - 1) / ch;
}

inline size_t ws_need(long long rows, int V, int dtype, int K) {
    return (size_t)rows * (size_t)chunks_of(V, dtype) * (size_t)rr_ps(K) * 4u;
}

inline int launched() { return hipGetLastError() == hipSuccess ? DDT_OK : DDT_ELAUNCH; }

inline bool logits_ok(const ddt_logits* x) {
    return x != nullptr && x->data != nullptr && x->V >= 1 && x->s0 >= 0 && x->s1 >= 0;
}

int check_tree(const ddt_tree* t) {
    if (t == nullptr || t->token == nullptr || t->parent == nullptr || t->depth == nullptr ||
        t->eslot == nullptr || t->key == nullptr || t->S == nullptr || t->logc == nullptr ||
        t->rmax == nullptr || t->rsp == nullptr || t->n_nodes == nullptr ||
        t->layer_base == nullptr || t->n_front == nullptr || t->frontier == nullptr ||
        t->front_S == nullptr || t->front_key == nullptr ||
        t->active == nullptr || t->k_draft == nullptr || t->cont == nullptr ||
        t->widths == nullptr || t->cast_state == nullptr || t->ticket == nullptr ||
        t->walk_buf == nullptr || t->walk_sync == nullptr || t->layer_sync == nullptr)
        return DDT_EINVAL;
    if (t->B < 1 || t->cap < 2 || t->D_max < 1 || t->R_max < 1) return DDT_EINVAL;
    if (t->cap > DDT_MAX_NODES || t->D_max > DDT_MAX_DEPTH || t->R_max > DDT_MAX_FRONT)
        return DDT_ECAPACITY;
    return DDT_OK;
}

int check_flat(const ddt_flat* f, int B) {
    if (f == nullptr || f->node == nullptr || f->token == nullptr || f->parent == nullptr ||
        f->pos == nullptr || f->mask == nullptr || f->retrieve == nullptr ||
        f->n_leaves == nullptr || f->m == nullptr)
        return DDT_EINVAL;
    if (f->B != B || f->P < 1 || f->W != (f->P + 31) / 32 || f->Dp < 0 || f->L < 1)
        return DDT_EINVAL;
    if (f->P > DDT_MAX_VERIFY + 1 || f->Dp > DDT_MAX_DEPTH) return DDT_ECAPACITY;
    return DDT_OK;
}

int check_cast(const ddt_cast* c, int B) {
    if (c->S_T == nullptr || c->S_D == nullptr || c->C1 == nullptr || c->C3 == nullptr)
        return DDT_EINVAL;
    if (c->L < 1 || c->M < 1 || c->N < 1 || c->R < 1 || c->R > 8 || c->ctx_verify < 0)
        return DDT_EINVAL;
    if (B > 64 || c->M > DDT_CAST_MAX_M) return DDT_ECAPACITY;
    return DDT_OK;
}

template <class T>
inline T* carve(char*& p, size_t n) {
    T* r = (T*)p;
    p += align256(n * sizeof(T));
    return r;
}

// timing hook (ddt_set_reduce_events)
void* const* g_events = nullptr;
int g_pairs = 0, g_used = 0;

// polls before a T > 0 walk's cross-workgroup wait gives up (ddt_set_walk_spin_limit)
unsigned g_walk_spin_limit = WALK_SPIN_LIMIT;

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream), taken once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_ptr(void* stream, void** out) {
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess) return DDT_ELAUNCH;
    dev = cur;
    if (stream != nullptr) {
        hipDevice_t d = 0;
        if (hipStreamGetDevice((hipStream_t)stream, &d) != hipSuccess) return DDT_EINVAL;
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxDevices) return DDT_ECAPACITY;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return DDT_ELAUNCH;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return DDT_ELAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DDT_OK;
}

// Workgroups of the verify kernel the device holds at once (cached per device).
int resident_verify_blocks() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    if (cache[dev] == 0) {
        int cus = 0, per = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_verify, VF_NT, 0) != hipSuccess) per = 0;
        cache[dev] = cus > 0 && per > 0 ? cus * per : 1;
    }
    return cache[dev];
}

// Launch with the reduction timing hook (ddt_set_reduce_events): while it is
// set, the runtime stamps the next event pair at the kernel's own start and
// end.  part: 0 = the whole timed span is this launch; 1 = this launch starts
// a span that the next launch (part 2) ends.
template <class Kern, class... Args>
int launch_timed(int part, Kern kern, dim3 grid, dim3 blk, size_t lds, hipStream_t s, Args... args) {
    if (g_events != nullptr && g_used < g_pairs) {
        hipEvent_t e0 = (hipEvent_t)g_events[2 * g_used], e1 = (hipEvent_t)g_events[2 * g_used + 1];
        hipExtLaunchKernelGGL(kern, grid, blk, lds, s, part == 2 ? nullptr : e0, part == 1 ? nullptr : e1, 0,
                              args...);
        if (part != 1) ++g_used;
        return launched();
    }
    hipLaunchKernelGGL(kern, grid, blk, lds, s, args...);
    return launched();
}

int launch_partials(const ddt_logits* x, int n0, int n1, const int32_t* count, int count_add,
                    int K, void* ws, hipStream_t s, const float* sum_if = nullptr, int part = 0,
                    bool flat = false) {
    RowSrc rs{};
    rs.base = x->data; rs.s0 = x->s0; rs.s1 = x->s1; rs.n1 = n1;
    rs.count = count; rs.count_add = count_add; rs.sum_if = sum_if;
    const long long rows = (long long)n0 * n1;
    const int groups = groups_of(rows, x->V, x->dtype, flat);
    const long long total = rows * groups;
    if (total <= 0) return DDT_OK;
    if (total > INT32_MAX) return DDT_ECAPACITY;
    const bool bf16 = x->dtype == DDT_BF16, wide = wide_rows(rows, flat);
    const dim3 grid((unsigned)total), blk(RR_NT);
    auto kern = bf16 ? (wide ? &k_row_partial<true, RR_NV_WIDE> : &k_row_partial<true, RR_NV>)
                     : (wide ? &k_row_partial<false, RR_NV_WIDE> : &k_row_partial<false, RR_NV>);
    return launch_timed(part, kern, grid, blk, 0, s, rs, x->V, groups, K, (uint32_t*)ws);
}

}  // namespace

extern "C" {

const char* ddt_strerror(int status) {
    switch (status) {
        case DDT_OK: return "ok";
        case DDT_EINVAL: return "invalid argument (null pointer or inconsistent size/stride)";
        case DDT_EDTYPE: return "unknown logit dtype";
        case DDT_ECAPACITY: return "size exceeds a documented limit";
        case DDT_EWORKSPACE: return "workspace too small";
        case DDT_ELAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int ddt_set_reduce_events(void* const* events, int n_pairs) {
    const int used = g_used;
    g_events = (events != nullptr && n_pairs > 0) ? events : nullptr;
    g_pairs = g_events ? n_pairs : 0;
    g_used = 0;
    return used;
}

unsigned ddt_set_walk_spin_limit(unsigned polls) {
    const unsigned prev = g_walk_spin_limit;
    g_walk_spin_limit = polls == 0 ? WALK_SPIN_LIMIT : polls;
    return prev;
}

int ddt_chunk_elems(int dtype) {
    if (dtype != DDT_F32 && dtype != DDT_BF16) return -1;
    return chunk_elems(dtype, false);
}

size_t ddt_workspace_bytes(int rows, int V, int dtype, int K) {
    if (rows < 0 || V < 1 || K < 1 || (dtype != DDT_F32 && dtype != DDT_BF16)) return 0;
    return ws_need(rows, V, dtype, K);
}

size_t ddt_tree_bytes(int B, int cap, int D_max, int R_max) {
    if (B < 1 || cap < 1 || D_max < 1 || R_max < 1) return 0;
    const size_t bc = (size_t)B * cap;
    size_t n = 0;
    n += 4 * align256(bc * 4);                                 // token parent depth eslot
    n += align256(bc * 8);                                     // key
    n += 2 * align256(bc * 4);                                 // S logc
    n += 2 * align256((size_t)B * D_max * R_max * 4);          // rmax rsp
    n += 5 * align256((size_t)B * 4);                          // n_nodes layer_base n_front active k_draft
    n += 2 * align256((size_t)B * R_max * 4);                  // frontier front_S
    n += align256((size_t)B * R_max * 8);                      // front_key
    n += align256(4);                                          // cont
    n += align256((size_t)D_max * 4);                          // widths
    n += align256(16 * 8);                                     // cast_state
    n += align256(4);                                          // ticket
    n += align256((size_t)B * DDT_WALK_STRIDE * 8);            // walk_buf
    n += align256((size_t)B * 2 * 4);                          // walk_sync
    n += align256(((size_t)B * R_max + B) * 4);                // layer_sync
    return n;
}

int ddt_tree_bind(ddt_tree* t, void* base, size_t bytes, int B, int cap, int D_max, int R_max) {
    if (t == nullptr || base == nullptr) return DDT_EINVAL;
    if (((uintptr_t)base & 255u) != 0) return DDT_EINVAL;
    if (B < 1 || cap < 2 || D_max < 1 || R_max < 1) return DDT_EINVAL;
    if (cap > DDT_MAX_NODES || D_max > DDT_MAX_DEPTH || R_max > DDT_MAX_FRONT) return DDT_ECAPACITY;
    if (bytes < ddt_tree_bytes(B, cap, D_max, R_max)) return DDT_EWORKSPACE;
    const size_t bc = (size_t)B * cap;
    char* p = (char*)base;
    t->B = B; t->cap = cap; t->D_max = D_max; t->R_max = R_max;
    t->token = carve<int32_t>(p, bc);
    t->parent = carve<int32_t>(p, bc);
    t->depth = carve<int32_t>(p, bc);
    t->eslot = carve<int32_t>(p, bc);
    t->key = carve<uint64_t>(p, bc);
    t->S = carve<float>(p, bc);
    t->logc = carve<float>(p, bc);
    t->rmax = carve<float>(p, (size_t)B * D_max * R_max);
    t->rsp = carve<float>(p, (size_t)B * D_max * R_max);
    t->n_nodes = carve<int32_t>(p, B);
    t->layer_base = carve<int32_t>(p, B);
    t->n_front = carve<int32_t>(p, B);
    t->active = carve<int32_t>(p, B);
    t->k_draft = carve<int32_t>(p, B);
    t->frontier = carve<int32_t>(p, (size_t)B * R_max);
    t->front_S = carve<float>(p, (size_t)B * R_max);
    t->front_key = carve<uint64_t>(p, (size_t)B * R_max);
    t->cont = carve<int32_t>(p, 1);
    t->widths = carve<int32_t>(p, D_max);
    t->cast_state = carve<double>(p, 16);
    t->ticket = carve<uint32_t>(p, 1);
    t->walk_buf = carve<double>(p, (size_t)B * DDT_WALK_STRIDE);
    t->walk_sync = carve<uint32_t>(p, (size_t)B * 2);
    t->layer_sync = carve<uint32_t>(p, (size_t)B * R_max + B);
    return DDT_OK;
}

size_t ddt_flat_bytes(int B, int m_max, int Dp) {
    if (B < 1 || m_max < 0 || Dp < 0) return 0;
    const size_t P = (size_t)m_max + 1, W = (P + 31) / 32, L = m_max > 1 ? m_max : 1;
    size_t n = 4 * align256((size_t)B * P * 4);
    n += align256((size_t)B * P * W * 4);
    n += align256((size_t)B * L * (Dp + 1) * 4);
    n += 2 * align256((size_t)B * 4);
    return n;
}

int ddt_flat_bind(ddt_flat* f, void* base, size_t bytes, int B, int m_max, int Dp) {
    if (f == nullptr || base == nullptr || B < 1 || m_max < 0 || Dp < 0) return DDT_EINVAL;
    if (((uintptr_t)base & 255u) != 0) return DDT_EINVAL;
    if (m_max > DDT_MAX_VERIFY || Dp > DDT_MAX_DEPTH) return DDT_ECAPACITY;
    if (bytes < ddt_flat_bytes(B, m_max, Dp)) return DDT_EWORKSPACE;
    const size_t P = (size_t)m_max + 1, W = (P + 31) / 32, L = m_max > 1 ? m_max : 1;
    char* p = (char*)base;
    f->B = B; f->P = (int)P; f->W = (int)W; f->Dp = Dp; f->L = (int)L;
    f->node = carve<int32_t>(p, B * P);
    f->token = carve<int32_t>(p, B * P);
    f->parent = carve<int32_t>(p, B * P);
    f->pos = carve<int32_t>(p, B * P);
    f->mask = carve<uint32_t>(p, B * P * W);
    f->retrieve = carve<int32_t>(p, B * L * (Dp + 1));
    f->n_leaves = carve<int32_t>(p, B);
    f->m = carve<int32_t>(p, B);
    return DDT_OK;
}

int ddt_tree_expand(const ddt_tree* t, int layer, const int32_t* root_tok, const ddt_logits* logits,
                    int K_n, int K_e, const ddt_cast* cast, const ddt_graft_gate* gate, void* ws,
                    size_t ws_bytes, void* stream) {
    int st = check_tree(t);
    if (st) return st;
    if (!logits_ok(logits) || ws == nullptr) return DDT_EINVAL;
    if (logits->dtype != DDT_F32 && logits->dtype != DDT_BF16) return DDT_EDTYPE;
    if (layer < 1 || layer > t->D_max) return DDT_EINVAL;
    if (layer == 1 && root_tok == nullptr) return DDT_EINVAL;
    if (K_n < 1 || K_e < 1 || K_n > logits->V) return DDT_EINVAL;
    if (K_n > DDT_MAX_K || K_e > t->R_max) return DDT_ECAPACITY;
    if (t->R_max * K_n > AT_SORT) return DDT_ECAPACITY;
    if (chunks_of(logits->V, logits->dtype) > DDT_MAX_CHUNKS) return DDT_ECAPACITY;
    if ((long long)1 + K_n + (long long)(t->D_max - 1) * K_e * K_n > t->cap) return DDT_ECAPACITY;
    if (cast != nullptr && gate != nullptr) return DDT_EINVAL;
    if (cast != nullptr && (st = check_cast(cast, t->B))) return st;
    if (cast != nullptr && K_e > cast->N) return DDT_EINVAL;
    if (gate != nullptr && (gate->n_ck < 0 || gate->n_ck > 4 || gate->K_max < 1)) return DDT_EINVAL;
    const int R = layer == 1 ? 1 : t->R_max;
    if (ws_bytes < ws_need((long long)t->B * t->R_max, logits->V, logits->dtype, K_n))
        return DDT_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;

    // one kernel: chunk partials, row merges and children, the frontier of
    // every request, CAST's batch rule
    const long long rows = (long long)t->B * R;
    LayerArgs a;
    a.t = *t;
    if (cast) a.c = *cast; else memset(&a.c, 0, sizeof(a.c));
    a.base = logits->data; a.s0 = logits->s0; a.s1 = logits->s1;
    a.part = (uint32_t*)ws; a.root_tok = root_tok;
    a.V = logits->V; a.groups = groups_of(rows, logits->V, logits->dtype);
    a.K_n = K_n; a.K_e = K_e; a.R = R; a.layer = layer;
    a.ck = 0; a.kd_ck = 0; a.tau = 0.f; a.gate_on = gate != nullptr; a.K_max = gate ? gate->K_max : 0;
    a.cast_on = cast != nullptr;
    if (gate != nullptr)
        for (int i = 0; i < gate->n_ck; ++i)
            if (gate->ck_depth[i] == layer) { a.ck = 1; a.kd_ck = gate->k_draft[i]; a.tau = gate->tau[i]; }
    const long long total = rows * a.groups;
    if (total > INT32_MAX) return DDT_ECAPACITY;
    const bool bf16 = logits->dtype == DDT_BF16, wide = wide_rows(rows);
    const size_t cast_lds = cast ? layer_lds_d(t->B, t->R_max, cast->M) : 0;
    if (wide) {
        // many rows: the plain reduction, then one workgroup per request
        st = launch_partials(logits, t->B, R, layer == 1 ? nullptr : t->n_front, 0, K_n, ws, s, nullptr, 1);
        if (st) return st;
        const size_t lds = finish_lds(t->R_max, K_n) + cast_lds;
        return launch_timed(2, &k_expand_finish, dim3((unsigned)t->B), dim3(EF_NT), lds, s, a);
    }
    size_t lds = std::max(sizeof(RRLds), (size_t)MRG_SCR * 8);
    lds = std::max(lds, layer_lds_c(t->R_max, K_n) + cast_lds);
    auto kern = bf16 ? &k_expand_layer<true, RR_NV> : &k_expand_layer<false, RR_NV>;
    return launch_timed(0, kern, dim3((unsigned)total), dim3(RR_NT), lds, s, a);
}

int ddt_tree_rerank(const ddt_tree* t, int m_max, const ddt_cast* cast, int use_k_draft,
                    int32_t* sel, int32_t* m_out, void* stream) {
    int st = check_tree(t);
    if (st) return st;
    if (sel == nullptr || m_out == nullptr || m_max < 0) return DDT_EINVAL;
    if (m_max > DDT_MAX_VERIFY) return DDT_ECAPACITY;
    if (cast != nullptr && (st = check_cast(cast, t->B))) return st;
    if (cast != nullptr && m_max > cast->N) return DDT_EINVAL;
    RerankArgs a;
    a.t = *t;
    if (cast) a.c = *cast; else memset(&a.c, 0, sizeof(a.c));
    a.cast_on = cast != nullptr; a.use_k_draft = use_k_draft != 0; a.m_max = m_max;
    a.sel = sel; a.m_out = m_out;
    hipLaunchKernelGGL(k_rerank, dim3(t->B), dim3(RK_NT), 0, (hipStream_t)stream, a);
    return launched();
}

int ddt_succ_gather(const ddt_tree* t, const int32_t* M, int64_t M_bstride, int V, int k_succ,
                    int tpl_depth, int tpl_width, int K_max, int m_max, int32_t* sel,
                    int32_t* m_out, void* stream) {
    return ddt_succ_gather_at(t, M, M_bstride, V, k_succ, tpl_depth, tpl_width, K_max, m_max,
                              DDT_GRAFT_ROOT, sel, m_out, stream);
}

int ddt_succ_gather_at(const ddt_tree* t, const int32_t* M, int64_t M_bstride, int V, int k_succ,
                       int tpl_depth, int tpl_width, int K_max, int m_max, int anchor, int32_t* sel,
                       int32_t* m_out, void* stream) {
    if (anchor != DDT_GRAFT_ROOT && anchor != DDT_GRAFT_TAIL) return DDT_EINVAL;
    int st = check_tree(t);
    if (st) return st;
    if (M == nullptr || sel == nullptr || m_out == nullptr || V < 1 || M_bstride < 0) return DDT_EINVAL;
    if (k_succ < 1 || tpl_depth < 1 || tpl_width < 1 || K_max < 1) return DDT_EINVAL;
    if (tpl_width > k_succ || tpl_width > 32) return DDT_EINVAL;
    if (tpl_depth > DDT_MAX_DEPTH || K_max > DDT_MAX_VERIFY) return DDT_ECAPACITY;
    if (m_max < K_max) return DDT_EINVAL;
    GatherArgs a;
    a.t = *t; a.M = M; a.M_bstride = M_bstride; a.V = V; a.k_succ = k_succ; a.depth = tpl_depth;
    a.width = tpl_width; a.K_max = K_max; a.m_cap = m_max; a.sel = sel; a.m_out = m_out;
    a.anchor = anchor;
    hipLaunchKernelGGL(k_succ_gather, dim3(t->B), dim3(64), 0, (hipStream_t)stream, a);
    return launched();
}

int ddt_tree_build_mask(const ddt_tree* t, const int32_t* sel, const int32_t* m, int prefix_len,
                        const ddt_flat* f, uint8_t* dense, void* stream) {
    int st = check_tree(t);
    if (st) return st;
    if ((st = check_flat(f, t->B))) return st;
    if (sel == nullptr || m == nullptr || prefix_len < 0) return DDT_EINVAL;
    if (f->P > MK_NT || f->W > 8) return DDT_ECAPACITY;
    MaskArgs a;
    a.t = *t; a.f = *f; a.sel = sel; a.m = m; a.prefix = prefix_len; a.dense = dense;
    hipLaunchKernelGGL(k_build_mask, dim3(t->B), dim3(MK_NT), 0, (hipStream_t)stream, a);
    return launched();
}

int ddt_tree_select(const ddt_tree* t, int m_max, const ddt_cast* cast, int use_k_draft,
                    int32_t* sel, int32_t* m_out, int prefix_len, const ddt_flat* f, uint8_t* dense,
                    void* stream) {
    int st = check_tree(t);
    if (st) return st;
    if (sel == nullptr || m_out == nullptr || m_max < 0) return DDT_EINVAL;
    if (m_max > DDT_MAX_VERIFY) return DDT_ECAPACITY;
    if (cast != nullptr && (st = check_cast(cast, t->B))) return st;
    if (cast != nullptr && m_max > cast->N) return DDT_EINVAL;
    if ((st = check_flat(f, t->B))) return st;
    if (prefix_len < 0) return DDT_EINVAL;
    if (f->P > MK_NT || f->W > 8) return DDT_ECAPACITY;
    RerankArgs ra;
    ra.t = *t;
    if (cast) ra.c = *cast; else memset(&ra.c, 0, sizeof(ra.c));
    ra.cast_on = cast != nullptr; ra.use_k_draft = use_k_draft != 0; ra.m_max = m_max;
    ra.sel = sel; ra.m_out = m_out;
    MaskArgs ma;
    ma.t = *t; ma.f = *f; ma.sel = sel; ma.m = m_out; ma.prefix = prefix_len; ma.dense = dense;
    hipLaunchKernelGGL(k_select, dim3(t->B), dim3(RK_NT), 0, (hipStream_t)stream, ra, ma);
    return launched();
}

int ddt_tree_verify(const ddt_tree* t, const ddt_flat* f, const ddt_logits* target,
                    const ddt_logits* draft, int64_t draft_layer_stride, const float* temperature,
                    const float* uniforms, int proposal, int k_top, int32_t* row_topk,
                    int32_t* row_argmax,
                    int32_t* accept_len, int32_t* accept_path, int32_t* next_token, void* ws,
                    size_t ws_bytes, void* stream) {
    int st = check_tree(t);
    if (st) return st;
    if ((st = check_flat(f, t->B))) return st;
    if (!logits_ok(target) || temperature == nullptr || uniforms == nullptr || ws == nullptr ||
        accept_len == nullptr || accept_path == nullptr || next_token == nullptr)
        return DDT_EINVAL;
    if (target->dtype != DDT_F32 && target->dtype != DDT_BF16) return DDT_EDTYPE;
    if (proposal != DDT_PROPOSAL_DRAFT && proposal != DDT_PROPOSAL_POINT) return DDT_EINVAL;
    if (draft != nullptr && (!logits_ok(draft) || draft->dtype != target->dtype ||
                             draft->V != target->V || draft_layer_stride < 0))
        return DDT_EINVAL;
    if (k_top < 0 || k_top > DDT_MAX_K || k_top > target->V) return DDT_ECAPACITY;
    if (k_top > 0 && row_topk == nullptr) return DDT_EINVAL;
    if (f->P > MK_NT) return DDT_ECAPACITY;
    if (chunks_of(target->V, target->dtype) > DDT_MAX_CHUNKS) return DDT_ECAPACITY;
    if ((target->V + VF_TILE - 1) / VF_TILE > VF_MAXTILES) return DDT_ECAPACITY;
    const int Kp = k_top > 0 ? k_top : 1;
    if (ws_bytes < ws_need((long long)t->B * f->P, target->V, target->dtype, Kp))
        return DDT_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    // greedy requests (temperature 0) use only the rows' argmax and top k
    st = launch_partials(target, t->B, f->P, f->m, 1, Kp, ws, s, temperature, 0, true);
    if (st) return st;
    VerifyArgs a;
    a.t = *t; a.f = *f; a.part = (const uint32_t*)ws;
    a.chunks = groups_of((long long)t->B * f->P, target->V, target->dtype, true); a.Kp = Kp;
    a.tgt = target->data; a.bf16 = target->dtype == DDT_BF16; a.V = target->V;
    a.ts0 = target->s0; a.ts1 = target->s1;
    a.point = proposal == DDT_PROPOSAL_POINT;
    a.spin_limit = g_walk_spin_limit;
    a.drf = draft ? draft->data : nullptr; a.dl = draft_layer_stride;
    a.ds0 = draft ? draft->s0 : 0; a.ds1 = draft ? draft->s1 : 0;
    a.temperature = temperature; a.U = uniforms; a.k_top = k_top; a.row_topk = row_topk;
    a.row_argmax = row_argmax; a.accept_len = accept_len; a.accept_path = accept_path;
    a.next_token = next_token;
    // T > 0 requests split their vocabulary passes over G workgroups; the grid
    // stays within what the device holds at once, so the workgroups of a
    // request are resident together.  At most 12: every residual pass ends in
    // a barrier of the request's workgroups, and beyond about 12 the wider
    // barrier costs more than the shorter slices save
    const int ntiles = (target->V + VF_TILE - 1) / VF_TILE;
    int G = resident_verify_blocks() / t->B;
    G = G < 1 ? 1 : (G > 12 ? 12 : G);
    if (G > ntiles) G = ntiles;
    a.G = G;
    hipLaunchKernelGGL(k_verify, dim3((unsigned)(t->B * G)), dim3(VF_NT), 0, s, a);
    return launched();
}

// Key splits of the attention: when the tiles alone leave the device
// underused, as many splits as fit one resident round of 512 workgroups (two
// per compute unit of a 256-unit device: more rounds lose more to the
// partials than they gain), at least two 64-key blocks per split, at most 32
// splits.  Returns the split count (0 on invalid sizes) and the blocks per
// split.
static int attn_split_plan(int B, int P, int Hq, int Hkv, int L, int req, int* spb) {
    if (B < 1 || P < 1 || Hq < 1 || Hkv < 1 || L < 0 || Hq % Hkv != 0) return 0;
    const long long tiles = ((long long)P * (Hq / Hkv) + TA_ROWS - 1) / TA_ROWS;
    const int nblk = (L + TA_KB - 1) / TA_KB + (P + TA_KB - 1) / TA_KB;
    long long s;
    if (req > 0) {
        s = req;
    } else {
        const long long base = (long long)B * Hkv * tiles;
        s = base >= 512 ? 1 : 512 / base;
        s = std::min<long long>(s, std::max(1, nblk / 2));
    }
    s = std::max<long long>(1, std::min<long long>({s, 32, nblk}));
    const int per = (int)((nblk + s - 1) / s);
    if (spb) *spb = per;
    return (nblk + per - 1) / per;
}

static size_t attn_ws_need(int B, int P, int Hq, int splits) {
    if (splits <= 1) return 0;
    const size_t rows = (size_t)splits * B * P * Hq;
    return align256(rows * TA_D * 4) + align256(rows * 8);
}

int ddt_tree_attention_splits(int B, int P, int Hq, int Hkv, int L, int splits) {
    return attn_split_plan(B, P, Hq, Hkv, L, splits, nullptr);
}

size_t ddt_tree_attention_ws_bytes(int B, int P, int Hq, int Hkv, int L, int splits) {
    const int s = attn_split_plan(B, P, Hq, Hkv, L, splits, nullptr);
    return s == 0 ? 0 : attn_ws_need(B, P, Hq, s);
}

static int tree_attention_run(const ddt_flat* f, const ddt_attn* a, float* out, int req, void* ws,
                              size_t ws_bytes, void* stream) {
    if (f == nullptr || a == nullptr || out == nullptr) return DDT_EINVAL;
    int st = check_flat(f, a->B);
    if (st) return st;
    if (a->P != f->P || a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->L < 0) return DDT_EINVAL;
    if (a->q == nullptr || a->k_tree == nullptr || a->v_tree == nullptr) return DDT_EINVAL;
    if (a->L > 0 && (a->k_pre == nullptr || a->v_pre == nullptr)) return DDT_EINVAL;
    if (a->Hq % a->Hkv != 0 || !(a->scale > 0.f) || !(a->scale < INFINITY)) return DDT_EINVAL;
    if (a->D != TA_D || a->Hq / a->Hkv > 16 || f->W > TA_MW) return DDT_ECAPACITY;
    const long long qn = (long long)a->B * a->P * a->Hq * TA_D;
    const long long pn = (long long)a->B * a->L * a->Hkv * TA_D;
    const long long tn = (long long)a->B * a->P * a->Hkv * TA_D;
    if (qn > INT32_MAX || pn > INT32_MAX || tn > INT32_MAX) return DDT_ECAPACITY;
    AttnArgs x;
    x.q = (const uint16_t*)a->q; x.kp = (const uint16_t*)a->k_pre; x.vp = (const uint16_t*)a->v_pre;
    x.kt = (const uint16_t*)a->k_tree; x.vt = (const uint16_t*)a->v_tree;
    x.mask = f->mask; x.m = f->m; x.out = out;
    x.P = a->P; x.W = f->W; x.Hq = a->Hq; x.Hkv = a->Hkv; x.G = a->Hq / a->Hkv; x.L = a->L;
    x.tiles = (a->P * x.G + TA_ROWS - 1) / TA_ROWS;
    x.groups = a->B * a->Hkv;
    x.sl2 = a->scale * DDT_LOG2E;
    x.splits = attn_split_plan(a->B, a->P, a->Hq, a->Hkv, a->L, req, &x.spb);
    x.po = x.pml = nullptr;
    if (x.splits > 1) {
        const size_t need = attn_ws_need(a->B, a->P, a->Hq, x.splits);
        if (ws == nullptr || ws_bytes < need || ((uintptr_t)ws & 255u) != 0) return DDT_EWORKSPACE;
        x.po = (float*)ws;
        x.pml = (float*)((char*)ws + align256((size_t)x.splits * a->B * a->P * a->Hq * TA_D * 4));
    }
    const long long grid = (long long)a->B * a->Hkv * x.tiles * x.splits;
    if (grid > INT32_MAX) return DDT_ECAPACITY;
    ddt_attention_launch(x, (unsigned)grid, (hipStream_t)stream);
    return launched();
}

int ddt_tree_attention(const ddt_flat* f, const ddt_attn* a, float* out, void* stream) {
    return tree_attention_run(f, a, out, 1, nullptr, 0, stream);
}

int ddt_tree_attention_split(const ddt_flat* f, const ddt_attn* a, float* out, int splits, void* ws,
                             size_t ws_bytes, void* stream) {
    if (splits < 0) return DDT_EINVAL;
    return tree_attention_run(f, a, out, splits, ws, ws_bytes, stream);
}

static int kv_check(const ddt_kv_cache* c, KvCache* out) {
    if (c == nullptr || c->k == nullptr || c->v == nullptr || c->table == nullptr || c->len == nullptr ||
        c->ref == nullptr || c->free_ids == nullptr || c->n_free == nullptr || c->plan == nullptr)
        return DDT_EINVAL;
    if (c->B < 1 || c->max_blocks < 1 || c->n_blocks < 1 || c->block < 1 || c->Hkv < 1 || c->D < 1)
        return DDT_EINVAL;
    if ((long long)c->Hkv * c->D > (1 << 20) || ((long long)c->Hkv * c->D) % 8 != 0) return DDT_EINVAL;
    if ((((uintptr_t)c->k) | ((uintptr_t)c->v) | ((uintptr_t)c->plan)) & 15) return DDT_EINVAL;
    if (c->B > KV_MAXB || c->max_blocks > KV_MAXBLK) return DDT_ECAPACITY;
    if ((long long)c->max_blocks * c->block > INT32_MAX) return DDT_ECAPACITY;
    out->k = (uint16_t*)c->k; out->v = (uint16_t*)c->v; out->table = c->table; out->len = c->len;
    out->ref = c->ref; out->free_ids = c->free_ids; out->n_free = c->n_free; out->plan = c->plan;
    out->B = c->B; out->max_blocks = c->max_blocks; out->n_blocks = c->n_blocks; out->block = c->block;
    out->Hkv = c->Hkv; out->D = c->D;
    return DDT_OK;
}

int ddt_kv_commit(const ddt_kv_cache* c, const int32_t* accept_len, const int32_t* accept_path, int Dp,
                  const void* k_tree, const void* v_tree, int P, int32_t* status, void* stream) {
    KvCommitArgs a;
    int st = kv_check(c, &a.c);
    if (st) return st;
    if (accept_len == nullptr || accept_path == nullptr || k_tree == nullptr || v_tree == nullptr ||
        status == nullptr || P < 1 || Dp < 0)
        return DDT_EINVAL;
    if (Dp > DDT_MAX_DEPTH) return DDT_ECAPACITY;
    if ((((uintptr_t)k_tree) | ((uintptr_t)v_tree)) & 15) return DDT_EINVAL;
    a.accept_len = accept_len; a.accept_path = accept_path; a.Dp = Dp;
    a.kt = (const uint16_t*)k_tree; a.vt = (const uint16_t*)v_tree; a.P = P; a.status = status;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(k_kv_plan, dim3(1), dim3(KV_NT), 0, s, a);
    st = launched();
    if (st) return st;
    hipLaunchKernelGGL(k_kv_copy, dim3(c->B, KV_SPLIT), dim3(KV_CT), 0, s, a);
    return launched();
}

int ddt_kv_fork(const ddt_kv_cache* c, const int32_t* src, const int32_t* dst, int n, int32_t* status,
                void* stream) {
    KvForkArgs a;
    int st = kv_check(c, &a.c);
    if (st) return st;
    if (n < 0) return DDT_EINVAL;
    if (n == 0) return DDT_OK;
    if (src == nullptr || dst == nullptr || status == nullptr) return DDT_EINVAL;
    a.src = src; a.dst = dst; a.n = n; a.status = status;
    hipLaunchKernelGGL(k_kv_fork, dim3(1), dim3(KV_NT), 0, (hipStream_t)stream, a);
    return launched();
}

int ddt_kv_release(const ddt_kv_cache* c, const int32_t* req, int n, void* stream) {
    KvReleaseArgs a;
    int st = kv_check(c, &a.c);
    if (st) return st;
    if (n < 0) return DDT_EINVAL;
    if (n == 0) return DDT_OK;
    if (req == nullptr) return DDT_EINVAL;
    a.req = req; a.n = n;
    hipLaunchKernelGGL(k_kv_release, dim3(1), dim3(KV_NT), 0, (hipStream_t)stream, a);
    return launched();
}

int ddt_succ_update(int32_t* M, int64_t M_bstride, int V, int k_succ, const ddt_flat* f,
                    const int32_t* row_topk, int k_top, const ddt_logits* target, void* ws,
                    size_t ws_bytes, void* stream) {
    if (M == nullptr || f == nullptr || V < 1 || M_bstride < 0) return DDT_EINVAL;
    int st = check_flat(f, f->B);
    if (st) return st;
    if (k_succ < 1 || k_succ > DDT_MAX_K) return DDT_ECAPACITY;
    hipStream_t s = (hipStream_t)stream;
    UpdateArgs a;
    a.f = *f; a.M = M; a.M_bstride = M_bstride; a.V = V; a.k_succ = k_succ; a.B = f->B;
    a.shared = M_bstride == 0 && f->B > 1;
    a.row_topk = row_topk; a.k_top = k_top; a.part = nullptr; a.chunks = 0; a.Kp = k_succ;
    if (row_topk != nullptr) {
        if (k_top < k_succ) return DDT_EINVAL;
    } else {
        if (!logits_ok(target) || ws == nullptr || target->V != V) return DDT_EINVAL;
        if (target->dtype != DDT_F32 && target->dtype != DDT_BF16) return DDT_EDTYPE;
        if (chunks_of(V, target->dtype) > DDT_MAX_CHUNKS) return DDT_ECAPACITY;
        if (ws_bytes < ws_need((long long)f->B * f->P, V, target->dtype, k_succ)) return DDT_EWORKSPACE;
        st = launch_partials(target, f->B, f->P, f->m, 1, k_succ, ws, s, nullptr, 0, true);
        if (st) return st;
        a.part = (const uint32_t*)ws; a.chunks = groups_of((long long)f->B * f->P, V, target->dtype, true);
    }
    hipLaunchKernelGGL(k_succ_update, dim3(a.shared ? 1 : f->B), dim3(UP_NT), 0, s, a);
    return launched();
}

int ddt_row_topk(const ddt_logits* x, int n0, int n1, int K, int32_t* ids, float* logc, float* rmax,
                 float* rsp, void* ws, size_t ws_bytes, void* stream) {
    if (!logits_ok(x) || ws == nullptr || n0 < 0 || n1 < 0) return DDT_EINVAL;
    if (x->dtype != DDT_F32 && x->dtype != DDT_BF16) return DDT_EDTYPE;
    if (K < 1 || K > x->V) return DDT_EINVAL;
    if (K > DDT_MAX_K || chunks_of(x->V, x->dtype) > DDT_MAX_CHUNKS) return DDT_ECAPACITY;
    const long long rows = (long long)n0 * n1;
    if (ws_bytes < ws_need(rows, x->V, x->dtype, K)) return DDT_EWORKSPACE;
    if (rows == 0) return DDT_OK;
    hipStream_t s = (hipStream_t)stream;
    int st = launch_partials(x, n0, n1, nullptr, 0, K, ws, s);
    if (st) return st;
    RowFinishArgs a;
    a.part = (const uint32_t*)ws; a.rows = (int)rows; a.chunks = groups_of(rows, x->V, x->dtype); a.K = K;
    a.ids = ids; a.logc = logc; a.rmax = rmax; a.rsp = rsp;
    hipLaunchKernelGGL(k_row_finish, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    return launched();
}

int ddt_row_topk_noalloc(const ddt_logits* x, int n0, int n1, int K, int32_t* ids, float* logc,
                         float* rmax, float* rsp, void* stream) {
    if (!logits_ok(x) || n0 < 0 || n1 < 0) return DDT_EINVAL;
    if (x->dtype != DDT_F32 && x->dtype != DDT_BF16) return DDT_EDTYPE;
    if (K < 1 || K > x->V) return DDT_EINVAL;
    if (K > DDT_MAX_K || chunks_of(x->V, x->dtype) > DDT_MAX_CHUNKS) return DDT_ECAPACITY;
    const long long rows = (long long)n0 * n1;
    if (ws_need(rows, x->V, x->dtype, K) > (size_t)DDT_NOALLOC_SCRATCH_BYTES) return DDT_ECAPACITY;
    if (rows == 0) return DDT_OK;
    void* ws = nullptr;
    const int st = scratch_ptr(stream, &ws);
    if (st) return st;
    // every partial the finish kernel reads is written by this call first:
    // nothing in the array has to start at zero
    return ddt_row_topk(x, n0, n1, K, ids, logc, rmax, rsp, ws, DDT_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
