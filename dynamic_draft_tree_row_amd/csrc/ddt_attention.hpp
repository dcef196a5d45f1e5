// Tree attention for the verify forward: every verified flat position attends
// to the context prefix and to its ancestors (itself included), never to a
// sibling (EAGLE-2 explainer, reranking section and engineering difficulty
// one; Graft review, execution-flow step 3).  The visible tree positions are
// the set bits of the flat mask row that the mask kernel writes.
//
// One 256-thread workgroup per (request, key/value head, tile of 128 query
// rows); query row r is flat position r / G with query head g*G + r % G, so
// the G heads of one position sit in adjacent rows.  Each wave owns 32 rows
// and walks the keys in blocks of 64: the prefix blocks first, then the tree
// blocks, which start on a block boundary so that a block is either all
// prefix (visible to every row; only a ragged last block needs a bound) or
// all tree (tested against the rows' mask words).  Blocks are staged in LDS,
// double-buffered, with the next block's global loads in flight while the
// current one is computed: K row-major with a 16-byte-chunk swizzle, V
// transposed.
//
// The products run on 32x32x16 bf16 MFMA in transposed form: S^T = K Q^T,
// then O^T = V^T P^T.  Lane l then holds scores and outputs of the single
// query row l % 32 (the two lane halves split the keys), so the online
// softmax statistics and the output rescaling stay in the lane.  Keys are fed
// to the first product in an order that leaves each lane half holding 8
// consecutive keys of every 16-key chunk, which is exactly the weight operand
// of the second product: the weights never move between lanes.
//
// The running maximum moves only when a block's maximum exceeds it by more
// than 2^8 in the exponent's units; until then the weights are taken against
// the stale maximum (at most 2^8, far from fp32 range).  Softmax does not
// depend on the offset, so only rounding differs from the exact-max form.
#pragma once
#include "ddt_device.hpp"

typedef __bf16 ta_bf16x8 __attribute__((ext_vector_type(8)));
typedef float ta_f32x16 __attribute__((ext_vector_type(16)));

#define TA_NT 256
#define TA_WR 32                // query rows per wave
#define TA_ROWS 128             // query rows per workgroup
#define TA_KB 64                // keys per block
#define TA_D 128                // head dimension
#define TA_VS (TA_KB + 8)       // LDS row of V^T, bf16 elements (padding spreads the banks)
#define TA_KBUF (TA_KB * TA_D)  // one K buffer, bf16 elements
#define TA_VBUF (TA_D * TA_VS)  // one V^T buffer
#define TA_MW 8                 // mask words per row (flat positions <= 256)
#define TA_HEADROOM 8.f         // log2 slack before the running maximum is moved
#define TA_MFLOOR (-1.0e30f)    // running maximum before any visible key

struct AttnArgs {
    const uint16_t* q;          // bf16 [B][P][Hq][D]
    const uint16_t* kp;         // bf16 [B][L][Hkv][D]
    const uint16_t* vp;
    const uint16_t* kt;         // bf16 [B][P][Hkv][D]
    const uint16_t* vt;
    const uint32_t* mask;       // [B][P][W]
    const int32_t* m;           // [B]
    float* out;                 // fp32 [B][P][Hq][D]
    int P, W, Hq, Hkv, G, L, tiles, groups;     // groups = B * Hkv
    float sl2;                  // scale * log2(e), > 0
};

__device__ __forceinline__ ta_bf16x8 ta_as_bf16x8(u32x4 v) { return __builtin_bit_cast(ta_bf16x8, v); }

// 16-byte chunk swizzle of K row k: keys that one read phase touches (k and
// k + 4, k + 8, k + 12 within 16) land on different chunks
__device__ __forceinline__ int ta_kswz(int k) { return (k & 3) | ((k >> 1) & 4) | ((k << 1) & 8); }

__global__ __launch_bounds__(TA_NT, 2) void k_tree_attention(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_k[2 * TA_KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2 * TA_VBUF];

    // workgroups are dealt to the 8 XCDs in turn; renumber so that each XCD
    // takes a contiguous run of (head, tile) and the tiles of one key/value
    // head read its keys through the same L2
    const int total = a.groups * a.tiles;
    const int xq = total >> 3, xr = total & 7;
    const int xc = blockIdx.x & 7, xs = blockIdx.x >> 3;
    const int lid = xc < xr ? xc * (xq + 1) + xs : xr * (xq + 1) + (xc - xr) * xq + xs;
    const int tile = lid % a.tiles, bg = lid / a.tiles;
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int rl = lane & 31, hh = lane >> 5;           // query row in the wave, lane half
    const int P = a.P, G = a.G, Hq = a.Hq, Hkv = a.Hkv, L = a.L;
    const int n = min(max(a.m[b], 0), P - 1) + 1;       // verified flat positions
    const int R = n * G;                                // live query rows
    const int RT = P * G;                               // rows of the output tensor
    const int r0 = tile * TA_ROWS;

    if (r0 >= R) {
        // only padding rows: zeros
        for (int e = tid; e < TA_ROWS * (TA_D / 4); e += TA_NT) {
            const int r = r0 + e / (TA_D / 4), d4 = e - (e / (TA_D / 4)) * (TA_D / 4);
            if (r < RT) {
                const int i = r / G, hq = g * G + (r - (r / G) * G);
                *(float4*)(a.out + (((size_t)b * P + i) * Hq + hq) * TA_D + 4 * d4) = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        return;
    }

    const int row = r0 + wid * TA_WR + rl;
    const bool live = row < R;
    const bool wave_live = r0 + wid * TA_WR < R;        // a wave of padding rows only stages
    const int rc = live ? row : R - 1;                  // loads of dead rows read a live one
    const int pc = rc / G, hc = g * G + (rc - pc * G);

    // query fragments (B operand of S^T): qf[c] = Q[row][16c + 8*hh .. +7]
    ta_bf16x8 qf[TA_D / 16];
    {
        const uint16_t* qrow = a.q + (((size_t)b * P + pc) * Hq + hc) * TA_D + 8 * hh;
        u32x4 qr[TA_D / 16];
#pragma unroll
        for (int c = 0; c < TA_D / 16; ++c) qr[c] = *(const u32x4*)(qrow + 16 * c);
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < TA_D / 16; ++c) qf[c] = ta_as_bf16x8(live ? qr[c] : z);
    }
    const uint32_t* mrow = a.mask + ((size_t)b * P + pc) * a.W;

    // staging: thread t carries key t/4, dims (t%4)*32 .. +31 of K and keys
    // 4*(t%16) .. +3, dims 8*(t/16) .. +7 of V (written transposed)
    const int HD = Hkv * TA_D;
    const int skl = tid >> 2, sd0 = (tid & 3) * 32;
    const int vkq = (tid & 15) * 4, vd0 = (tid >> 4) * 8;
    const uint16_t* kpb = a.kp + ((size_t)b * L * Hkv + g) * TA_D;
    const uint16_t* vpb = a.vp + ((size_t)b * L * Hkv + g) * TA_D;
    const uint16_t* ktb = a.kt + ((size_t)b * P * Hkv + g) * TA_D;
    const uint16_t* vtb = a.vt + ((size_t)b * P * Hkv + g) * TA_D;
    const int npb = (L + TA_KB - 1) / TA_KB;            // prefix blocks
    const int nblk = npb + (n + TA_KB - 1) / TA_KB;     // then tree blocks
    // block x: first key, bound, and source (prefix or tree)
    auto blk_base = [&](int x) { return x < npb ? x * TA_KB : (x - npb) * TA_KB; };
    auto blk_lim = [&](int x) { return x < npb ? L : n; };

    u32x4 pk[4], pv[4];
    uint32_t vval = 0u;                                 // bit u: V key vkq + u valid
    // every load reads a valid row (invalid keys read the block source's
    // first row) and is issued straight-line, so the next block's loads stay
    // in flight across the current block's compute
    auto fetch = [&](int x) {
        const bool pre = x < npb;
        const int base = blk_base(x), lim = blk_lim(x);
        const uint16_t* ks = pre ? kpb : ktb;
        const uint16_t* vs = pre ? vpb : vtb;
        int jk = base + skl;
        jk = jk < lim ? jk : 0;
        const uint16_t* src = ks + (size_t)jk * HD + sd0;
#pragma unroll
        for (int u = 0; u < 4; ++u) pk[u] = *(const u32x4*)(src + 8 * u);
        vval = 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int jv = base + vkq + u;
            vval |= jv < lim ? (1u << u) : 0u;
            jv = jv < lim ? jv : 0;
            pv[u] = *(const u32x4*)(vs + (size_t)jv * HD + vd0);
        }
    };
    auto stage = [&](int x, int buf) {
        uint16_t* sk = s_k + buf * TA_KBUF;
        uint16_t* sv = s_vt + buf * TA_VBUF;
        const int swz = ta_kswz(skl);
#pragma unroll
        for (int u = 0; u < 4; ++u) *(u32x4*)(sk + skl * TA_D + (((4 * (tid & 3) + u) ^ swz) << 3)) = pk[u];
        if (blk_base(x) + TA_KB > blk_lim(x)) {
            // values of invalid keys are zero (their weights are zero too)
            const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < 4; ++u) pv[u] = (vval >> u) & 1u ? pv[u] : z;
        }
        // word w of key u holds dims 2w (low half) and 2w + 1 (high half)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t e01 = __builtin_amdgcn_perm(pv[1][w], pv[0][w], 0x05040100u);
            const uint32_t e23 = __builtin_amdgcn_perm(pv[3][w], pv[2][w], 0x05040100u);
            const uint32_t o01 = __builtin_amdgcn_perm(pv[1][w], pv[0][w], 0x07060302u);
            const uint32_t o23 = __builtin_amdgcn_perm(pv[3][w], pv[2][w], 0x07060302u);
            *(uint2*)(sv + (vd0 + 2 * w) * TA_VS + vkq) = make_uint2(e01, e23);
            *(uint2*)(sv + (vd0 + 2 * w + 1) * TA_VS + vkq) = make_uint2(o01, o23);
        }
    };

    // A row rho of a 32-key half of S^T is key 16*(rho/16) + 8*((rho/4)%2)
    // + 4*((rho/8)%2) + rho%4, so that accumulator j of lane half hh is key
    // 16*(j/8) + 8*hh + j%8 of that half
    const int krow = 16 * (rl >> 4) + 8 * ((rl >> 2) & 1) + 4 * ((rl >> 3) & 1) + (rl & 3);
    int koff[TA_D / 16];                                // element offset of chunk 2c + hh of K row krow
    {
        const int swz = ta_kswz(krow);
#pragma unroll
        for (int c = 0; c < TA_D / 16; ++c) koff[c] = krow * TA_D + (((2 * c + hh) ^ swz) << 3);
    }
    const int voff = rl * TA_VS + 8 * hh;               // V^T row rl, keys 8*hh ..

    ta_f32x16 o[TA_D / 32];
#pragma unroll
    for (int t = 0; t < TA_D / 32; ++t)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[t][j] = 0.f;
    float mrun = TA_MFLOOR, lsum = 0.f;
    const float sl2 = a.sl2;

    auto compute = [&](int x, int buf) {
        const uint16_t* sk = s_k + buf * TA_KBUF;
        const uint16_t* sv = s_vt + buf * TA_VBUF;
        const bool pre = x < npb;
        const int base = blk_base(x);
        // tree blocks: this row's mask words, loaded ahead of the products
        uint32_t mw[2] = {0u, 0u};
        if (!pre) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int w = (base >> 5) + kb;
                const uint32_t v = mrow[min(w, a.W - 1)];
                const int nb = n - 32 * w;                  // positions < n only
                const uint32_t lim = nb >= 32 ? 0xFFFFFFFFu : nb <= 0 ? 0u : (1u << nb) - 1u;
                mw[kb] = (v & lim) >> (8 * hh);
            }
        }
        ta_f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
#pragma unroll
        for (int c = 0; c < TA_D / 16; ++c) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const ta_bf16x8 kf = ta_as_bf16x8(*(const u32x4*)(sk + koff[c] + kb * 32 * TA_D));
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
            }
        }
        if (!pre) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (!((mw[kb] >> (16 * (j >> 3) + (j & 7))) & 1u)) s[kb][j] = -INFINITY;
        } else if (base + TA_KB > L) {
            const int lim = L - base - 8 * hh;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (32 * kb + 16 * (j >> 3) + (j & 7) >= lim) s[kb][j] = -INFINITY;
        }
        // block maximum of the row (both lane halves)
        float bm = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) bm = fmaxf(bm, s[kb][j]);
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mnew = fmaxf(mrun, bm);
        if (__ballot((mnew - mrun) * sl2 > TA_HEADROOM) != 0ull) {
            const float alpha = __builtin_amdgcn_exp2f((mrun - mnew) * sl2);
#pragma unroll
            for (int t = 0; t < TA_D / 32; ++t) o[t] *= alpha;
            lsum *= alpha;
            mrun = mnew;
        }
        // weights 2^(sl2 * (s - mrun)) <= 2^8, summed in fp32, bf16 for the product
        const float nm = -mrun * sl2;
        float ps = 0.f;
        ta_bf16x8 pf[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][j], sl2, nm));
                ps += p;
                pf[2 * kb + (j >> 3)][j & 7] = (__bf16)p;
            }
        lsum += ps;
        // O^T += V^T P^T over 16-key chunks q; tile t covers dims 32t .. 32t + 31
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int t = 0; t < TA_D / 32; ++t) {
                const ta_bf16x8 vf = ta_as_bf16x8(*(const u32x4*)(sv + voff + 32 * t * TA_VS + 16 * q));
                o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[q], o[t], 0, 0, 0);
            }
    };

    fetch(0);
    stage(0, 0);
    __syncthreads();
    for (int x = 0; x < nblk; x += 2) {
        // two blocks per trip so that the buffer offsets are constants
        if (x + 1 < nblk) fetch(x + 1);
        if (wave_live) compute(x, 0);
        if (x + 1 < nblk) stage(x + 1, 1);
        __syncthreads();
        if (x + 1 >= nblk) break;
        if (x + 2 < nblk) fetch(x + 2);
        if (wave_live) compute(x + 1, 1);
        if (x + 2 < nblk) stage(x + 2, 0);
        __syncthreads();
    }

    // normalise by the row's weight total (both lane halves); accumulator j of
    // tile t is dim 32t + 8*(j/4) + 4*hh + j%4 of the lane's row
    lsum += __shfl_xor(lsum, 32);
    if (row < RT) {
        const float inv = live && lsum > 0.f ? 1.f / lsum : 0.f;
        const int i = row / G, hq = g * G + (row - (row / G) * G);
        float* dst = a.out + (((size_t)b * P + i) * Hq + hq) * TA_D + 4 * hh;
#pragma unroll
        for (int t = 0; t < TA_D / 32; ++t)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq)
                *(float4*)(dst + 32 * t + 8 * jq) =
                    make_float4(o[t][4 * jq] * inv, o[t][4 * jq + 1] * inv, o[t][4 * jq + 2] * inv, o[t][4 * jq + 3] * inv);
    }
}
