// Tree attention for the verify forward: every verified flat position attends
// to the context prefix and to its ancestors (itself included), never to a
// sibling (EAGLE-2 explainer, reranking section and engineering difficulty
// one; Graft review, execution-flow step 3).  The visible tree positions are
// the set bits of the flat mask row that the mask kernel writes.
//
// One 256-thread workgroup per (request, key/value head, tile of 64 query
// rows); query row r is flat position r / G with query head g*G + r % G, so
// the G heads of one position sit in adjacent rows and share its mask row.
// Each wave owns 16 rows and walks the keys (prefix, then the verified tree
// positions) in blocks of 64 staged in LDS: K row-major, V transposed.
//
// The products run on 16x16x32 bf16 MFMA in transposed form: S^T = K Q^T,
// then O^T = V^T P^T.  Lane l then holds scores and outputs of the single
// query row l % 16, so the online softmax statistics and the rescaling of
// the output stay in the lane.  Keys are fed to the first product in an
// order that leaves each lane holding 8 consecutive keys of every 32-key
// chunk, which is exactly the weight operand of the second product: the
// weights never move between lanes.
#pragma once
#include "ddt_device.hpp"

typedef __bf16 ta_bf16x8 __attribute__((ext_vector_type(8)));
typedef float ta_f32x4 __attribute__((ext_vector_type(4)));

#define TA_NT 256
#define TA_ROWS 64              // query rows per workgroup (16 per wave)
#define TA_KB 64                // keys per block
#define TA_D 128                // head dimension
#define TA_KS (TA_D + 8)        // LDS row of K, bf16 elements (padding spreads the banks)
#define TA_VS (TA_KB + 8)       // LDS row of V^T
#define TA_MW 8                 // mask words per row (flat positions <= 256)

struct AttnArgs {
    const uint16_t* q;          // bf16 [B][P][Hq][D]
    const uint16_t* kp;         // bf16 [B][L][Hkv][D]
    const uint16_t* vp;
    const uint16_t* kt;         // bf16 [B][P][Hkv][D]
    const uint16_t* vt;
    const uint32_t* mask;       // [B][P][W]
    const int32_t* m;           // [B]
    float* out;                 // fp32 [B][P][Hq][D]
    int P, W, Hq, Hkv, G, L, tiles;
    float sl2;                  // scale * log2(e)
};

__device__ __forceinline__ ta_bf16x8 ta_as_bf16x8(u32x4 v) { return __builtin_bit_cast(ta_bf16x8, v); }

__global__ __launch_bounds__(TA_NT) void k_tree_attention(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_k[TA_KB * TA_KS];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[TA_D * TA_VS];
    __shared__ uint32_t s_mask[TA_ROWS * TA_MW];

    const int tile = blockIdx.x % a.tiles;
    const int bg = blockIdx.x / a.tiles;
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int P = a.P, G = a.G, Hq = a.Hq, Hkv = a.Hkv, L = a.L;
    const int n = min(max(a.m[b], 0), P - 1) + 1;       // verified flat positions
    const int R = n * G;                                // live query rows
    const int RT = P * G;                               // rows of the output tensor
    const int r0 = tile * TA_ROWS;

    // this lane's query row (the column of its S^T and O^T fragments)
    const int row = r0 + wid * 16 + (lane & 15);
    const bool live = row < R;
    const int pi = row / G, h = g * G + (row - (row / G) * G);
    const int gq = lane >> 4;                           // lane group: k offset 8*gq

    if (r0 >= R) {
        // only padding rows: zeros
        for (int e = tid; e < TA_ROWS * TA_D; e += TA_NT) {
            const int r = r0 + e / TA_D, d = e - (e / TA_D) * TA_D;
            if (r < RT) {
                const int i = r / G, hh = g * G + (r - (r / G) * G);
                a.out[(((size_t)b * P + i) * Hq + hh) * TA_D + d] = 0.f;
            }
        }
        return;
    }

    // the rows' mask words, and the lane's query fragments (B operand of S^T:
    // lane l holds Q[row][32c + 8*gq .. +7] for d-chunk c)
    for (int e = tid; e < TA_ROWS * TA_MW; e += TA_NT) {
        const int rr = e / TA_MW, w = e - (e / TA_MW) * TA_MW;
        const int r = r0 + rr;
        uint32_t v = 0u;
        if (r < R && w < a.W) v = a.mask[((size_t)b * P + r / G) * a.W + w];
        s_mask[e] = v;
    }
    ta_bf16x8 qf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (live) v = *(const u32x4*)(a.q + (((size_t)b * P + pi) * Hq + h) * TA_D + 32 * c + 8 * gq);
        qf[c] = ta_as_bf16x8(v);
    }

    ta_f32x4 o[TA_D / 16];
#pragma unroll
    for (int t = 0; t < TA_D / 16; ++t) o[t] = ta_f32x4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lsum = 0.f;
    const int lrow = wid * 16 + (lane & 15);            // row within the tile
    const int NK = L + n;                               // keys: prefix, then tree positions

    for (int k0 = 0; k0 < NK; k0 += TA_KB) {
        __syncthreads();                                // previous block consumed (and s_mask written)
        // stage K: thread t -> key t/4, dims (t%4)*32 .. +31
        {
            const int kl = tid >> 2, d0 = (tid & 3) * 32;
            const int j = k0 + kl;
            const uint16_t* src = nullptr;
            if (j < L) src = a.kp + (((size_t)b * L + j) * Hkv + g) * TA_D;
            else if (j < NK) src = a.kt + (((size_t)b * P + (j - L)) * Hkv + g) * TA_D;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (src) v = *(const u32x4*)(src + d0 + 8 * u);
                *(u32x4*)(s_k + kl * TA_KS + d0 + 8 * u) = v;
            }
        }
        // stage V transposed: thread t -> keys 4*(t%16) .. +3, dims 8*(t/16) .. +7
        {
            const int kq = (tid & 15) * 4, d0 = (tid >> 4) * 8;
            uint32_t w[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = k0 + kq + u;
                const uint16_t* src = nullptr;
                if (j < L) src = a.vp + (((size_t)b * L + j) * Hkv + g) * TA_D;
                else if (j < NK) src = a.vt + (((size_t)b * P + (j - L)) * Hkv + g) * TA_D;
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (src) v = *(const u32x4*)(src + d0);
                w[u][0] = v[0]; w[u][1] = v[1]; w[u][2] = v[2]; w[u][3] = v[3];
            }
            // element e of key u is half (e & 1) of word e >> 1
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sh = (e & 1) * 16;
                const uint32_t lo = ((w[0][e >> 1] >> sh) & 0xFFFFu) | (((w[1][e >> 1] >> sh) & 0xFFFFu) << 16);
                const uint32_t hi = ((w[2][e >> 1] >> sh) & 0xFFFFu) | (((w[3][e >> 1] >> sh) & 0xFFFFu) << 16);
                *(uint2*)(s_vt + (d0 + e) * TA_VS + kq) = make_uint2(lo, hi);
            }
        }
        __syncthreads();

        // S^T = K Q^T per 16-key sub-block: A row rho of sub-block s of chunk
        // c2 is key 32*c2 + 8*(rho/4) + 4*s + rho%4, so that accumulator j of
        // lane l is key 32*c2 + 8*gq + 4*s + j
        float sc[2][2][4];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int rho = lane & 15;
                const int kl = 32 * c2 + 8 * (rho >> 2) + 4 * s + (rho & 3);
                ta_f32x4 acc = ta_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const ta_bf16x8 kf = ta_as_bf16x8(*(const u32x4*)(s_k + kl * TA_KS + 32 * c + 8 * gq));
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], acc, 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) sc[c2][s][j] = acc[j];
            }
        }
        // visibility and the online softmax (row statistics over the 4 lane
        // groups that share this query row)
        float bmax = -INFINITY;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = k0 + 32 * c2 + 8 * gq + 4 * s + j;
                    bool vis = key < L;
                    if (!vis && key < NK) {
                        const int tp = key - L;
                        vis = (s_mask[lrow * TA_MW + (tp >> 5)] >> (tp & 31)) & 1u;
                    }
                    const float v = vis && live ? sc[c2][s][j] * a.sl2 : -INFINITY;
                    sc[c2][s][j] = v;
                    bmax = fmaxf(bmax, v);
                }
            }
        }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
        const float mnew = fmaxf(mrun, bmax);
        const float alpha = mnew == -INFINITY ? 1.f : exp2f(mrun - mnew);
        float psum = 0.f;
        ta_bf16x8 pf[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p = mnew == -INFINITY ? 0.f : exp2f(sc[c2][s][j] - mnew);
                    psum += p;
                    pf[c2][4 * s + j] = (__bf16)p;
                }
            }
        }
        lsum = lsum * alpha + psum;
        mrun = mnew;
        // O^T += V^T P^T: tile t covers dims 16t .. 16t + 15; lane l reads
        // V^T[16t + l%16][32*c2 + 8*gq .. +7]
#pragma unroll
        for (int t = 0; t < TA_D / 16; ++t) {
            o[t] *= alpha;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const ta_bf16x8 vf = ta_as_bf16x8(*(const u32x4*)(s_vt + (16 * t + (lane & 15)) * TA_VS + 32 * c2 + 8 * gq));
                o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[c2], o[t], 0, 0, 0);
            }
        }
    }

    // normalise: the row's weight total over its 4 lane groups; accumulator j
    // of tile t is dim 16t + 4*gq + j of the lane's row
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (row < RT) {
        const float inv = live && lsum > 0.f ? 1.f / lsum : 0.f;
        float* dst = a.out + (((size_t)b * P + pi) * Hq + h) * TA_D;
#pragma unroll
        for (int t = 0; t < TA_D / 16; ++t)
            *(ta_f32x4*)(dst + 16 * t + 4 * gq) = o[t] * inv;
    }
}
