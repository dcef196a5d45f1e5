// Tree-attention kernel (see ddt_attention.hpp for the design); compiled on
// its own with -fno-honor-nans -mno-amdgpu-ieee.
#include <hip/hip_runtime.h>
#include "ddt_attention.hpp"

__global__ __launch_bounds__(TA_NT, 2) void k_tree_attention(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t s_k[2 * TA_KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[2 * TA_VBUF];

    // workgroups are dealt to the 8 XCDs in turn; renumber so that each XCD
    // takes a contiguous run of (head, split, tile) and the tiles of one
    // key/value head and split read their keys through the same L2
    const int total = a.groups * a.tiles * a.splits;
    const int xq = total >> 3, xr = total & 7;
    const int xc = blockIdx.x & 7, xs = blockIdx.x >> 3;
    const int lid = xc < xr ? xc * (xq + 1) + xs : xr * (xq + 1) + (xc - xr) * xq + xs;
    const int tile = lid % a.tiles, rest = lid / a.tiles;
    const int sp = rest % a.splits, bg = rest / a.splits;
    const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int rl = lane & 31, hh = lane >> 5;           // query row in the wave, lane half
    const int P = a.P, G = a.G, Hq = a.Hq, Hkv = a.Hkv, L = a.L;
    const int n = min(max(a.m[b], 0), P - 1) + 1;       // verified flat positions
    const int R = n * G;                                // live query rows
    const int RT = P * G;                               // rows of the output tensor
    const int r0 = tile * TA_ROWS;

    if (r0 >= R) {
        // only padding rows: zeros (split partials cover live rows only; the
        // combination writes the padding rows)
        if (a.splits > 1) return;
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

    // staging: with sr = t/16 and sc = t%16, thread t carries dims 8*sc .. +7
    // of K keys 16u + sr and of V keys 4*sr + u (u = 0..3); the V keys are
    // written transposed, 4 keys to an 8-byte store
    const int HD = Hkv * TA_D;
    const int sr = tid >> 4, sc = tid & 15;
    // V keys and dims of this thread: keys 4*vsr .. +3, dims 8*vsc .. +7.
    // The 16 lanes of one 8-byte LDS store phase then hold both key halves of
    // one 8-key group and 8 dims 16 apart, whose 16-byte dim slots fall on 8
    // different bank groups: the transposed stores are conflict-free
    const int vsr = 2 * (tid >> 5) + (tid & 1), vsc = 2 * ((tid >> 1) & 7) + ((tid >> 4) & 1);
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
    uint32_t vval = 0u;                                 // bit u: V key 4*vsr + u valid
    // every load reads a valid row (invalid keys read the block source's
    // first row) and is issued straight-line, so the next block's loads stay
    // in flight across the current block's compute
    auto fetch = [&](int x) {
        const bool pre = x < npb;
        const int base = blk_base(x), lim = blk_lim(x);
        const uint16_t* ks = pre ? kpb : ktb;
        const uint16_t* vs = pre ? vpb : vtb;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int jk = base + 16 * u + sr;
            jk = jk < lim ? jk : 0;
            pk[u] = *(const u32x4*)(ks + (size_t)jk * HD + 8 * sc);
        }
        vval = 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int jv = base + 4 * vsr + u;
            vval |= jv < lim ? (1u << u) : 0u;
            jv = jv < lim ? jv : 0;
            pv[u] = *(const u32x4*)(vs + (size_t)jv * HD + 8 * vsc);
        }
    };
    auto stage = [&](int x, int buf) {
        uint16_t* sk = s_k + buf * TA_KBUF;
        uint16_t* sv = s_vt + buf * TA_VBUF;
        const int kofs = sr * TA_D + ((sc ^ ta_kswz(sr)) << 3);     // the swizzle of 16u + sr is that of sr
#pragma unroll
        for (int u = 0; u < 4; ++u) *(u32x4*)(sk + kofs + 16 * u * TA_D) = pk[u];
        if (blk_base(x) + TA_KB > blk_lim(x)) {
            // values of invalid keys are zero (their weights are zero too)
            const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < 4; ++u) pv[u] = (vval >> u) & 1u ? pv[u] : z;
        }
        // word w of key u holds dims 8*vsc + 2w (low half) and + 2w + 1 (high
        // half); keys 4*vsr .. +3 are half vsr % 2 of group vsr / 2, and dim
        // 8*vsc + e sits at 8*(8*vsc + vsc/2 + e) in the group
        const int vofs = (vsr >> 1) * TA_VG + 4 * (vsr & 1) + 8 * (8 * vsc + (vsc >> 1));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t e01 = __builtin_amdgcn_perm(pv[1][w], pv[0][w], 0x05040100u);
            const uint32_t e23 = __builtin_amdgcn_perm(pv[3][w], pv[2][w], 0x05040100u);
            const uint32_t o01 = __builtin_amdgcn_perm(pv[1][w], pv[0][w], 0x07060302u);
            const uint32_t o23 = __builtin_amdgcn_perm(pv[3][w], pv[2][w], 0x07060302u);
            *(uint2*)(sv + vofs + 16 * w) = make_uint2(e01, e23);
            *(uint2*)(sv + vofs + 16 * w + 8) = make_uint2(o01, o23);
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
    const int voff = hh * TA_VG + 8 * (rl + (rl >> 4)); // group hh, dim rl

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
        // the next block's loads go out between the score products, one per
        // product pair, so that the load queue drains while the matrix pipe
        // is busy instead of holding up the wave in a burst
        fetch(x + 1);
        ta_f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
        // the two 32-key halves one after the other, so that the softmax of
        // the first half runs while the products of the second are in the pipe
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int c = 0; c < TA_D / 16; ++c) {
                const ta_bf16x8 kf = ta_as_bf16x8(*(const u32x4*)(sk + koff[c] + kb * 32 * TA_D));
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
            }
        }
        // LDS reads run two products ahead
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);          // 4 LDS reads
#pragma unroll
        for (int c = 0; c < TA_D / 16; ++c) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // 2 MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      // 1 global load
            if (c < TA_D / 16 - 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        // online softmax and the value product per 32-key half
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!pre) {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (!((mw[kb] >> (16 * (j >> 3) + (j & 7))) & 1u)) s[kb][j] = -INFINITY;
            } else if (base + TA_KB > L) {
                const int lim = L - base - 8 * hh;
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (32 * kb + 16 * (j >> 3) + (j & 7) >= lim) s[kb][j] = -INFINITY;
            }
            // maximum of the row over the half (both lane halves)
            float bm = s[kb][0];
#pragma unroll
            for (int j = 1; j < 16; ++j) bm = fmaxf(bm, s[kb][j]);
            // the other lane half: the swap hands each lane its partner's value
            // in one of the two results and its own in the other
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false, false);
            bm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
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
            float ps[4] = {0.f, 0.f, 0.f, 0.f};
            ta_bf16x8 pf[2];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][j], sl2, nm));
                ps[j & 3] += p;
                pf[j >> 3][j & 7] = (__bf16)p;
            }
            lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
            // O^T += V^T P^T over the half's 16-key chunks q (groups 2q and
            // 2q + 1); tile t covers dims 32t .. 32t + 31, and dim 32t + rl
            // sits 8*34*t further
#pragma unroll
            for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                for (int t = 0; t < TA_D / 32; ++t) {
                    const int q = 2 * kb + qq;
                    const ta_bf16x8 vf = ta_as_bf16x8(*(const u32x4*)(sv + voff + 2 * q * TA_VG + 8 * 34 * t));
                    o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qq], o[t], 0, 0, 0);
                }
        }
    };

    // this workgroup's key blocks: split sp of the blocks (all of them with
    // one split); an empty range leaves the partial at no weight
    const int x0 = sp * a.spb, x1 = min(nblk, x0 + a.spb);
    if (x0 < x1) {
        fetch(x0);
        stage(x0, 0);
    }
    __syncthreads();
    // compute(x) also loads block x + 1 (past the last block every key is
    // invalid and reads a valid row, so the final extra loads stay in bounds)
    for (int x = x0; x < x1; x += 2) {
        // two blocks per trip so that the buffer offsets are constants
        if (wave_live) compute(x, 0);
        else fetch(x + 1);
        if (x + 1 < x1) stage(x + 1, 1);
        __syncthreads();
        if (x + 1 >= x1) break;
        if (wave_live) compute(x + 1, 1);
        else fetch(x + 2);
        if (x + 2 < x1) stage(x + 2, 0);
        __syncthreads();
    }

    // normalise by the row's weight total (both lane halves); accumulator j of
    // tile t is dim 32t + 8*(j/4) + 4*hh + j%4 of the lane's row
    {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
        lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const int i = row / G, hq = g * G + (row - (row / G) * G);
    if (a.splits > 1) {
        // this split's share: outputs against the running maximum, unscaled
        if (live) {
            const size_t prow = (((size_t)sp * (a.groups / Hkv) + b) * P + i) * Hq + hq;
            float* dst = a.po + prow * TA_D + 4 * hh;
#pragma unroll
            for (int t = 0; t < TA_D / 32; ++t)
#pragma unroll
                for (int jq = 0; jq < 4; ++jq)
                    *(float4*)(dst + 32 * t + 8 * jq) =
                        make_float4(o[t][4 * jq], o[t][4 * jq + 1], o[t][4 * jq + 2], o[t][4 * jq + 3]);
            if (hh == 0) *(float2*)(a.pml + 2 * prow) = make_float2(mrun, lsum);
        }
        return;
    }
    if (row < RT) {
        const float inv = live && lsum > 0.f ? 1.f / lsum : 0.f;
        float* dst = a.out + (((size_t)b * P + i) * Hq + hq) * TA_D + 4 * hh;
#pragma unroll
        for (int t = 0; t < TA_D / 32; ++t)
#pragma unroll
            for (int jq = 0; jq < 4; ++jq)
                *(float4*)(dst + 32 * t + 8 * jq) =
                    make_float4(o[t][4 * jq] * inv, o[t][4 * jq + 1] * inv, o[t][4 * jq + 2] * inv, o[t][4 * jq + 3] * inv);
    }
}

// Combination of the splits: 32 lanes per output row (request, flat
// position, query head), four dims per lane.  With m_s and l_s the running
// maximum and weight total of split s and o_s its unnormalised output, all
// against 2^(sl2 * (score - m_s)), the row is
//   sum_s 2^(sl2 (m_s - M)) o_s / sum_s 2^(sl2 (m_s - M)) l_s,  M = max_s m_s.
// Positions past the request's m are written as 0.
#define TA_CNT 256
#define TA_CROWS (TA_CNT / 32)          // rows per workgroup
__global__ __launch_bounds__(TA_CNT) void k_attn_combine(AttnArgs a) {
    const int lane = threadIdx.x & 31;
    const int B = a.groups / a.Hkv, P = a.P, Hq = a.Hq;
    const long long rows = (long long)B * P * Hq;
    const long long r = (long long)blockIdx.x * TA_CROWS + (threadIdx.x >> 5);
    if (r >= rows) return;
    const int b = (int)(r / ((long long)P * Hq));
    const int i = (int)((r / Hq) % P);
    const int n = min(max(a.m[b], 0), P - 1) + 1;
    float4 res = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < n) {
        const size_t split_rows = (size_t)rows;
        float M = TA_MFLOOR;
#pragma unroll 4
        for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.pml[2 * (s * split_rows + r)]);
        float den = 0.f;
        float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
        for (int s = 0; s < a.splits; ++s) {
            const float2 ml = *(const float2*)(a.pml + 2 * (s * split_rows + r));
            const float w = __builtin_amdgcn_exp2f((ml.x - M) * a.sl2);
            const float4 os = *(const float4*)(a.po + (s * split_rows + r) * TA_D + 4 * lane);
            den = fmaf(w, ml.y, den);
            num.x = fmaf(w, os.x, num.x);
            num.y = fmaf(w, os.y, num.y);
            num.z = fmaf(w, os.z, num.z);
            num.w = fmaf(w, os.w, num.w);
        }
        const float inv = den > 0.f ? 1.f / den : 0.f;
        res = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
    }
    *(float4*)(a.out + (size_t)r * TA_D + 4 * lane) = res;
}

void ddt_attention_launch(const AttnArgs& a, unsigned grid, hipStream_t stream) {
    hipLaunchKernelGGL(k_tree_attention, dim3(grid), dim3(TA_NT), 0, stream, a);
    if (a.splits > 1) {
        const long long rows = (long long)(a.groups / a.Hkv) * a.P * a.Hq;
        const unsigned cg = (unsigned)((rows + TA_CROWS - 1) / TA_CROWS);
        hipLaunchKernelGGL(k_attn_combine, dim3(cg), dim3(TA_CNT), 0, stream, a);
    }
}
