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
// transposed in groups of 8 keys.  Every global load instruction of a wave
// reads 4 whole 256-byte key rows, 64 contiguous bytes per quad of lanes.
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

// The kernel lives in its own translation unit (ddt_attention.hip), built
// with NaNs assumed absent and the IEEE mode off, so that the float maxima of
// the softmax compile to plain v_max3 with no operand canonicalisation.

typedef __bf16 ta_bf16x8 __attribute__((ext_vector_type(8)));
typedef float ta_f32x16 __attribute__((ext_vector_type(16)));

#define TA_NT 256
#define TA_WR 32                // query rows per wave
#define TA_ROWS 128             // query rows per workgroup
#define TA_KB 64                // keys per block
#define TA_D 128                // head dimension
#define TA_KBUF (TA_KB * TA_D)  // one K buffer, bf16 elements
// V^T in groups of 8 keys: 8 keys of dim d are 16 contiguous bytes at
// 8*(d + d/16) elements into the group (16 bytes of padding after every 16
// dims spread both the transposed writes and the operand reads over the banks)
#define TA_VG (8 * (TA_D + TA_D / 16))
#define TA_VBUF (TA_KB / 8 * TA_VG)     // one V^T buffer
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
    // key splits: split s takes key blocks [s * spb, (s + 1) * spb); with
    // splits > 1 the rows' unnormalised outputs go to po [splits][B][P][Hq][D]
    // and their (running maximum, weight total) to pml [splits][B][P][Hq][2]
    int splits, spb;
    float* po;
    float* pml;
};

__device__ __forceinline__ ta_bf16x8 ta_as_bf16x8(u32x4 v) { return __builtin_bit_cast(ta_bf16x8, v); }

// 16-byte chunk swizzle of K row k: keys that one read phase touches (k and
// k + 4, k + 8, k + 12 within 16) land on different chunks
__device__ __forceinline__ int ta_kswz(int k) { return (k & 3) | ((k >> 1) & 4) | ((k << 1) & 8); }

// Launches k_tree_attention on grid workgroups of TA_NT threads, then, with
// more than one split, the combination of the splits' partials into out.
void ddt_attention_launch(const AttnArgs& a, unsigned grid, hipStream_t stream);
