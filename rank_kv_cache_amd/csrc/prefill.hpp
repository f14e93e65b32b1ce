// prefill.hpp -- parameter blocks of the prefill kernels (prefill.hip), shared with api.cpp.
#pragma once

#include "common.hpp"

namespace starkv {

// Prefill (a chunk of queries per sequence, causal). Query l of sequence b sits at position
// pos0 + l and attends to tokens [0, pos0 + l] when l < chunk_len(b) (else its output row is 0);
// sequence b holds latents for tokens [0, pos0 + chunk_len(b)) (its fill).
//
// Preparation: the keys and values of every 32-token tile, rebuilt once per call from
// token-major latent rows (Zhou notes, Alg. 2 step 4b for the keys; the values per head,
// Z_v B_v^h, section 5.3 reassociated: for a chunk of queries the product with B_v is cheaper
// before the attention sum than after it). Per (sequence, head, tile) a record of 256 * D bytes:
//   keys   [D/16 steps][hi, lo][64 lanes][8] binary16: the A operand of S^T = K Q^T; lane l holds
//          key l % 32 and, for step 2*mt + s, dims 32*mt + 16*s + 8*(e/4) + 4*(l/32) + e%4
//          (e < 8), rotated to the key's position and scaled by 2^kexp;
//   values [D/32 tiles][2 steps][hi, lo][64 lanes][8] binary16: the A operand of O^T = V^T P^T;
//          lane l of tile n, step t holds dim 32*n + l % 32 of keys 16*t + 8*(e/4) + 4*(l/32) +
//          e%4, scaled by 2^vexp;
// and exps [2] (kexp, vexp) per record. Tokens at or past the sequence's fill are zero.
struct PrefillKVParams {
    // latent rows (storage type; the layer's channel layout) of Tr = 32 * ntiles rows per sequence,
    // in fragment order: (row r, channel c) of sequence b at
    // (((b * ntiles + r / 32) * C / 8 + c / 8) * 32 + r % 32) * 8 + c % 8, C = Rk or rv
    const void* zk_rows;   // unused when zk_cache is set
    const void* zv_rows;
    // 16-bit caches: the key latents are read straight from the cache's block layout
    // zk[block][R_k/16][64][16] (block = the pages' block of (b, token / 64)), where eight ranks of
    // a token are already one 16-byte unit and the 32 tokens of a tile 1 KB; NULL: from zk_rows
    const void* zk_cache = nullptr;
    BlockMap pages;
    int nblk_cap = 0;
    const void* bk;        // key factors [R_k caller rows][D]
    const void* bv;        // value factor [rv_src][H*D]
    void* bvf;             // [H][rv/16][D/32][64][8]: B_v in B-operand fragment order (written here)
    void* kv;              // [B][H][ntiles] records
    int32_t* exps;         // [B][H][ntiles][2]
    const int32_t* chunk_lens = nullptr;  // per-sequence chunk lengths (device) or NULL
    int B, H, D, Rk, rv, rv_src, Tr, ntiles, chunk, pos0;
    int16_t koff[kMaxHeads + 1];
    int16_t rank[kMaxHeads];
    int16_t soff[kMaxHeads + 1];
    int16_t srank[kMaxHeads];
    double rope_rev[64];   // theta_i / (2 pi)
};

// Attention over the prepared records, 32 queries per wave, online softmax per query.
struct PrefillFlashParams {
    const float* q;        // [B][chunk][H][D], rotated to each query's position
    float* out;            // [B][chunk][H][D]
    const void* kv;        // records as above
    const int32_t* exps;
    const int32_t* chunk_lens = nullptr;
    int B, H, D, chunk, pos0, ntiles;
    float q_scale;         // softmax scale * log2(e)
};

}  // namespace starkv
