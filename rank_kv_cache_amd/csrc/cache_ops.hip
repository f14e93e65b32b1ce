// cache_ops.hip -- cache maintenance kernels (gfx950): append new tokens' latents (Zhou, STAR-KV
// reading notes, Algorithm 2 steps 1-3) and read cached tokens back in token-major order.
//
// Layouts: token-major rows [B][cap][H*d] for dense K/V; 64-token blocks of 16-channel groups for
// the latents (key: token-major inside a group, value: 16-token runs per channel inside a group;
// see zk_block_at / zv_block_at). The block transposes go through LDS so that both the row
// side and the block side are accessed in order.

#include "common.hpp"

namespace starkv {

// Copy one contiguous byte range per sequence (row-major side of append and read-back).
__global__ __launch_bounds__(256) void copy_rows(const RowCopyParams p) {
    const int b = blockIdx.y;
    const long long n16 = p.bytes / 16;
    long long dst_off = p.dst_off;
    if (p.positions) {
        const long long pb = p.positions[b];
        if (pb < 0 || pb >= p.pos_limit) return;
        dst_off += (p.pos_mod ? pb % p.pos_mod : pb) * p.bytes;
    }
    const u32x4* s = reinterpret_cast<const u32x4*>(p.src + b * p.src_seq_stride + p.src_off);
    u32x4* d = reinterpret_cast<u32x4*>(p.dst + b * p.dst_seq_stride + dst_off);
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long long)gridDim.x * 256)
        d[i] = s[i];
}

// Token-major rows <-> block layout (key or value latent), one (64-token block, 64-channel chunk,
// sequence) per workgroup, staged through an LDS tile so both sides are accessed in order.
// FR (blocks -> rows only): the rows side is in MFMA fragment order instead, 32-token tiles of
// 8-channel runs: element (row r, channel c) of sequence b at
// (((b * rows_per_seq / 32 + r / 32) * C / 8 + c / 8) * 32 + r % 32) * 8 + c % 8
// (rows_per_seq a multiple of 32), so eight channels of one token are one 16-byte unit and the
// 32 tokens of a tile are 512 contiguous bytes.
template <typename E, bool FR>
__global__ __launch_bounds__(256) void block_transpose(const BlockXposeParams p) {
    __shared__ E tile[64][65];                        // [token in block][channel in chunk]
    const int blk = p.blk_first + blockIdx.x;
    const int c0 = blockIdx.y * 64;
    const int b = blockIdx.z;
    const long long tb = (long long)blk * 64;
    const E* src = static_cast<const E*>(p.src);
    E* dst = static_cast<E*>(p.dst);
    const int ncg = min(64, p.C - c0) >> 4;            // 16-channel groups in this chunk
    const size_t gbase = block_id(p.pages, p.nblk_cap, b, blk) * (size_t)(p.C >> 4) + (size_t)(c0 >> 4);
    // element e of the chunk's contiguous block-layout range -> (token, channel)
    auto decode = [&](int e, int* tok, int* ch) {
        const int gl = e >> 10, w = e & 1023;
        if (p.layout == 0) {                          // [t][k]
            *tok = w >> 4;
            *ch = 16 * gl + (w & 15);
        } else {                                      // [u][k][v]
            *tok = 16 * (w >> 8) + (w & 15);
            *ch = 16 * gl + ((w >> 4) & 15);
        }
    };
    if (p.to_blocks) {
        for (int e = threadIdx.x; e < 64 * 64; e += 256) {
            const int r = e >> 6, cc = e & 63;          // r: token in block, cc: channel
            const long long t = tb + r;
            if (t >= p.t_begin && t < p.t_end && c0 + cc < p.C)
                tile[r][cc] = src[((size_t)b * p.rows_per_seq + (t - p.row0)) * p.C + c0 + cc];
        }
        __syncthreads();
        for (int e = threadIdx.x; e < ncg * 1024; e += 256) {
            int tok, ch;
            decode(e, &tok, &ch);
            const long long t = tb + tok;
            if (t >= p.t_begin && t < p.t_end) dst[gbase * 1024 + e] = tile[tok][ch];
        }
    } else {
        // this sequence's end (a ragged prefill reads each sequence only up to its own fill)
        const long long t_end = p.chunk_lens
            ? min(p.t_end, p.pos0 + (long long)min(max(p.chunk_lens[b], 0), p.chunk)) : p.t_end;
        if (tb >= t_end) return;                       // uniform: the whole block is past the end
        for (int e = threadIdx.x; e < ncg * 1024; e += 256) {
            int tok, ch;
            decode(e, &tok, &ch);
            const long long t = tb + tok;
            if (t >= p.t_begin && t < t_end) tile[tok][ch] = src[gbase * 1024 + e];
        }
        __syncthreads();
        if constexpr (FR) {
            // thread per (8-channel run, token): consecutive threads write consecutive 16-byte units
            struct __attribute__((aligned(8 * sizeof(E)))) Run { E v[8]; };
            for (int e = threadIdx.x; e < 64 * 8; e += 256) {
                const int r = (e & 31) + 32 * ((e >> 5) & 1), qq = e >> 6;
                const long long t = tb + r;
                if (t >= p.t_begin && t < t_end && c0 + 8 * qq < p.C) {
                    Run v;
#pragma unroll
                    for (int k = 0; k < 8; ++k) v.v[k] = tile[r][8 * qq + k];
                    const long long rr = t - p.row0;
                    reinterpret_cast<Run*>(dst)[(((size_t)b * (p.rows_per_seq >> 5) + (rr >> 5)) * (p.C >> 3) +
                                                 ((c0 >> 3) + qq)) * 32 + (rr & 31)] = v;
                }
            }
        } else {
            for (int e = threadIdx.x; e < 64 * 64; e += 256) {
                const int r = e >> 6, cc = e & 63;
                const long long t = tb + r;
                if (t >= p.t_begin && t < t_end && c0 + cc < p.C)
                    dst[((size_t)b * p.rows_per_seq + (t - p.row0)) * p.C + c0 + cc] = tile[r][cc];
            }
        }
    }
}

// Append of a few tokens to both latents in one launch: thread per (sequence, token, run of 8
// channels). A run is contiguous in the key layout (one vector store) and strided by 16 elements
// in the value layout.
template <typename E>
__global__ __launch_bounds__(256) void append_small(const AppendSmallParams p) {
    struct __attribute__((aligned(16))) Run { E v[8]; };
    const int runs_k = p.Rk >> 3, runs_v = p.rv >> 3;
    const long long per_tok = runs_k + runs_v;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.B * p.n * per_tok) return;
    const int run = (int)(idx % per_tok);
    const long long bt = idx / per_tok;
    const int t = (int)(bt % p.n);
    const int b = (int)(bt / p.n);
    const long long tok = p.positions ? (long long)p.positions[b] : p.pos + t;
    if (p.positions && (tok < 0 || tok >= (long long)p.nblk_cap * 64)) return;
    if (run < runs_k) {
        const int c = run * 8;
        const Run v = *reinterpret_cast<const Run*>(static_cast<const E*>(p.zk_src) + (bt * p.Rk + c));
        *reinterpret_cast<Run*>(static_cast<E*>(p.zk) + zk_block_at(block_id(p.pages, p.nblk_cap, b, tok >> 6), p.Rk, tok, c)) = v;
    } else {
        const int c = (run - runs_k) * 8;
        const Run v = *reinterpret_cast<const Run*>(static_cast<const E*>(p.zv_src) + (bt * p.rv + c));
        E* dst = static_cast<E*>(p.zv);
        const size_t id = block_id(p.pages, p.nblk_cap, b, tok >> 6);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[zv_block_at(id, p.rv, tok, c + e)] = v.v[e];
    }
}

// Latents whose ranks were rounded up to the 16-channel tile. Thread per (sequence, row, channel):
// channels of the stored width when writing the cache (padding channels get zero, so that the
// zero factor rows they meet never multiply stale memory), caller channels when reading back.
template <typename E>
__global__ __launch_bounds__(256) void padded_rows(const PaddedRowsParams p) {
    const int C = p.to_cache ? p.C : p.C_src;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.B * p.n * C) return;
    const int c = (int)(idx % C);
    const long long bt = idx / C;
    const long long row = bt % p.n;
    const int b = (int)(bt / p.n);
    const long long tok = p.positions ? (long long)p.positions[b] : p.t0 + row;
    if (p.positions && (tok < 0 || tok >= (long long)p.nblk_cap * 64)) return;
    E* cache = static_cast<E*>(p.cache);
    if (p.to_cache) {
        const int cs = p.which ? (c < p.C_src ? c : -1) : src_key_channel(p.map, c);
        const E v = cs >= 0 ? static_cast<const E*>(p.rows)[bt * p.C_src + cs] : E(0);
        const size_t id = block_id(p.pages, p.nblk_cap, b, tok >> 6);
        cache[p.which ? zv_block_at(id, p.C, tok, c) : zk_block_at(id, p.C, tok, c)] = v;
    } else {
        const int cc = p.which ? c : pad_key_channel(p.map, c);
        static_cast<E*>(const_cast<void*>(p.rows))[bt * p.C_src + c] =
            cache[p.which ? zv_block_at(block_id(p.pages, p.nblk_cap, b, tok >> 6), p.C, tok, cc)
                          : zk_block_at(block_id(p.pages, p.nblk_cap, b, tok >> 6), p.C, tok, cc)];
    }
}

hipError_t launch_padded_rows(const PaddedRowsParams& p, int elem_bytes, hipStream_t st) {
    const long long n = (long long)p.B * p.n * (p.to_cache ? p.C : p.C_src);
    if (n <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (elem_bytes == 2)
        hipLaunchKernelGGL(padded_rows<uint16_t>, grid, dim3(256), 0, st, p);
    else if (elem_bytes == 4)
        hipLaunchKernelGGL(padded_rows<uint32_t>, grid, dim3(256), 0, st, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// Rows of a paged dense cache: thread per 16 bytes of a (sequence, row); each token's row lives in
// its block's page.
__global__ __launch_bounds__(256) void paged_rows(const PagedRowsParams p) {
    const long long per_row = p.row_bytes / 16;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.B * p.n * per_row) return;
    const long long chunk = idx % per_row;
    const long long br = idx / per_row;
    const long long row = br % p.n;
    const int b = (int)(br / p.n);
    const long long tok = p.positions ? (long long)p.positions[b] : p.t0 + row;
    if (p.positions && (tok < 0 || tok >= (long long)p.nblk_cap * 64)) return;
    u32x4* c = reinterpret_cast<u32x4*>(p.cache + (block_id(p.pages, p.nblk_cap, b, tok >> 6) * 64 + (tok & 63)) * p.row_bytes) + chunk;
    u32x4* r = reinterpret_cast<u32x4*>(const_cast<char*>(p.rows) + br * p.row_bytes) + chunk;
    if (p.to_cache)
        *c = *r;
    else
        *r = *c;
}

hipError_t launch_paged_rows(const PagedRowsParams& p, hipStream_t st) {
    const long long n = (long long)p.B * p.n * (p.row_bytes / 16);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(paged_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_append_small(const AppendSmallParams& p, int elem_bytes, hipStream_t st) {
    const long long n = (long long)p.B * p.n * ((p.Rk + p.rv) / 8);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (elem_bytes == 2)
        hipLaunchKernelGGL(append_small<uint16_t>, grid, dim3(256), 0, st, p);
    else if (elem_bytes == 4)
        hipLaunchKernelGGL(append_small<uint32_t>, grid, dim3(256), 0, st, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_copy_rows(const RowCopyParams& p, int B, hipStream_t st) {
    const long long n16 = p.bytes / 16;
    long long blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(copy_rows, dim3((unsigned)blocks, B), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_block_transpose(const BlockXposeParams& p, int elem_bytes, hipStream_t st, bool frag_rows) {
    if (p.t_end <= p.t_begin) return hipSuccess;
    if (frag_rows && (p.to_blocks || elem_bytes != 2 || (p.rows_per_seq & 31) || (p.row0 & 31) || (p.C & 7)))
        return hipErrorInvalidValue;
    const int blk_last = (int)((p.t_end - 1) / 64);
    const dim3 grid(blk_last - p.blk_first + 1, (p.C + 63) / 64, p.B);
    if (frag_rows)
        hipLaunchKernelGGL((block_transpose<uint16_t, true>), grid, dim3(256), 0, st, p);
    else if (elem_bytes == 2)
        hipLaunchKernelGGL((block_transpose<uint16_t, false>), grid, dim3(256), 0, st, p);
    else if (elem_bytes == 4)
        hipLaunchKernelGGL((block_transpose<uint32_t, false>), grid, dim3(256), 0, st, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace starkv
