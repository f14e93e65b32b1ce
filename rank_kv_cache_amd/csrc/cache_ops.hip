// cache_ops.hip -- cache maintenance kernels (gfx950): append new tokens' latents (Zhou, STAR-KV
// reading notes, Algorithm 2 steps 1-3) and read cached tokens back in token-major order.
//
// Layouts: token-major rows [B][cap][C] for key latents and for dense K/V; channel-major 64-token
// blocks [B][cap/64][C][64] for the joint value latent. The block transposes go through LDS so
// that both the row side and the block side are accessed with coalesced loads and stores.

#include "common.hpp"

namespace starkv {

// Copy one contiguous byte range per sequence (row-major side of append and read-back).
__global__ __launch_bounds__(256) void copy_rows(const RowCopyParams p) {
    const int b = blockIdx.y;
    const long long n16 = p.bytes / 16;
    const u32x4* s = reinterpret_cast<const u32x4*>(p.src + b * p.src_seq_stride + p.src_off);
    u32x4* d = reinterpret_cast<u32x4*>(p.dst + b * p.dst_seq_stride + p.dst_off);
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long long)gridDim.x * 256)
        d[i] = s[i];
}

// Row <-> block transpose of the value latent, one (64-token block, 64-channel chunk) per
// workgroup.
template <typename E>
__global__ __launch_bounds__(256) void block_transpose(const BlockXposeParams p) {
    __shared__ E tile[64][65];
    const int blk = p.blk_first + blockIdx.x;
    const int c0 = blockIdx.y * 64;
    const int b = blockIdx.z;
    const long long tb = (long long)blk * 64;
    const size_t nblk = (size_t)p.cap / 64;
    const E* src = static_cast<const E*>(p.src);
    E* dst = static_cast<E*>(p.dst);
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    if (p.to_blocks) {
        for (int r = ty; r < 64; r += 4) {             // r: token in block, tx: channel
            const long long t = tb + r;
            const int c = c0 + tx;
            if (t >= p.t_begin && t < p.t_end && c < p.C)
                tile[r][tx] = src[((size_t)b * p.rows_per_seq + (t - p.row0)) * p.C + c];
        }
        __syncthreads();
        for (int r = ty; r < 64; r += 4) {             // r: channel in chunk, tx: token in block
            const long long t = tb + tx;
            const int c = c0 + r;
            if (t >= p.t_begin && t < p.t_end && c < p.C)
                dst[(((size_t)b * nblk + blk) * p.C + c) * 64 + tx] = tile[tx][r];
        }
    } else {
        for (int r = ty; r < 64; r += 4) {             // r: channel, tx: token in block
            const long long t = tb + tx;
            const int c = c0 + r;
            if (t >= p.t_begin && t < p.t_end && c < p.C)
                tile[tx][r] = src[(((size_t)b * nblk + blk) * p.C + c) * 64 + tx];
        }
        __syncthreads();
        for (int r = ty; r < 64; r += 4) {             // r: token, tx: channel
            const long long t = tb + r;
            const int c = c0 + tx;
            if (t >= p.t_begin && t < p.t_end && c < p.C)
                dst[((size_t)b * p.rows_per_seq + (t - p.row0)) * p.C + c] = tile[r][tx];
        }
    }
}

hipError_t launch_copy_rows(const RowCopyParams& p, int B, hipStream_t st) {
    const long long n16 = p.bytes / 16;
    long long blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(copy_rows, dim3((unsigned)blocks, B), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_block_transpose(const BlockXposeParams& p, int elem_bytes, hipStream_t st) {
    if (p.t_end <= p.t_begin) return hipSuccess;
    const int blk_last = (int)((p.t_end - 1) / 64);
    const dim3 grid(blk_last - p.blk_first + 1, (p.C + 63) / 64, p.B);
    if (elem_bytes == 2)
        hipLaunchKernelGGL(block_transpose<uint16_t>, grid, dim3(256), 0, st, p);
    else if (elem_bytes == 4)
        hipLaunchKernelGGL(block_transpose<uint32_t>, grid, dim3(256), 0, st, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace starkv
