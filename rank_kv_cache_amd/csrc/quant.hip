// quant.hip -- mixed 4/3-bit latent cache (gfx950): quantise whole 64-token groups on append and
// read them back (Zhou, STAR-KV reading notes, section 6.1 and Algorithm 2 step 3: the new
// token's latents are quantised, then appended; low-rank-aware mixed precision keeps the leading
// channels of each latent at 4 bits and the rest at 3 bits).
//
// Per (channel, 64-token group), asymmetric with a binary16 scale and zero point:
//   s = (max - min) / (2^bits - 1) in fp32, s16 = binary16(s) (0 when max == min),
//   z16 = binary16(min) (a zero is stored as +0),
//   q = 0 if s16 == 0, else clamp(rint_even((x - z16) / s16), 0, 2^bits - 1), fp32 arithmetic,
//   x^ = binary16(q * s16 + z16), the exact value rounded once (one fp16 FMA).
//
// Code layouts of one 64-token block (bytes per block: Q43Layout::block_bytes):
//  * key latent (token-major, consumed as MFMA operands of eight channels of one token): 16-channel
//    groups, group g at byte goff[g], holding 64 rows of 48 + n bits (n = gn[g] = 4-bit channels
//    at the start of the group); row t starts at bit t * (48 + n) of the group; in a row, bits
//    3e .. 3e+2 are the low three bits of channel e, and bit 48 + e the fourth bit of channel
//    e < n. Bits are little-endian in little-endian 32-bit words.
//  * value latent (channel-major, consumed as operands of eight tokens of one channel): channel c
//    at byte 32c (4-bit, c < n_hi) or 32 n_hi + 24 (c - n_hi) (3-bit), in 32-bit words whose low
//    16 bits hold the even tokens of the word's span and whose high 16 bits hold the odd tokens,
//    so that tokens 2i and 2i+1 sit 16 bits apart (one AND-OR then yields both halves of a packed
//    binary16 pair). 4-bit run: word t/8, bit 16(t%2) + 4((t/2)%4); 3-bit run: words 0..3 the low
//    two bits (word t/16, bit 16(t%2) + 2((t/2)%8)), words 4..5 the third bit (word 4 + t/32,
//    bit 16(t%2) + (t/2)%16).
//  * meta [B][cap/64][2][C] binary16: per block a row of scales, then a row of zero points (so
//    that the scales, and the zero points, of neighbouring channels pair up in one word);
//    tail [B][64][C] binary16 holds the rows of the unfinished group.

#include "common.hpp"

namespace starkv {

__device__ __forceinline__ uint16_t f16_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ __forceinline__ _Float16 bits_f16(uint16_t u) { return __builtin_bit_cast(_Float16, u); }

// Quantiser of one value (see the header comment); IEEE fp32 subtract, divide and rint.
__device__ __forceinline__ int q43_code(_Float16 x, uint16_t s16, uint16_t z16, int qmax) {
    if ((s16 & 0x7fffu) == 0) return 0;
    const float v = ((float)x - (float)bits_f16(z16)) / (float)bits_f16(s16);
    float r = __builtin_rintf(v);
    r = fminf(fmaxf(r, 0.0f), (float)qmax);
    return (int)r;
}

// ------------------------------------------------------------------------------------------------
// Quantise complete groups: workgroup per (group, 64-channel chunk, sequence). The group's 64 rows
// are gathered from the tail (tokens appended by earlier calls) and the new rows.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void q43_quantize(const Q43QuantParams p) {
    __shared__ _Float16 x[64][65];
    __shared__ float s_mn[4][64], s_mx[4][64];
    __shared__ uint16_t s_s[64], s_z[64];
    __shared__ uint8_t code[64][65];
    __shared__ uint32_t words[4][136];

    const Q43Layout& L = p.L;
    const int tid = threadIdx.x;
    const int c0 = blockIdx.y * 64;
    const int b = blockIdx.z;
    int g = p.g_first + blockIdx.x;
    long long pos = p.pos;
    if (p.positions) {                 // one token per sequence: quantise only a completed group
        const long long pb = p.positions[b];
        if (pb < 0 || pb >= (long long)p.nblk_cap * 64 || (pb & 63) != 63) return;
        g = (int)(pb >> 6);
        pos = pb + 1;                  // every row of the group is in the tail
    }
    const int C = L.C;
    const long long tok0 = (long long)g * 64;
    const _Float16* src = static_cast<const _Float16*>(p.src);
    const _Float16* tail = static_cast<const _Float16*>(p.tail);

    for (int e = tid; e < 64 * 64; e += 256) {
        const int t = e >> 6, cc = e & 63, c = c0 + cc;
        const long long tok = tok0 + t;
        _Float16 v = (_Float16)0.0f;
        if (c < C)
            v = tok < pos ? tail[((size_t)b * 64 + t) * C + c]
                          : src[((size_t)b * p.n + (tok - pos)) * C + c];
        x[t][cc] = v;
    }
    __syncthreads();
    {
        const int cc = tid & 63, part = tid >> 6;
        float mn = INFINITY, mx = -INFINITY;
        for (int t = 16 * part; t < 16 * part + 16; ++t) {
            const float v = (float)x[t][cc];
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
        }
        s_mn[part][cc] = mn;
        s_mx[part][cc] = mx;
    }
    __syncthreads();
    if (tid < 64 && c0 + tid < C) {
        const int c = c0 + tid;
        float mn = s_mn[0][tid], mx = s_mx[0][tid];
        for (int k = 1; k < 4; ++k) {
            mn = fminf(mn, s_mn[k][tid]);
            mx = fmaxf(mx, s_mx[k][tid]);
        }
        const int qmax = q43_is_hi(L, c) ? 15 : 7;
        const float diff = mx - mn;
        const uint16_t s16 = diff == 0.0f ? 0 : f16_bits((_Float16)(diff / (float)qmax));
        uint16_t z16 = f16_bits((_Float16)mn);
        if (z16 == 0x8000u) z16 = 0;
        s_s[tid] = s16;
        s_z[tid] = z16;
        uint16_t* meta = static_cast<uint16_t*>(p.meta) + block_id(p.pages, p.nblk_cap, b, g) * 2 * C + c;
        meta[0] = s16;
        meta[C] = z16;
    }
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += 256) {
        const int t = e >> 6, cc = e & 63, c = c0 + cc;
        code[t][cc] = c < C ? (uint8_t)q43_code(x[t][cc], s_s[cc], s_z[cc], q43_is_hi(L, c) ? 15 : 7) : 0;
    }
    __syncthreads();

    uint8_t* blk = static_cast<uint8_t*>(p.codes) + block_id(p.pages, p.nblk_cap, b, g) * L.block_bytes;
    if (!L.is_key) {
        // value latent: thread per channel writes its whole run
        if (tid < 64 && c0 + tid < C) {
            const int c = c0 + tid;
            uint32_t* run = reinterpret_cast<uint32_t*>(blk + q43_value_run_offset(L, c));
            // token k of a word's span: bit 16 * (k & 1) + width * (k >> 1)
            if (q43_is_hi(L, c)) {
                for (int w = 0; w < 8; ++w) {
                    uint32_t v = 0;
                    for (int k = 0; k < 8; ++k) v |= (uint32_t)code[8 * w + k][tid] << (16 * (k & 1) + 4 * (k >> 1));
                    run[w] = v;
                }
            } else {
                for (int w = 0; w < 4; ++w) {
                    uint32_t v = 0;
                    for (int k = 0; k < 16; ++k)
                        v |= (uint32_t)(code[16 * w + k][tid] & 3u) << (16 * (k & 1) + 2 * (k >> 1));
                    run[w] = v;
                }
                for (int w = 0; w < 2; ++w) {
                    uint32_t v = 0;
                    for (int k = 0; k < 32; ++k)
                        v |= (uint32_t)((code[32 * w + k][tid] >> 2) & 1u) << (16 * (k & 1) + (k >> 1));
                    run[4 + w] = v;
                }
            }
        }
        return;
    }
    // key latent: thread (group gl in chunk, token t) ORs its row into an LDS image of the group
    for (int e = tid; e < 4 * 136; e += 256) (&words[0][0])[e] = 0u;
    __syncthreads();
    const int gl = tid >> 6, t = tid & 63;
    const int g16 = (c0 >> 4) + gl;
    const bool gok = c0 + 16 * gl < C;
    int n = 0;
    if (gok) {
        n = L.gn[g16];
        uint64_t row = 0;
        for (int e = 0; e < 16; ++e) {
            const uint32_t q = code[t][16 * gl + e];
            row |= (uint64_t)(q & 7u) << (3 * e);
            if (e < n) row |= (uint64_t)((q >> 3) & 1u) << (48 + e);
        }
        const int bit = t * (48 + n);
        const int w0 = bit >> 5, sh = bit & 31;
        // the row's bits i land at bit sh + i of words w0, w0 + 1, w0 + 2
        atomicOr(&words[gl][w0], (uint32_t)(row << sh));
        atomicOr(&words[gl][w0 + 1], (uint32_t)(row >> (32 - sh)));
        if (sh) atomicOr(&words[gl][w0 + 2], (uint32_t)(row >> (64 - sh)));
    }
    __syncthreads();
    if (gok) {
        const int nwords = (384 + 8 * n) / 4;
        uint32_t* dst = reinterpret_cast<uint32_t*>(blk + L.goff[g16]);
        for (int w = t; w < nwords; w += 64) dst[w] = words[gl][w];
    }
}

// ------------------------------------------------------------------------------------------------
// Read-back: rows [t0, t1) of a latent as binary16, thread per (sequence, token, 8 channels).
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ int q43_key_code(const uint8_t* blk, const Q43Layout& L, int c, int t) {
    const int g16 = c >> 4, e = c & 15, n = L.gn[g16];
    const uint8_t* gb = blk + L.goff[g16];
    const int rowbit = t * (48 + n);
    auto bit = [&](int i) -> uint32_t { return (gb[i >> 3] >> (i & 7)) & 1u; };
    uint32_t q = bit(rowbit + 3 * e) | (bit(rowbit + 3 * e + 1) << 1) | (bit(rowbit + 3 * e + 2) << 2);
    if (e < n) q |= bit(rowbit + 48 + e) << 3;
    return (int)q;
}

__device__ __forceinline__ int q43_value_code(const uint8_t* blk, const Q43Layout& L, int c, int t) {
    const uint32_t* run = reinterpret_cast<const uint32_t*>(blk + q43_value_run_offset(L, c));
    const int odd = 16 * (t & 1);
    if (q43_is_hi(L, c)) return (run[t >> 3] >> (odd + 4 * ((t >> 1) & 3))) & 15;
    return ((run[t >> 4] >> (odd + 2 * ((t >> 1) & 7))) & 3) | (((run[4 + (t >> 5)] >> (odd + ((t >> 1) & 15))) & 1) << 2);
}

__device__ __forceinline__ _Float16 q43_dequant(int q, uint16_t s16, uint16_t z16) {
    return __builtin_fmaf16((_Float16)q, bits_f16(s16), bits_f16(z16));
}

// FR: rows in MFMA fragment order (32-token tiles of 8-channel runs, as block_transpose writes
// them for prefill), t1 - t0 rounded up to 32 rows per sequence; else token-major [B][t1 - t0][C].
template <bool FR>
__global__ __launch_bounds__(256) void q43_readback(const Q43ReadParams p) {
    const Q43Layout& L = p.L;
    const int runs = L.C >> 3;
    const long long n = p.t1 - p.t0;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.B * n * runs) return;
    const int run = (int)(idx % runs);
    const long long bt = idx / runs;
    const long long tok = p.t0 + bt % n;
    const int b = (int)(bt / n);
    const int c = run * 8;
    long long full = p.full_tokens;
    if (p.chunk_lens) {
        // this sequence's end: rows past it are not written, and none of its codes past it read
        const long long end = p.pos0 + min(max(p.chunk_lens[b], 0), p.chunk);
        if (tok >= end) return;
        full = end >> 6 << 6;
    }
    _Float16 v[8];
    if (tok < full) {
        const int g = (int)(tok >> 6), t = (int)(tok & 63);
        const size_t bid = block_id(p.pages, p.nblk_cap, b, g);
        const uint8_t* blk = static_cast<const uint8_t*>(p.codes) + bid * L.block_bytes;
        const uint16_t* meta = static_cast<const uint16_t*>(p.meta) + bid * 2 * L.C + c;
        for (int e = 0; e < 8; ++e) {
            const int q = L.is_key ? q43_key_code(blk, L, c + e, t) : q43_value_code(blk, L, c + e, t);
            v[e] = q43_dequant(q, meta[e], meta[L.C + e]);
        }
    } else {
        const _Float16* tail = static_cast<const _Float16*>(p.tail) + ((size_t)b * 64 + (tok & 63)) * L.C + c;
        for (int e = 0; e < 8; ++e) v[e] = tail[e];
    }
    if constexpr (FR) {
        struct __attribute__((aligned(16))) Run { _Float16 v[8]; } r;
        for (int e = 0; e < 8; ++e) r.v[e] = v[e];
        const long long rr = tok - p.t0, tiles = (n + 31) >> 5;
        reinterpret_cast<Run*>(p.out)[(((size_t)b * tiles + (rr >> 5)) * runs + run) * 32 + (rr & 31)] = r;
    } else {
        _Float16* dst = static_cast<_Float16*>(p.out) + (size_t)bt * L.C + c;
        for (int e = 0; e < 8; ++e) dst[e] = v[e];
    }
}

// ------------------------------------------------------------------------------------------------
// Offline preparation: blockwise Hadamard rotation (Zhou notes, section 6.1 / Fig. 5), binary16 in
// and out. Output element = binary16(fp64(exact signed sum of the b inputs) * fp64(1 / sqrt(b))):
// the sum of at most 64 binary16 values is exact in fp64 (each is an integer multiple of 2^-24 below
// 2^16), so only the product and the final conversion round.
// ------------------------------------------------------------------------------------------------

// binary64 -> binary16, round to nearest, ties to even (IEEE 754 conversion, written out on bits).
__device__ __forceinline__ uint16_t f64_to_f16_rne(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const int e = (int)((u >> 52) & 0x7ff);
    uint64_t m = u & ((1ull << 52) - 1);
    if (e == 0x7ff) return sign | (m ? 0x7e00u : 0x7c00u);          // NaN, infinity
    if (e == 0) return sign;                                           // fp64 subnormals -> 0
    const int E = e - 1023;                                            // unbiased exponent
    if (E > 15) return sign | 0x7c00u;                                  // overflow
    m |= 1ull << 52;                                                   // significand, 53 bits
    // binary16 keeps 11 significant bits for normals (E >= -14); fewer below, down to 2^-24
    const int shift = (E >= -14) ? 42 : 42 + (-14 - E);
    if (shift > 53) return sign;                                        // below half of 2^-24
    const uint64_t q = m >> shift;
    const uint64_t rem = m & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    uint64_t r = q + ((rem > half || (rem == half && (q & 1))) ? 1 : 0);
    uint32_t bits;
    if (E >= -14) {
        // r in [2^10, 2^11]; a carry to 2^11 moves to the next binade
        int ee = E + 15;
        if (r == (1ull << 11)) { r >>= 1; ++ee; }
        if (ee >= 31) return sign | 0x7c00u;
        bits = ((uint32_t)ee << 10) | (uint32_t)(r & 0x3ff);
    } else {
        bits = (uint32_t)r;                                            // subnormal (or 2^-14 on carry)
    }
    return sign | (uint16_t)bits;
}

__global__ __launch_bounds__(256) void hadamard_rotate(const HadamardParams p) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= p.n * p.C) return;
    // kind 0: element (row, c) = idx / C, idx % C; kind 1: (c, col) = idx / n, idx % n
    const long long outer = p.kind == 0 ? idx / p.C : idx / p.n;
    const long long inner = p.kind == 0 ? idx % p.C : idx % p.n;
    const int c = (int)(p.kind == 0 ? inner : outer);
    int g = 0;
    while (g + 1 < p.nseg && c >= p.seg_start[g + 1]) ++g;
    const int s0 = p.seg_start[g], b = p.seg_block[g];
    const double inv = p.seg_inv[g];
    const bool in_seg = c >= s0 && c < s0 + p.seg_width[g];
    const size_t out_i = (size_t)idx;
    if (!in_seg) { p.dst[out_i] = p.src[out_i]; return; }
    const int j0 = s0 + ((c - s0) / b) * b, i = c - j0;
    double acc = 0.0;
    for (int j = 0; j < b; ++j) {
        const size_t src_i = p.kind == 0 ? (size_t)outer * p.C + (size_t)(j0 + j)
                                         : (size_t)(j0 + j) * (size_t)p.n + (size_t)inner;
        const double v = (double)bits_f16(p.src[src_i]);
        acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -v : v;
    }
    p.dst[out_i] = f64_to_f16_rne(acc * inv);
}

hipError_t launch_hadamard_rotate(const HadamardParams& p, hipStream_t st) {
    const long long total = p.n * p.C;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(hadamard_rotate, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_q43_quantize(const Q43QuantParams& p, int ngroups, hipStream_t st) {
    if (ngroups <= 0) return hipSuccess;
    const dim3 grid(ngroups, (p.L.C + 63) / 64, p.B);
    hipLaunchKernelGGL(q43_quantize, grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_q43_readback(const Q43ReadParams& p, hipStream_t st, bool frag_rows) {
    const long long n = (long long)p.B * (p.t1 - p.t0) * (p.L.C / 8);
    if (n <= 0) return hipSuccess;
    if (frag_rows)
        hipLaunchKernelGGL(q43_readback<true>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL(q43_readback<false>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace starkv
