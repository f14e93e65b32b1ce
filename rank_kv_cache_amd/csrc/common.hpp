// common.hpp -- element traits, MFMA fragment helpers and kernel parameter blocks shared by the
// HIP kernels of the latent-KV decode library and its host planner. gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace starkv {

// ------------------------------------------------------------------------------------------------
// Element types. Storage is F32 (float), F16 (_Float16) or BF16 (raw bits in uint16_t).
// ------------------------------------------------------------------------------------------------
enum ElemKind { kF32 = 0, kF16 = 1, kBF16 = 2 };

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// fp32 -> bf16 bits, nearest-even (finite inputs).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <int K> struct Elem;
template <> struct Elem<kF32> {
    using storage = float;
    using frag = f32x8;                 // 8 consecutive K elements per lane, 32 bytes
    static constexpr int bytes = 4;
};
template <> struct Elem<kF16> {
    using storage = _Float16;
    using frag = f16x8;                 // 16 bytes
    static constexpr int bytes = 2;
};
template <> struct Elem<kBF16> {
    using storage = uint16_t;
    using frag = bf16x8;                // 16 bytes
    static constexpr int bytes = 2;
};

// Load 8 consecutive elements (16-byte aligned for 16-bit types, 32-byte for fp32).
// Latent fragments are streamed once: non-temporal loads keep them from displacing data that is
// re-read (probabilities, block statistics, factor fragments) in the caches.
template <int K>
__device__ __forceinline__ typename Elem<K>::frag load_frag(const void* base, size_t elem_off) {
    using F = typename Elem<K>::frag;
    return __builtin_nontemporal_load(reinterpret_cast<const F*>(static_cast<const char*>(base) + elem_off * Elem<K>::bytes));
}

template <int K>
__device__ __forceinline__ typename Elem<K>::frag zero_frag() {
    typename Elem<K>::frag f;
    for (int i = 0; i < 8; ++i) f[i] = 0;
    return f;
}

// ------------------------------------------------------------------------------------------------
// 32x32 output tile, K = 16 per step. Operand convention (both operands): lane l supplies row
// (A) / column (B) l % 32 and the 8 K-slots 8*(l/32) .. 8*(l/32)+7. The fp16/bf16 forms are one
// v_mfma_f32_32x32x16_{f16,bf16}; the fp32 form issues eight v_mfma_f32_32x32x2_f32, step j
// contracting slot j of both lane halves (K index j and 8+j), which covers the same 16 K values.
// Accumulator: register r of lane l holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
// ------------------------------------------------------------------------------------------------
template <int K>
__device__ __forceinline__ f32x16 mma32(const typename Elem<K>::frag& a,
                                        const typename Elem<K>::frag& b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mma32<kF16>(const f16x8& a, const f16x8& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mma32<kBF16>(const bf16x8& a, const bf16x8& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mma32<kF32>(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Lane exchanges without LDS traffic: DPP inside rows of 16 lanes, permlane swaps across rows.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// (v[lane], v[lane ^ 16]) and (v[lane], v[lane ^ 32]) in some order; op(a, b) of the pair is the
// same in every lane for a commutative op
struct LanePair { float a, b; };
__device__ __forceinline__ LanePair swap16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair swap32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// v + v[lane ^ 32]
__device__ __forceinline__ float add_xor32(float v) {
    const LanePair p = swap32(v);
    return p.a + p.b;
}

// Wave-wide reductions (64 lanes): lane ^ 1, ^ 2 (quad permutations), the other quad of eight
// (half-row mirror), the other eight of sixteen (row mirror), then the row swaps.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    LanePair p = swap16(v);
    v = fmaxf(p.a, p.b);
    p = swap32(v);
    return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    LanePair p = swap16(v);
    v = p.a + p.b;
    p = swap32(v);
    return p.a + p.b;
}
// Reductions over each 32-lane half of the wave (the first five steps of the wave-wide ones):
// every lane gets the result of its own half.
// 2^d for d = m_t - M, the difference of two integer tile maxima (d <= 0, an integer, or -inf
// for a tile with no tokens): exact, where the hardware exp2 is an approximation
__device__ __forceinline__ float tile_factor(float d) {
    return d >= -149.0f ? ldexpf(1.0f, (int)d) : 0.0f;
}

// The maximum runs on integer keys of the float bits (non-negative values keep their bits,
// negative ones have their magnitude bits flipped), which order like the values for every
// non-NaN input including -inf; an integer maximum fuses with the DPP lane move, where a float
// maximum is preceded by a canonicalising operation on each operand.
__device__ __forceinline__ int float_order_key(float v) {
    const int i = __float_as_int(v);
    return i ^ (int)((uint32_t)(i >> 31) >> 1);
}
// v from another lane; the old value is the identity of a signed maximum, so that the move can
// be folded into the maximum that consumes it
template <int CTRL>
__device__ __forceinline__ int dpp_max_src(int v) {
    return __builtin_amdgcn_update_dpp((int)0x80000000, v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float half_max(float x) {
    int v = float_order_key(x);
    v = max(v, dpp_max_src<0xB1>(v));
    v = max(v, dpp_max_src<0x4E>(v));
    v = max(v, dpp_max_src<0x141>(v));
    v = max(v, dpp_max_src<0x140>(v));
    const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    const int m = max((int)r[0], (int)r[1]);
    return __int_as_float(m ^ (int)((uint32_t)(m >> 31) >> 1));   // the key map is its own inverse
}
__device__ __forceinline__ float half_sum(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    const LanePair p = swap16(v);
    return p.a + p.b;
}

// cos and sin of 2*pi*x for x in [0, 1) (hardware v_cos_f32 / v_sin_f32 take revolutions).
__device__ __forceinline__ void sincos_rev(float x, float* c, float* s) {
    *c = __builtin_amdgcn_cosf(x);
    *s = __builtin_amdgcn_sinf(x);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// both 16-bit halves of x shifted right by s
__device__ __forceinline__ uint32_t pk_shr16(uint32_t x, int s) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const u16x2 v = __builtin_bit_cast(u16x2, x) >> (u16x2){(unsigned short)s, (unsigned short)s};
    return __builtin_bit_cast(uint32_t, v);
}

// Eight mixed 4/3-bit key codes of one token (one 16-channel group, channels 8*half .. +7) to an
// fp16 MFMA operand fragment. w0..w2: the aligned 96-bit window holding the token's row, sh: the
// row's first bit in the window, n: 4-bit channels at the start of the group; sc / zc: the scales
// and zero points of the eight channels, two per word. Each value is binary16(q*s + z) rounded
// once (one fp16 FMA per pair); q is formed exactly as binary16(1024 + q) - 1024.
__device__ __forceinline__ f16x8 q43_key_frag(uint32_t w0, uint32_t w1, uint32_t w2, int sh, int n,
                                             int half, const u32x4& sc, const u32x4& zc) {
    const uint32_t lo = __builtin_amdgcn_alignbit(w1, w0, sh);    // row bits 0 .. 31
    const uint32_t hi = __builtin_amdgcn_alignbit(w2, w1, sh);    // row bits 32 .. 63
    // the lane's eight 3-bit fields (row bits 24*half ..) and the fourth bits of those of its
    // channels that are 4-bit (row bits 48 + 8*half ..)
    const uint32_t L = __builtin_amdgcn_alignbit(hi, lo, 24 * half);
    const uint32_t ext = __builtin_amdgcn_ubfe(hi, 16 + 8 * half, min(max(n - 8 * half, 0), 8));
    // Channel pair (2k, 2k+1) goes to the low and high 16-bit halves, code bits 0-2 and fourth
    // bit 3. m_a holds fields 0.. in its low half and fields 1.. in its high half (pair 0; pair 1
    // after a 6-bit shift of each half), m_b the same from field 4 (pairs 2 and 3). The fourth
    // bits fill the slots those shifts leave free (bits 3 and 9 of each half): one 24-bit multiply
    // by 2^3 + 2^18 + 2^7 + 2^22 moves bits 0..3 of a nibble to 3, 19, 9, 25 (no two partial
    // products overlap, so no carries) and the merge keeps only those four bits.
    const uint32_t w_a = (L & 0xffffu) | ((L << 13) & 0xffff0000u);
    const uint32_t w_b = ((L >> 12) & 0xffffu) | ((L << 1) & 0xffff0000u);
    constexpr uint32_t kSpread = (1u << 3) | (1u << 18) | (1u << 7) | (1u << 22);
    constexpr uint32_t kSlots = 0x02080208u;
    const uint32_t m_a = (__umul24(ext & 15u, kSpread) & kSlots) | (w_a & ~kSlots);
    const uint32_t m_b = (__umul24(ext >> 4, kSpread) & kSlots) | (w_b & ~kSlots);
    f16x8 out;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = 2 * k;
        const uint32_t bits = (pk_shr16(k < 2 ? m_a : m_b, (k & 1) * 6) & 0x000f000fu) | 0x64006400u;
        const f16x2 qv = __builtin_bit_cast(f16x2, bits) - (f16x2){(_Float16)1024.0f, (_Float16)1024.0f};
        // vector elements are copied to scalars first: a bit cast applied directly to an
        // element of an ext_vector value has been compiled as a cast of element 0
        const uint32_t sk = sc[k], zk = zc[k];
        const f16x2 r = __builtin_elementwise_fma(qv, __builtin_bit_cast(f16x2, sk),
                                                  __builtin_bit_cast(f16x2, zk));
        out[e] = r[0];
        out[e + 1] = r[1];
    }
    return out;
}

// ------------------------------------------------------------------------------------------------
// Parameter blocks (passed by value; each stays well under the 4 KB kernel-argument limit).
// ------------------------------------------------------------------------------------------------
constexpr int kMaxHeads = 32;
constexpr int kTile = 64;              // tokens per cache block
constexpr int kFragLdsBytes = 96 * 1024;   // key-factor fragments of one head group in LDS
// several queries per sequence: a smaller factor budget (the rotated queries take the room) and
// at most this many heads per group
constexpr int kFragLdsBytesMQ = 64 * 1024;
constexpr int kMaxGroupHeadsMQ = 16;
constexpr int kMaxGroups = 32;
constexpr int kValueWaves = 4;         // waves per value workgroup
constexpr int kMaxBlocksPerSplit = 256;

// Latent cache block layouts (64-token blocks, 16-channel groups of 1024 elements):
//   key latent   zk[b][blk][g][t][k]      t < 64 token in block, k < 16 channel in group
//   value latent zv[b][blk][g][u][k][v]   u < 4, v < 16: token 16u + v, k < 16 channel in group
// so that one 16-byte lane load of eight consecutive elements feeds an MFMA operand fragment and
// the 64 lanes of a wave read 1 KB (key) or two 512-byte runs (value) of contiguous memory.
// Where 64-token block blk of sequence b lives: block b * nblk_cap + blk of the buffer, or, for a
// paged cache, page table[b * stride + blk] of the buffer's pool (the caller's block table).
struct BlockMap {
    const int32_t* table = nullptr;
    int stride = 0;
};
__device__ inline size_t block_id(const BlockMap& m, int nblk_cap, size_t b, long long blk) {
    return m.table ? (size_t)m.table[b * (size_t)m.stride + (size_t)blk] : b * (size_t)nblk_cap + (size_t)blk;
}
// element (token t, channel c) of a latent of C channels whose token t lies in block `id`
__host__ __device__ inline size_t zk_block_at(size_t id, int C, long long t, int c) {
    return (id * (size_t)(C >> 4) + (size_t)(c >> 4)) * 1024 + (size_t)(t & 63) * 16 + (size_t)(c & 15);
}
__host__ __device__ inline size_t zv_block_at(size_t id, int C, long long t, int c) {
    return (id * (size_t)(C >> 4) + (size_t)(c >> 4)) * 1024 + (size_t)((t & 63) >> 4) * 256 +
           (size_t)(c & 15) * 16 + (size_t)(t & 15);
}

// Ranks rounded up to the 16-channel tile: the cache stores each head's key latent with
// rank[h] = 16 * ceil(srank[h] / 16) channels at koff[h] and the value latent with rv channels
// (rv_src rounded up); the extra channels hold zeros. Callers' rows and factors keep the true
// ranks srank[h] at soff[h] (and rv_src). For ranks that are already multiples of 16 both views
// coincide.
struct PadMap {
    int H, rv, rv_src;
    int16_t koff[kMaxHeads + 1];
    int16_t soff[kMaxHeads + 1];
    int16_t srank[kMaxHeads];
};
// stored key channel of caller channel c
__device__ inline int pad_key_channel(const PadMap& m, int c) {
    int h = 0;
    while (h + 1 < m.H && c >= m.soff[h + 1]) ++h;
    return m.koff[h] + (c - m.soff[h]);
}
// caller key channel of stored channel c, or -1 for a padding channel
__device__ inline int src_key_channel(const PadMap& m, int c) {
    int h = 0;
    while (h + 1 < m.H && c >= m.koff[h + 1]) ++h;
    const int local = c - m.koff[h];
    return local < m.srank[h] ? m.soff[h] + local : -1;
}

// Mixed 4/3-bit code layout of one latent (see quant.hip for the byte layout).
constexpr int kMaxKeyGroups = 256;          // R_k <= 4096
struct Q43Layout {
    int C;                      // channels of the latent
    int block_bytes;            // code bytes per 64-token block
    int is_key;                 // 1: token-major key layout, 0: channel-major value layout
    int n_hi;                   // value latent: channels [0, n_hi) are 4-bit
    int32_t goff[kMaxKeyGroups];   // key latent: byte offset of 16-channel group g in a block
    uint8_t gn[kMaxKeyGroups];     // key latent: 4-bit channels at the start of group g
};

__host__ __device__ inline bool q43_is_hi(const Q43Layout& L, int c) {
    return L.is_key ? (c & 15) < L.gn[c >> 4] : c < L.n_hi;
}
__host__ __device__ inline int q43_value_run_offset(const Q43Layout& L, int c) {
    return c < L.n_hi ? 32 * c : 32 * L.n_hi + 24 * (c - L.n_hi);
}

struct ScoreParams {
    const void* zk;        // key latent, block layout
    const void* bk;        // key factors [R_k caller rows][D], head h's rows at soff[h]
    const float* q;        // [B][H][D]
    void* P;               // [B][H][Tp] probabilities, relative to each 32-token tile's maximum
    float* stats;          // [B][H][2 * nblk][2] per 32-token tile: max (log2 units), sum of probabilities
    int B, H, D, Rk, nblk_cap, seq_len, nblk, Tp, blocks_per_wg;
    const int32_t* seq_lens = nullptr;   // per-sequence lengths (device, clamped to [0, seq_len])
    const int32_t* seq_map = nullptr;    // query row b reads cache sequence seq_map[b] (or b)
    int cache_batch = 0;
    BlockMap pages;
    float q_scale;         // softmax scale * log2(e)
    int8_t order[kMaxHeads];          // heads grouped: group g = order[gstart[g] .. gstart[g+1])
    int8_t gstart[kMaxGroups + 1];
    int16_t koff[kMaxHeads + 1];
    int16_t rank[kMaxHeads];
    int16_t soff[kMaxHeads + 1];   // caller rows of head h's factor (true rank srank[h] <= rank[h])
    int16_t srank[kMaxHeads];
    double rope_rev[64];   // theta_i / (2 pi): RoPE frequency in revolutions per position
    // mixed 4/3-bit key cache only: codes in zk, scales / zero points, binary16 tail rows
    const void* zk_meta;   // [B][cap/64][2][Rk]
    const void* zk_tail;   // [B][64][Rk]
    // Per query row (or NULL: the row's own length): the longest length among the call's rows
    // that read the same cache sequence. For a mixed 4/3-bit cache, the sequence's complete
    // 64-token groups below it are quantised and its partial last group is in the tail buffer.
    const int32_t* row_fill = nullptr;
    Q43Layout ql;
};

struct ValueParams {
    const void* zv;        // value latent, block layout
    const void* P;         // [B][H][Tp]
    const float* stats;    // [B][H][2 * nblk][2] per 32-token tile
    float* ws_ml;          // [B][S][H][2]   (max in log2 units, sum)
    float* ws_acc;         // [B][S][H][rv]
    int B, H, rv, nblk_cap, seq_len, nblk, Tp, S, blocks_per_split;
    const int32_t* seq_lens = nullptr;   // per-sequence lengths (device) or NULL
    const int32_t* seq_map = nullptr;    // query row b reads cache sequence seq_map[b] (or b)
    int cache_batch = 0;
    BlockMap pages;
    // mixed 4/3-bit value cache only
    const void* zv_meta;   // [B][cap/64][2][rv]
    const void* zv_tail;   // [B][64][rv]
    const int32_t* row_fill = nullptr;   // as in ScoreParams
    int block_bytes, n_hi;
};

// row_fill[i] = the largest clamped length among rows that read the same cache sequence as row i
struct RowFillParams {
    const int32_t* seq_map;
    const int32_t* seq_lens;
    int32_t* row_fill;
    int rows, cache_batch, max_len;
};

struct MergeParams {
    const float* ws_ml;    // [B][S][H][2]
    const float* ws_acc;   // [B][S][H][W]
    float* ws_a;           // [B][H][W] merged, normalised
    int B, H, S, W, active_splits;
};

struct ProjectParams {
    const float* ws_ml;    // [B][S][H][2] split (max, sum)
    const float* ws_acc;   // [B][S][H][rv] split partial sums, merged while loading
    const void* bv;        // [rv_src][H*D] (stored value channels past rv_src are zero)
    float* out;            // [B][H][D]
    int B, H, D, rv, S, rv_src;
};

// Rows times a weight matrix, y[m][n] = sum_k x[m][k] W[n][k] (weights output-major: row n holds
// output n's Kd weights), split over Kd. Row m of a launch is (sequence b0 + m / tl, token
// t0 + m % tl) and reads x + (b * x_tokens + t) * Kd. Output rows [0, N0) use w0, [N0, N) use w1.
struct LinearParams {
    const float* x;
    const void* w0;
    const void* w1;
    float* part;           // [S][M][N] partial sums, one slice per split of Kd
    int M, N, N0, Kd, S;
    int b0, t0, tl, x_tokens;
};

// Sum of the split partials and the store of row (b, t), output n:
//   kind 0: fp32 y[(b * x_tokens + t) * N + n]
//   kind 1: latent cache block layout, key channel n < N0 / value channel n - N0, token pos + t
//   kind 2: dense cache rows [B][cap][N0] (keys) and [B][cap][N - N0] (values), token pos + t
//   kind 3: binary16 tail rows [B][64][N0] / [B][64][N - N0], row (pos + t) % 64
struct LinearStoreParams {
    const float* part;
    void* dst0;
    void* dst1;
    int M, N, N0, S;
    int b0, t0, tl, x_tokens;
    int kind;
    long long pos;
    long long cap;         // kind 1: capacity / 64 blocks; kind 2: capacity in tokens
    int padded;            // kind 1 with rounded ranks: outputs map through `map`, pads are zeroed
    PadMap map;
    BlockMap pages;        // kinds 1 and 2
};

struct DenseDecodeParams {
    const void* k;         // [B][cap][H*D]
    const void* v;         // [B][cap][H*D]
    const float* q;        // [B][H][D]
    float* ws_ml;          // [B][S][H][2]
    float* ws_acc;         // [B][S][H][D]
    int B, H, D, cap, seq_len, S, tiles_per_split;
    const int32_t* seq_lens = nullptr;   // per-sequence lengths (device) or NULL
    const int32_t* seq_map = nullptr;    // query row b reads cache sequence seq_map[b] (or b)
    int cache_batch = 0;
    BlockMap pages;
    float q_scale;
    double rope_rev[64];
};

// A sequence's length: its entry of the per-sequence array clamped to [0, the launch's maximum],
// or the launch's length.
__device__ inline int seq_length(const int32_t* lens, int b, int max_len) {
    return lens ? min(max(lens[b], 0), max_len) : max_len;
}
// The cache sequence a query row reads: its entry of the map clamped to [0, cache_batch), or the
// row itself (one query per sequence).
__device__ inline int cache_seq(const int32_t* map, int b, int cache_batch) {
    return map ? min(max(map[b], 0), cache_batch - 1) : b;
}

// Copy one contiguous byte range per sequence: dst[b*dst_seq_stride + dst_off + i] =
// src[b*src_seq_stride + src_off + i] for i < bytes (a multiple of 16, 16-byte aligned).
struct RowCopyParams {
    const char* src;
    char* dst;
    long long src_seq_stride, dst_seq_stride;
    long long src_off, dst_off;
    long long bytes;
    // one row per sequence at its own position (device array, or NULL): dst_off grows by
    // (positions[b] % pos_mod, or positions[b] when pos_mod is 0) * bytes; sequences whose
    // position lies outside [0, pos_limit) are skipped
    const int32_t* positions = nullptr;
    int pos_mod = 0;
    long long pos_limit = 0;
};

// Token-major rows <-> block layout of a latent (layout 0: key, 1: value). to_blocks = 1:
// rows[b][t - row0][c] -> blocks for absolute tokens t in [t_begin, t_end); 0: the reverse.
struct BlockXposeParams {
    const void* src;
    void* dst;
    int B, C, nblk_cap;
    long long t_begin, t_end;
    long long row0;             // absolute token of row 0 of the row-major side
    long long rows_per_seq;     // rows per sequence on the row-major side
    int blk_first;              // first 64-token block touched
    int to_blocks;
    int layout;
    BlockMap pages;
    // blocks -> rows only: sequence b ends at min(t_end, pos0 + clamp(chunk_lens[b], 0, chunk))
    // (its later rows are left as they are, and none of its blocks past that end is read)
    const int32_t* chunk_lens = nullptr;
    long long pos0 = 0;
    int chunk = 0;
};

struct AppendSmallParams {
    const void* zk_src;         // [B][n][Rk] rows
    const void* zv_src;         // [B][n][rv] rows
    void* zk;
    void* zv;
    int B, Rk, rv, nblk_cap;
    long long pos, n;
    const int32_t* positions = nullptr;   // n == 1: sequence b's token goes to positions[b]
                                // (device; skipped outside [0, capacity)), or NULL: tokens pos ..
                                // pos + n - 1
    BlockMap pages;
};

// Rows of a latent with rounded ranks between the caller's layout [B][n][C_src] and the cache
// (token t0 + row): to_cache writes every stored channel (zeros in the padding), otherwise the
// caller channels are gathered back.
struct PaddedRowsParams {
    const void* rows;
    void* cache;
    int B, nblk_cap, which, C, C_src, to_cache;
    long long t0, n;
    const int32_t* positions = nullptr;   // as in AppendSmallParams (n == 1), or NULL
    BlockMap pages;
    PadMap map;
};

// Token rows of a paged dense cache: rows [B][n][row_bytes] <-> tokens t0 + i of sequence b (or
// positions[b] when n == 1 and positions is set; positions outside [0, capacity) are skipped).
struct PagedRowsParams {
    const char* rows;
    char* cache;
    long long row_bytes, t0, n;
    int B, nblk_cap, to_cache;
    const int32_t* positions = nullptr;
    BlockMap pages;
};

struct Q43QuantParams {
    Q43Layout L;
    const void* src;            // new rows [B][n][C] binary16
    const void* tail;           // [B][64][C] binary16
    void* codes;                // [B][cap/64][block_bytes]
    void* meta;                 // [B][cap/64][2][C] binary16 (scales, then zero points)
    int B, nblk_cap, g_first;
    long long pos, n;
    // one appended token per sequence (device array, or NULL): the group of sequence b is
    // quantised from the tail only when positions[b] is its last token
    const int32_t* positions = nullptr;
    BlockMap pages;
};

// Blockwise Hadamard rotation of binary16 rows (kind 0: latent rows dst = src . H, [n][C]) or
// factor rows (kind 1: dst = H^T . src, [C][ncols]); segments (start, width) cover the channels,
// each rotated by blockdiag(H_b) with its block size b.
constexpr int kMaxRotSegments = 2 * kMaxHeads;
struct HadamardParams {
    const uint16_t* src;
    uint16_t* dst;
    long long n;               // rows (kind 0) or columns (kind 1)
    int C;                     // channels
    int kind;
    int nseg;
    int seg_start[kMaxRotSegments];
    int seg_width[kMaxRotSegments];
    int seg_block[kMaxRotSegments];
    double seg_inv[kMaxRotSegments];   // fp64 value of 1 / sqrt(block size)
};

struct Q43ReadParams {
    Q43Layout L;
    const void* codes;
    const void* meta;
    const void* tail;
    void* out;                  // [B][t1 - t0][C] binary16
    int B, nblk_cap;
    long long t0, t1, full_tokens;   // tokens below full_tokens sit in complete groups
    BlockMap pages;
    // sequence b ends at e_b = pos0 + clamp(chunk_lens[b], 0, chunk): its complete groups are
    // those below e_b rounded down to 64 tokens, and its rows at or past e_b are left as they are
    const int32_t* chunk_lens = nullptr;
    long long pos0 = 0;
    int chunk = 0;
};

}  // namespace starkv
