// linear.hip -- rows of fp32 activations times an output-major weight matrix on the matrix cores,
// with the store of the result fused into the reduction of the split partial sums. It serves the
// two dense products around decode attention in the low-rank method (STAR-KV, Alg. 2): the
// down-projection of a new token's hidden state to its key and value latents before they are
// appended (steps 1-3), and the output projection of the heads' concatenated attention outputs
// (step 8). gfx950 (CDNA4) only.
//
// y[m][n] = sum_k x[m][k] W[n][k]. The weight W is read exactly once and is the only large operand
// (Kd x N elements against M <= 32 rows per workgroup), so the kernel is bound by HBM: per 64-wide
// K tile a wave reads 64 contiguous bytes of each of its weight rows (two lanes per row, one full
// 128-byte line), and the matrix cores make the multiply-adds free next to the load. The fp32
// rows are split into two 16-bit parts (x = hi + lo, lo the rounding remainder) and both are
// multiplied, which keeps the products within a few fp32 ulps of x * W; fp32 weights use the fp32
// matrix instruction on x as it is.
//
// A wave owns 128 weight rows (64 for fp32 weights) and all 32 activation rows of its tile, so one
// activation fragment and its split feed four matrix instructions. Kd is split over workgroups
// (grid.y) so that a launch has about two workgroups per CU; each workgroup's four waves take
// interleaved 64-wide K tiles of its range and reduce through LDS, then write one [M][N] slice of
// partial sums. A second kernel sums the slices in a fixed order (the result
// does not depend on scheduling) and stores each output where it belongs: fp32 rows, or the
// latent / dense cache in its storage type.

#include <type_traits>

#include "common.hpp"

namespace starkv {

namespace {

constexpr int kLinWaves = 4;

// Two 16-bit parts of eight fp32 values: hi = round(v), lo = round(v - hi). v - hi is exact in
// fp32, so x * W is recovered up to the rounding of lo (2^-22 |v| for binary16, 2^-16 |v| for
// bfloat16) and the fp32 accumulation.
template <int K> struct Split;
template <> struct Split<kF16> {
    __device__ static __forceinline__ void run(const f32x4& a, const f32x4& b, f16x8& hi, f16x8& lo) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = e < 4 ? a[e] : b[e - 4];
            const _Float16 h = (_Float16)v;
            hi[e] = h;
            lo[e] = (_Float16)(v - (float)h);
        }
    }
};
template <> struct Split<kBF16> {
    __device__ static __forceinline__ void run(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = e < 4 ? a[e] : b[e - 4];
            const __bf16 h = (__bf16)v;
            hi[e] = h;
            lo[e] = (__bf16)(v - (float)h);
        }
    }
};

// Weight row tiles of 32 per wave: four for 16-bit weights (128 rows share each activation
// fragment and its split), two for fp32 weights (register budget).
template <int K> constexpr int lin_row_tiles() { return K == kF32 ? 2 : 4; }

template <int K>
__global__ __launch_bounds__(256, 2) void linear_partial(const LinearParams p) {
    constexpr int RT = lin_row_tiles<K>();
    constexpr int ES = Elem<K>::bytes;
    constexpr int CH = 64 * ES / 16;           // 16-byte chunks per weight row of a 64-wide K tile
    constexpr int RPI = 64 / CH;               // weight rows per wave load (1 KB contiguous per row group)
    constexpr int NI = RT * 32 / RPI;          // wave loads per tile (16 KB)
    constexpr int ROW = RT * 32 + 4;           // floats per reduction row (padding keeps rows apart)
    // Weight tiles staged per wave ([row][chunk], chunk c of row r stored at c ^ (r % CH) so that
    // the fragment reads of 8 consecutive rows hit distinct banks); the same memory later holds
    // the waves' [m][n] results for the reduction.
    constexpr int kStage = kLinWaves * RT * 32 * CH * 16;
    constexpr int kRed = kLinWaves * 32 * ROW * 4;
    __shared__ __attribute__((aligned(16))) char s_mem[kStage > kRed ? kStage : kRed];
    u32x4 (*s_w)[RT * 32][CH] = reinterpret_cast<u32x4 (*)[RT * 32][CH]>(s_mem);
    float (*s_red)[32][ROW] = reinterpret_cast<float (*)[32][ROW]>(s_mem);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int n0 = blockIdx.x * 32 * RT, m0 = blockIdx.z * 32, s = blockIdx.y;
    const int kt = p.Kd >> 6;
    const int tb = (int)((long long)s * kt / p.S), te = (int)((long long)(s + 1) * kt / p.S);

    // B operand: activation row m0 + l32; rows past the end contribute zeros
    const bool mok = m0 + l32 < p.M;
    const int m = min(m0 + l32, p.M - 1);
    const int b = p.b0 + m / p.tl, t = p.t0 + m % p.tl;
    const float* xrow = p.x + ((size_t)b * p.x_tokens + t) * p.Kd;
    // weight rows this lane loads: row group i covers rows RPI*i .. RPI*i + RPI - 1 of the tile;
    // rows past the end are read from the last valid row and only feed outputs never stored
    const int lrow = lane / CH, lc = lane % CH;
    const char* wsrc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int n = min(n0 + RPI * i + lrow, p.N - 1);
        wsrc[i] = (n < p.N0 ? static_cast<const char*>(p.w0) + (size_t)n * p.Kd * ES
                            : static_cast<const char*>(p.w1) + (size_t)(n - p.N0) * p.Kd * ES) + lc * 16;
    }

    f32x16 acc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][i] = 0.0f;

    // K slot 8*half + e of step j holds k = 64*tile + 32*half + 8*j + e in both operands.
    for (int ti = tb + wave; ti < te; ti += kLinWaves) {
        {
            u32x4 buf[NI];
#pragma unroll
            for (int i = 0; i < NI; ++i)
                buf[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wsrc[i] + (size_t)ti * 64 * ES));
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int r = RPI * i + lrow;
                s_w[wave][r][lc ^ (r % CH)] = buf[i];
            }
        }
        const int k = ti * 64 + 32 * half;
        f32x4 xv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            xv[i] = mok ? *reinterpret_cast<const f32x4*>(xrow + k + 4 * i) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            typename Elem<K>::frag w[RT];
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const int row = 32 * r + l32;
                if constexpr (K == kF32) {
                    const int c = 8 * half + 2 * j;
                    const u32x4 lo4 = s_w[wave][row][c ^ (row % CH)];
                    const u32x4 hi4 = s_w[wave][row][(c + 1) ^ (row % CH)];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        w[r][e] = __uint_as_float(lo4[e]);
                        w[r][e + 4] = __uint_as_float(hi4[e]);
                    }
                } else {
                    const u32x4 v = s_w[wave][row][(4 * half + j) ^ (row % CH)];
                    w[r] = __builtin_bit_cast(typename Elem<K>::frag, v);
                }
            }
            if constexpr (K == kF32) {
                f32x8 xf;
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[e] = e < 4 ? xv[2 * j][e] : xv[2 * j + 1][e - 4];
#pragma unroll
                for (int r = 0; r < RT; ++r) acc[r] = mma32<kF32>(w[r], xf, acc[r]);
            } else {
                typename Elem<K>::frag hi, lo;
                Split<K>::run(xv[2 * j], xv[2 * j + 1], hi, lo);
#pragma unroll
                for (int r = 0; r < RT; ++r) acc[r] = mma32<K>(w[r], hi, acc[r]);
#pragma unroll
                for (int r = 0; r < RT; ++r) acc[r] = mma32<K>(w[r], lo, acc[r]);
            }
        }
    }
    __syncthreads();                            // the staging area becomes the reduction area

    // Reduce the four waves' tiles through LDS as [m][n]: accumulator registers 4g..4g+3 of a lane
    // are four consecutive outputs n of its row m, one 16-byte write.
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(&s_red[wave][l32][32 * r + 8 * g + 4 * half]) =
                f32x4{acc[r][4 * g], acc[r][4 * g + 1], acc[r][4 * g + 2], acc[r][4 * g + 3]};
    __syncthreads();
    const bool vec = (p.N & 3) == 0;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int idx = tid + 256 * i;                // (m, four outputs) items, 32 x 8*RT
        const int ml = idx / (8 * RT), nl = 4 * (idx % (8 * RT));
        f32x4 v = *reinterpret_cast<const f32x4*>(&s_red[0][ml][nl]);
#pragma unroll
        for (int w = 1; w < kLinWaves; ++w) v += *reinterpret_cast<const f32x4*>(&s_red[w][ml][nl]);
        const int n = n0 + nl;
        if (m0 + ml >= p.M || n >= p.N) continue;
        float* dst = p.part + ((size_t)s * p.M + m0 + ml) * p.N + n;
        if (vec) {
            *reinterpret_cast<f32x4*>(dst) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < p.N) dst[e] = v[e];
        }
    }
}

template <int E>
__device__ __forceinline__ void store_elem(void* base, size_t i, float v) {
    if constexpr (E == kF32)
        static_cast<float*>(base)[i] = v;
    else if constexpr (E == kF16)
        static_cast<_Float16*>(base)[i] = (_Float16)v;
    else
        static_cast<uint16_t*>(base)[i] = float_to_bf16_bits(v);
}

template <int E>
__device__ __forceinline__ void store_one(const LinearStoreParams& p, int m, int n, float v) {
    const int b = p.b0 + m / p.tl, t = p.t0 + m % p.tl;
    const long long tok = p.pos + t;
    const bool key = n < p.N0;
    const int c = key ? n : n - p.N0;
    const int C = key ? p.N0 : p.N - p.N0;
    void* dst = key ? p.dst0 : p.dst1;
    switch (p.kind) {
    case 0:
        static_cast<float*>(p.dst0)[((size_t)b * p.x_tokens + t) * p.N + n] = v;
        break;
    case 1:
        if (!p.padded) {
            const size_t id = block_id(p.pages, (int)p.cap, b, tok >> 6);
            store_elem<E>(dst, key ? zk_block_at(id, C, tok, c) : zv_block_at(id, C, tok, c), v);
        } else if (key) {
            // caller channel c of head h goes to stored channel koff[h] + (c - soff[h]); the
            // head's last channel also zeroes the head's padding channels of this token
            const PadMap& m = p.map;
            int h = 0;
            while (h + 1 < m.H && c >= m.soff[h + 1]) ++h;
            const int Cs = m.koff[m.H], cs = m.koff[h] + (c - m.soff[h]);
            const size_t id = block_id(p.pages, (int)p.cap, b, tok >> 6);
            store_elem<E>(dst, zk_block_at(id, Cs, tok, cs), v);
            if (c + 1 == m.soff[h + 1])
                for (int z = cs + 1; z < m.koff[h + 1]; ++z) store_elem<E>(dst, zk_block_at(id, Cs, tok, z), 0.0f);
        } else {
            const int Cs = p.map.rv;
            const size_t id = block_id(p.pages, (int)p.cap, b, tok >> 6);
            store_elem<E>(dst, zv_block_at(id, Cs, tok, c), v);
            if (c + 1 == p.map.rv_src)
                for (int z = c + 1; z < Cs; ++z) store_elem<E>(dst, zv_block_at(id, Cs, tok, z), 0.0f);
        }
        break;
    case 2:
        store_elem<E>(dst, (block_id(p.pages, (int)(p.cap >> 6), b, tok >> 6) * 64 + (tok & 63)) * C + c, v);
        break;
    default:
        store_elem<kF16>(dst, ((size_t)b * 64 + (tok & 63)) * C + c, v);
        break;
    }
}

// Thread per four consecutive outputs of a row (N a multiple of 4, so the slices' loads are
// 16 bytes) or per output: the S slices are loaded eight at a time and summed in split order.
// E: storage type of kinds 1 and 2 (kind 0 stores fp32, kind 3 binary16).
template <int E, int V>
__global__ __launch_bounds__(256) void linear_store(const LinearStoreParams p) {
    using T = typename std::conditional<V == 4, f32x4, float>::type;
    const int per_row = p.N / V;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.M * per_row) return;
    const int m = (int)(idx / per_row), n = V * (int)(idx - (long long)m * per_row);
    const T* src = reinterpret_cast<const T*>(p.part + (size_t)m * p.N + n);
    const size_t slice = (size_t)p.M * p.N / V;
    T v = T{};
    int s = 0;
    for (; s + 8 <= p.S; s += 8) {
        T a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = src[(s + i) * slice];
#pragma unroll
        for (int i = 0; i < 8; ++i) v += a[i];
    }
    for (; s < p.S; ++s) v += src[s * slice];
    if constexpr (V == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) store_one<E>(p, m, n + e, v[e]);
    } else {
        store_one<E>(p, m, n, v);
    }
}

}  // namespace

int linear_rows_per_workgroup(int elem) { return 32 * (elem == kF32 ? lin_row_tiles<kF32>() : lin_row_tiles<kF16>()); }

hipError_t launch_linear(const LinearParams& p, int elem, hipStream_t st) {
    const int rows = linear_rows_per_workgroup(elem);
    const dim3 grid((p.N + rows - 1) / rows, p.S, (p.M + 31) / 32);
    switch (elem) {
    case kF32: hipLaunchKernelGGL(linear_partial<kF32>, grid, dim3(256), 0, st, p); break;
    case kF16: hipLaunchKernelGGL(linear_partial<kF16>, grid, dim3(256), 0, st, p); break;
    case kBF16: hipLaunchKernelGGL(linear_partial<kBF16>, grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int V>
static hipError_t launch_store_v(const LinearStoreParams& p, int elem, hipStream_t st) {
    const long long n = (long long)p.M * (p.N / V);
    const dim3 grid((unsigned)((n + 255) / 256));
    switch (elem) {
    case kF32: hipLaunchKernelGGL((linear_store<kF32, V>), grid, dim3(256), 0, st, p); break;
    case kF16: hipLaunchKernelGGL((linear_store<kF16, V>), grid, dim3(256), 0, st, p); break;
    case kBF16: hipLaunchKernelGGL((linear_store<kBF16, V>), grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_linear_store(const LinearStoreParams& p, int elem, hipStream_t st) {
    return (p.N & 3) == 0 ? launch_store_v<4>(p, elem, st) : launch_store_v<1>(p, elem, st);
}

}  // namespace starkv
