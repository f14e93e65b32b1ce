// linear.hip -- rows of fp32 activations times an output-major weight matrix on the matrix cores,
// with the store of the result fused into the reduction of the split partial sums. It serves the
// two dense products around decode attention in the low-rank method (STAR-KV, Alg. 2): the
// down-projection of a new token's hidden state to its key and value latents before they are
// appended (steps 1-3), and the output projection of the heads' concatenated attention outputs
// (step 8). gfx950 (CDNA4) only.
//
// y[m][n] = sum_k x[m][k] W[n][k]. The weight W is read exactly once and is the only large operand
// (Kd x N elements against M <= 32 rows per workgroup), so the kernel is bound by HBM: a wave owns
// 32 weight rows and reads 64 contiguous bytes of each per 64-wide K tile (two lanes per row, one
// full 128-byte line), and the matrix cores make the multiply-adds free next to the load. The fp32
// rows are split into two 16-bit parts (x = hi + lo, lo the rounding remainder) and both are
// multiplied, which keeps the products within a few fp32 ulps of x * W; fp32 weights use the fp32
// matrix instruction on x as it is.
//
// Kd is split over workgroups (grid.y) so that a launch has about two workgroups per CU; each
// workgroup's four waves take interleaved K tiles of its range and reduce through LDS, then write
// one [M][N] slice of partial sums. A second kernel sums the slices in a fixed order (the result
// does not depend on scheduling) and stores each output where it belongs: fp32 rows, or the
// latent / dense cache in its storage type.

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

template <int K>
__global__ __launch_bounds__(256) void linear_partial(const LinearParams p) {
    __shared__ float s_red[kLinWaves][32][33];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, half = lane >> 5, l32 = lane & 31;
    const int n0 = blockIdx.x * 32, m0 = blockIdx.z * 32, s = blockIdx.y;
    const int kt = p.Kd >> 6;
    const int tb = (int)((long long)s * kt / p.S), te = (int)((long long)(s + 1) * kt / p.S);

    // A operand: weight row n; B operand: activation row m. Rows past the end are read from the
    // last valid row and only feed outputs that are never stored.
    const int n = min(n0 + l32, p.N - 1);
    const void* wrow;
    if (n < p.N0)
        wrow = static_cast<const char*>(p.w0) + (size_t)n * p.Kd * Elem<K>::bytes;
    else
        wrow = static_cast<const char*>(p.w1) + (size_t)(n - p.N0) * p.Kd * Elem<K>::bytes;
    const int m = min(m0 + l32, p.M - 1);
    const int b = p.b0 + m / p.tl, t = p.t0 + m % p.tl;
    const float* xrow = p.x + ((size_t)b * p.x_tokens + t) * p.Kd;

    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    // K slot 8*half + e of step j holds k = 64*tile + 32*half + 8*j + e in both operands: each
    // lane reads 32 consecutive k of its row, and the four steps cover the tile once.
    auto load_w = [&](typename Elem<K>::frag (&w)[4], int ti) __attribute__((always_inline)) {
        const int k = ti * 64 + 32 * half;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = load_frag<K>(wrow, (size_t)k + 8 * j);
    };
    auto tile = [&](const typename Elem<K>::frag (&w)[4], int ti) __attribute__((always_inline)) {
        const int k = ti * 64 + 32 * half;
        f32x4 xv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = *reinterpret_cast<const f32x4*>(xrow + k + 4 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (K == kF32) {
                f32x8 xf;
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[e] = e < 4 ? xv[2 * j][e] : xv[2 * j + 1][e - 4];
                acc = mma32<kF32>(w[j], xf, acc);
            } else {
                typename Elem<K>::frag hi, lo;
                Split<K>::run(xv[2 * j], xv[2 * j + 1], hi, lo);
                acc = mma32<K>(w[j], hi, acc);
                acc = mma32<K>(w[j], lo, acc);
            }
        }
    };
    // two tiles' weights in flight per wave
    int ti = tb + wave;
    for (; ti + kLinWaves < te; ti += 2 * kLinWaves) {
        typename Elem<K>::frag wa[4], wb[4];
        load_w(wa, ti);
        load_w(wb, ti + kLinWaves);
        tile(wa, ti);
        tile(wb, ti + kLinWaves);
    }
    if (ti < te) {
        typename Elem<K>::frag wa[4];
        load_w(wa, ti);
        tile(wa, ti);
    }

#pragma unroll
    for (int r = 0; r < 16; ++r) s_red[wave][acc_row(r, lane)][l32] = acc[r];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + 256 * i;
        const int nl = idx & 31, ml = idx >> 5;
        const float v = s_red[0][nl][ml] + s_red[1][nl][ml] + s_red[2][nl][ml] + s_red[3][nl][ml];
        if (m0 + ml < p.M && n0 + nl < p.N)
            p.part[((size_t)s * p.M + m0 + ml) * p.N + n0 + nl] = v;
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

// E: storage type of kinds 1 and 2 (kind 0 stores fp32, kind 3 binary16)
template <int E>
__global__ __launch_bounds__(256) void linear_store(const LinearStoreParams p) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.M * p.N) return;
    const int m = (int)(idx / p.N), n = (int)(idx - (long long)m * p.N);
    float v = 0.0f;
    for (int s = 0; s < p.S; ++s) v += p.part[((size_t)s * p.M + m) * p.N + n];
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
        store_elem<E>(dst, key ? zk_block_index(b, p.cap, C, tok, c) : zv_block_index(b, p.cap, C, tok, c), v);
        break;
    case 2:
        store_elem<E>(dst, ((size_t)b * p.cap + tok) * C + c, v);
        break;
    default:
        store_elem<kF16>(dst, ((size_t)b * 64 + (tok & 63)) * C + c, v);
        break;
    }
}

}  // namespace

hipError_t launch_linear(const LinearParams& p, int elem, hipStream_t st) {
    const dim3 grid((p.N + 31) / 32, p.S, (p.M + 31) / 32);
    switch (elem) {
    case kF32: hipLaunchKernelGGL(linear_partial<kF32>, grid, dim3(256), 0, st, p); break;
    case kF16: hipLaunchKernelGGL(linear_partial<kF16>, grid, dim3(256), 0, st, p); break;
    case kBF16: hipLaunchKernelGGL(linear_partial<kBF16>, grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_linear_store(const LinearStoreParams& p, int elem, hipStream_t st) {
    const long long n = (long long)p.M * p.N;
    const dim3 grid((unsigned)((n + 255) / 256));
    switch (elem) {
    case kF32: hipLaunchKernelGGL(linear_store<kF32>, grid, dim3(256), 0, st, p); break;
    case kF16: hipLaunchKernelGGL(linear_store<kF16>, grid, dim3(256), 0, st, p); break;
    case kBF16: hipLaunchKernelGGL(linear_store<kBF16>, grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace starkv
