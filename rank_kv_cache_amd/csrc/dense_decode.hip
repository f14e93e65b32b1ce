// dense_decode.hip -- decode attention for exempt (uncompressed) layers on gfx950.
//
// The pages keep layers 0, 1 and 31 uncompressed (Zhou, STAR-KV reading notes, section 4 and
// Algorithm 1 step 2); such a layer is the identity-factor special case of the latent path:
//   s_n = scale * q_h . RoPE_n(K_h[n]),  out_h = softmax(s) V_h,  K stored pre-RoPE.
// One workgroup per (split, sequence) covers all heads, so the RoPE table of a tile is computed
// once and shared by every head. Per 64-token tile:
//   * score phase: a (head, token) item is handled by D/8 lanes, each rotating 4 RoPE pairs
//     (8 dims) and reducing the partial dot with lane shuffles;
//   * softmax phase: as in the latent kernel (wave-shuffle max/sum, running state per head);
//   * value phase: thread (head, 16-dim slice) accumulates p * V over the tile's tokens.
// The split's (max, sum, acc) goes to the workspace and the latent path's merge kernel finishes.

#include "common.hpp"

namespace starkv {

template <int K>
__device__ __forceinline__ void load4(const void* base, size_t i, float* out);
template <> __device__ __forceinline__ void load4<kF32>(const void* base, size_t i, float* out) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
}
template <> __device__ __forceinline__ void load4<kF16>(const void* base, size_t i, float* out) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 v = *reinterpret_cast<const h4*>(static_cast<const _Float16*>(base) + i);
    out[0] = (float)v[0]; out[1] = (float)v[1]; out[2] = (float)v[2]; out[3] = (float)v[3];
}
template <> __device__ __forceinline__ void load4<kBF16>(const void* base, size_t i, float* out) {
    typedef uint16_t u4 __attribute__((ext_vector_type(4)));
    const u4 v = *reinterpret_cast<const u4*>(static_cast<const uint16_t*>(base) + i);
    out[0] = bf16_bits_to_float(v[0]); out[1] = bf16_bits_to_float(v[1]);
    out[2] = bf16_bits_to_float(v[2]); out[3] = bf16_bits_to_float(v[3]);
}

template <int D, int K>
__global__ __launch_bounds__(256) void dense_decode_split(const DenseDecodeParams p) {
    constexpr int NF = D / 2;
    constexpr int SG = D / 8;              // lanes per (head, token) item in the score phase
    constexpr int NG = 256 / SG;           // items in flight per pass
    constexpr int TPH = 8;                 // threads per head in the value phase
    constexpr int DPT = D / TPH;           // dims per thread in the value phase
    constexpr int TRIG_STRIDE = 2 * NF + 4;
    constexpr int SC_STRIDE = kTile + 4;

    __shared__ __attribute__((aligned(16))) float s_trig[kTile * TRIG_STRIDE];
    __shared__ __attribute__((aligned(16))) float s_q[kMaxHeads * D];
    __shared__ __attribute__((aligned(16))) float s_score[kMaxHeads * SC_STRIDE];
    __shared__ __attribute__((aligned(16))) float s_p[kMaxHeads * SC_STRIDE];
    __shared__ __attribute__((aligned(16))) float s_alpha[kMaxHeads];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int split = blockIdx.x;
    const int b = blockIdx.y;
    const int H = p.H;
    const size_t W = (size_t)H * D;
    const int ntiles = (p.seq_len + kTile - 1) / kTile;
    const int tile_begin = split * p.tiles_per_split;
    const int tile_end = min(ntiles, tile_begin + p.tiles_per_split);

    for (int i = tid; i < H * D; i += 256) s_q[i] = p.q[(size_t)b * H * D + i] * p.q_scale;

    // softmax state: wave w owns heads w + 4*j
    float m_run[8], l_run[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.0f; }
    // value accumulators: head hv, dims dv0 .. dv0 + DPT - 1
    const int hv = tid / TPH;
    const int dv0 = (tid % TPH) * DPT;
    float accv[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) accv[i] = 0.0f;
    __syncthreads();

    const int g = tid / SG, sub = tid % SG;
    for (int tile = tile_begin; tile < tile_end; ++tile) {
        const int t0 = tile * kTile;
        for (int e = tid; e < kTile * NF; e += 256) {
            const int j = e / NF, i = e - j * NF;
            const double rev = (double)(t0 + j) * p.rope_rev[i];
            const float x = (float)(rev - floor(rev));
            float c, s;
            sincos_rev(x, &c, &s);
            s_trig[j * TRIG_STRIDE + 2 * i] = c;
            s_trig[j * TRIG_STRIDE + 2 * i + 1] = s;
        }
        __syncthreads();

        // score phase
        for (int item = g; item < H * kTile; item += NG) {
            const int h = item / kTile, t = item - h * kTile;
            const size_t row = ((size_t)b * p.cap + t0 + t) * W + (size_t)h * D;
            float k1[4], k2[4];
            load4<K>(p.k, row + 4 * sub, k1);
            load4<K>(p.k, row + NF + 4 * sub, k2);
            const float* tr = &s_trig[t * TRIG_STRIDE + 8 * sub];
            const float* qh = &s_q[h * D];
            float sc = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float c = tr[2 * r], s = tr[2 * r + 1];
                const float q1 = qh[4 * sub + r], q2 = qh[NF + 4 * sub + r];
                sc += q1 * (k1[r] * c - k2[r] * s) + q2 * (k2[r] * c + k1[r] * s);
            }
#pragma unroll
            for (int o = SG / 2; o > 0; o >>= 1) sc += __shfl_xor(sc, o, 64);
            if (sub == 0) s_score[h * SC_STRIDE + t] = (t0 + t < p.seq_len) ? sc : -INFINITY;
        }
        __syncthreads();

        // softmax phase
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int h = wave + 4 * j;
            if (h < H) {
                const float v = s_score[h * SC_STRIDE + lane];
                const float m_new = fmaxf(m_run[j], wave_max(v));
                const float alpha = __builtin_amdgcn_exp2f(m_run[j] - m_new);
                const float pr = __builtin_amdgcn_exp2f(v - m_new);
                l_run[j] = l_run[j] * alpha + wave_sum(pr);
                m_run[j] = m_new;
                s_p[h * SC_STRIDE + lane] = pr;
                if (lane == 0) s_alpha[h] = alpha;
            }
        }
        __syncthreads();

        // value phase
        if (hv < H) {
            const float al = s_alpha[hv];
#pragma unroll
            for (int i = 0; i < DPT; ++i) accv[i] *= al;
            const int nt = min(kTile, p.seq_len - t0);
            for (int t = 0; t < nt; ++t) {
                const float pr = s_p[hv * SC_STRIDE + t];
                const size_t row = ((size_t)b * p.cap + t0 + t) * W + (size_t)hv * D + dv0;
#pragma unroll
                for (int i = 0; i < DPT; i += 4) {
                    float v[4];
                    load4<K>(p.v, row + i, v);
#pragma unroll
                    for (int r = 0; r < 4; ++r) accv[i + r] += pr * v[r];
                }
            }
        }
    }

    const size_t part = (size_t)b * p.S + split;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int h = wave + 4 * j;
        if (h < H && lane == 0) {
            p.ws_ml[(part * H + h) * 2 + 0] = m_run[j];
            p.ws_ml[(part * H + h) * 2 + 1] = l_run[j];
        }
    }
    if (hv < H) {
#pragma unroll
        for (int i = 0; i < DPT; ++i) p.ws_acc[(part * H + hv) * D + dv0 + i] = accv[i];
    }
}

template <int D, int K>
static hipError_t launch_dense_t(const DenseDecodeParams& p, hipStream_t st) {
    hipLaunchKernelGGL((dense_decode_split<D, K>), dim3(p.S, p.B), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_dense_split(const DenseDecodeParams& p, int elem, hipStream_t st) {
    if (p.D == 128) {
        switch (elem) {
        case kF32: return launch_dense_t<128, kF32>(p, st);
        case kF16: return launch_dense_t<128, kF16>(p, st);
        case kBF16: return launch_dense_t<128, kBF16>(p, st);
        }
    } else if (p.D == 64) {
        switch (elem) {
        case kF32: return launch_dense_t<64, kF32>(p, st);
        case kF16: return launch_dense_t<64, kF16>(p, st);
        case kBF16: return launch_dense_t<64, kBF16>(p, st);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace starkv
