// dense_decode.hip -- decode attention for exempt (uncompressed) layers on gfx950.
//
// The pages keep layers 0, 1 and 31 uncompressed (Zhou, STAR-KV reading notes, section 4 and
// Algorithm 1 step 2); such a layer is the identity-factor special case of the latent path:
//   s_n = scale * q_h . RoPE_n(K_h[n]),  out_h = softmax(s) V_h,  K stored pre-RoPE.
//
// The layer streams 4 * d bytes per (token, head) and does O(d) arithmetic on them, so it is bound
// by HBM and the kernel is plain SIMT: no MFMA, no LDS traffic on the data path. A wave owns
// 64 / LPH heads of one sequence for a range of tokens; the LPH lanes of a head each hold eight
// RoPE pairs (dims 8c .. 8c+7 and d/2 + 8c .. +7), loaded as 16-byte vectors, so a wave reads
// whole contiguous head rows. Waves never synchronise with each other.
//
// RoPE uses R_{t0+j} = R_{t0} R_j: per 32-token sub-tile the lane's query pairs are rotated back
// by t0 once (q' = R_{t0}^T q), and the rotation by j < 32 comes from a table of cos / sin of
// j * theta_i computed once per workgroup in LDS. Scores of a sub-tile stay in registers; the
// online softmax rescale happens once per sub-tile; the (max, sum, acc) of the split goes to the
// workspace and the latent path's merge kernel finishes.

#include "common.hpp"

namespace starkv {

// Eight consecutive elements as fp32 (16-byte loads; 32 bytes for fp32), non-temporal: K and V
// are streamed once.
template <int K> __device__ __forceinline__ void load8(const void* base, size_t i, float* out);
template <> __device__ __forceinline__ void load8<kF32>(const void* base, size_t i, float* out) {
    const f32x4* s = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i);
    const f32x4 a = __builtin_nontemporal_load(s), b = __builtin_nontemporal_load(s + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) { out[e] = a[e]; out[4 + e] = b[e]; }
}
template <> __device__ __forceinline__ void load8<kF16>(const void* base, size_t i, float* out) {
    const f16x8 v = __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(static_cast<const _Float16*>(base) + i));
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
}
template <> __device__ __forceinline__ void load8<kBF16>(const void* base, size_t i, float* out) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + i));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t w = v[e];
        out[2 * e] = __uint_as_float(w << 16);
        out[2 * e + 1] = __uint_as_float(w & 0xffff0000u);
    }
}

// Sum over aligned groups of LPH (4 or 8) lanes with DPP lane permutations.
template <int LPH>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_mov<0xB1>(v);                     // quad_perm [1,0,3,2]: partner lane ^ 1
    v += dpp_mov<0x4E>(v);                     // quad_perm [2,3,0,1]: partner lane ^ 2
    if constexpr (LPH == 8) v += dpp_mov<0x141>(v);   // row_half_mirror: the other quad of eight
    return v;
}

constexpr int kDenseSub = 32;          // tokens per sub-tile (rotation table rows)
constexpr int kDenseGroup = 8;         // tokens per online-softmax step

template <int D, int K>
__global__ __launch_bounds__(256) void dense_decode_split(const DenseDecodeParams p) {
    constexpr int NF = D / 2;          // RoPE frequencies
    constexpr int LPH = NF / 8;        // lanes per head
    constexpr int HPW = 64 / LPH;      // heads per wave
    constexpr int TT = kDenseSub;
    static_assert(LPH == 4 || LPH == 8, "head_dim 64 or 128");

    __shared__ __attribute__((aligned(16))) float s_cs[TT][NF][2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int split = blockIdx.x;
    const int b = blockIdx.y;
    const int H = p.H;
    const size_t W = (size_t)H * D;
    const int c = lane % LPH;
    const int h_raw = wave * HPW + lane / LPH;
    const bool hok = h_raw < H;
    const int h = min(h_raw, H - 1);
    const int seq_len = seq_length(p.seq_lens, b, p.seq_len);   // this sequence's length
    const int bc = cache_seq(p.seq_map, b, p.cache_batch);      // the cache sequence read
    const int t_begin = split * p.tiles_per_split * kTile;
    const int t_end = min(seq_len, t_begin + p.tiles_per_split * kTile);

    for (int e = tid; e < TT * NF; e += blockDim.x) {
        const int j = e / NF, i = e - j * NF;
        const double rev = (double)j * p.rope_rev[i];
        float cs, sn;
        sincos_rev((float)(rev - floor(rev)), &cs, &sn);
        s_cs[j][i][0] = cs;
        s_cs[j][i][1] = sn;
    }
    float q1[8], q2[8];
    {
        const float* qh = p.q + ((size_t)b * H + h) * D;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            q1[r] = qh[8 * c + r] * p.q_scale;
            q2[r] = qh[NF + 8 * c + r] * p.q_scale;
        }
    }
    __syncthreads();

    float m_run = -INFINITY, l_run = 0.0f;
    float acc1[8], acc2[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) { acc1[r] = 0.0f; acc2[r] = 0.0f; }

    const size_t col = (size_t)h * D + 8 * c;
    for (int t0 = t_begin; t0 < t_end; t0 += TT) {
        // q' = R_{t0}^T q for the lane's eight frequencies
        float qa[8], qb[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const double rev = (double)t0 * p.rope_rev[8 * c + r];
            float cb, sb;
            sincos_rev((float)(rev - floor(rev)), &cb, &sb);
            qa[r] = q1[r] * cb + q2[r] * sb;
            qb[r] = q2[r] * cb - q1[r] * sb;
        }
        // groups of kDenseGroup tokens: scores, one online-softmax rescale, values
#pragma unroll 1
        for (int j0 = 0; j0 < TT && t0 + j0 < t_end; j0 += kDenseGroup) {
            const int nt = min(kDenseGroup, t_end - t0 - j0);
            float sc[kDenseGroup];
#pragma unroll
            for (int jj = 0; jj < kDenseGroup; ++jj) {
                const int j = j0 + jj;
                // rows past the sequence end lie inside the 64-token-aligned capacity; their
                // scores are replaced below, so the loads stay unconditional
                const size_t row = (block_id(p.pages, p.cap >> 6, bc, (t0 + j) >> 6) * 64 + ((t0 + j) & 63)) * W + col;
                float k1[8], k2[8];
                load8<K>(p.k, row, k1);
                load8<K>(p.k, row + NF, k2);
                const f32x4* cs = reinterpret_cast<const f32x4*>(&s_cs[j][8 * c][0]);
                float s = 0.0f;
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const f32x4 t = cs[r4];            // (cos, sin) of two frequencies
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int r = 2 * r4 + u;
                        const float cr = t[2 * u], sr = t[2 * u + 1];
                        s = fmaf(qa[r], fmaf(-k2[r], sr, k1[r] * cr), s);
                        s = fmaf(qb[r], fmaf(k1[r], sr, k2[r] * cr), s);
                    }
                }
                sc[jj] = jj < nt ? group_sum<LPH>(s) : -INFINITY;
            }
            float m_g = sc[0];
#pragma unroll
            for (int jj = 1; jj < kDenseGroup; ++jj) m_g = fmaxf(m_g, sc[jj]);
            const float m_new = fmaxf(m_run, m_g);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float lsum = 0.0f;
#pragma unroll
            for (int jj = 0; jj < kDenseGroup; ++jj) {
                sc[jj] = __builtin_amdgcn_exp2f(sc[jj] - m_new);
                lsum += sc[jj];
            }
            l_run = l_run * alpha + lsum;
            m_run = m_new;
#pragma unroll
            for (int r = 0; r < 8; ++r) { acc1[r] *= alpha; acc2[r] *= alpha; }
#pragma unroll
            for (int jj = 0; jj < kDenseGroup; ++jj) {
                // the row index is clamped to the last valid token, whose weight is then zero in
                // this slot: rows past the end may hold anything (0 * NaN is NaN)
                const int j = j0 + min(jj, nt - 1);
                const float pj = jj < nt ? sc[jj] : 0.0f;
                const size_t row = (block_id(p.pages, p.cap >> 6, bc, (t0 + j) >> 6) * 64 + ((t0 + j) & 63)) * W + col;
                float v1[8], v2[8];
                load8<K>(p.v, row, v1);
                load8<K>(p.v, row + NF, v2);
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    acc1[r] = fmaf(pj, v1[r], acc1[r]);
                    acc2[r] = fmaf(pj, v2[r], acc2[r]);
                }
            }
        }
    }

    if (hok) {
        const size_t part = ((size_t)b * p.S + split) * H + h;
        if (c == 0) {
            p.ws_ml[part * 2 + 0] = m_run;
            p.ws_ml[part * 2 + 1] = l_run;
        }
        float* a = p.ws_acc + part * D;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            a[8 * c + r] = acc1[r];
            a[NF + 8 * c + r] = acc2[r];
        }
    }
}

template <int D, int K>
static hipError_t launch_dense_t(const DenseDecodeParams& p, hipStream_t st) {
    constexpr int HPW = 64 / (D / 16);
    const int waves = (p.H + HPW - 1) / HPW;
    hipLaunchKernelGGL((dense_decode_split<D, K>), dim3(p.S, p.B), dim3(64 * waves), 0, st, p);
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
