// latent_decode.hip -- decode attention straight from a low-rank latent KV cache (gfx950).
//
// Computes, for every sequence b and head h (Zhou, STAR-KV reading notes, Algorithm 2 steps 4-7
// and section 5.3):
//   s_n   = scale * q_h . RoPE_n(Z_k[h][n] B_k[h])        keys rebuilt per tile in registers
//   p     = softmax_n(s)                                  online over tiles, split-K over n
//   out_h = (sum_n p_n Z_v[n]) B_v[:, h*d:(h+1)*d]        values summed in latent space
// No full-width K or V is ever written to memory.
//
// Kernel 1 (latent_decode_split): one workgroup per (split, sequence), 8 waves. For each 64-token
// tile of its split:
//   * RoPE table: cos/sin of n*theta_i for the tile's 64 positions into LDS (angles in fp64,
//     reduced to one revolution, then the hardware sin/cos).
//   * key phase: waves 0-3 take tokens 0-31 of the tile, waves 4-7 tokens 32-63; each wave owns a
//     rank-balanced subset of heads. Per head, K~^T (d x 32 tokens) = B_k[h]^T Z_k[h]^T on MFMA
//     32x32x16 (A = packed factor fragments, B = latent rows loaded straight from HBM), then the
//     rotate-half RoPE and the dot with q are done in registers: a lane holds 64 of the 128
//     reconstructed dims of one token, with each RoPE partner (i, i+d/2) in the same lane, so the
//     dot needs one cross-half swap. Scores (log2 domain) go to LDS.
//   * softmax phase: each head's 64 scores are reduced with wave shuffles; running max/sum are
//     kept per head; probabilities (fp16 for fp16 caches, hi+lo bf16 pair for bf16, fp32 for fp32)
//     go to LDS with the rescale factor of the running accumulator.
//   * value phase: Acc[H x r_v] += P[H x 64] Z_v[64 x r_v] on MFMA, all heads in one contraction
//     (the stacking of the notes' section 5.3); wave w owns r_v columns 32*(w + 8k). Z_v is stored
//     channel-major inside each 64-token block so every lane loads 8 consecutive tokens of one
//     channel with one 16-byte load.
//   At the end the split's (max, sum, Acc) partial goes to the workspace.
// Kernel 2 (merge_splits): log-sum-exp weighted merge of the splits per (b, h), normalised.
// Kernel 3 (project_heads): out[b][h] = a[b][h] . B_v[:, h*d:(h+1)*d] for all b at once.

#include "common.hpp"

namespace starkv {

// ------------------------------------------------------------------------------------------------
// Probability tile storage in LDS, per element kind, and the value-side MFMA that consumes it.
// Row = head (32 rows), column = token in tile (64).
// ------------------------------------------------------------------------------------------------
template <int K> struct ProbTile;

template <> struct ProbTile<kF16> {
    static constexpr int kStride = kTile + 8;                // halves per row (144 bytes)
    _Float16 p[kMaxHeads * kStride];
    __device__ void zero(int tid, int nthreads) {
        for (int i = tid; i < kMaxHeads * kStride; i += nthreads) p[i] = (_Float16)0.0f;
    }
    __device__ void store(int h, int t, float v) { p[h * kStride + t] = (_Float16)v; }
    __device__ f32x16 mma(int row, int tcol, const f16x8& z, f32x16 acc) const {
        f16x8 a = *reinterpret_cast<const f16x8*>(&p[row * kStride + tcol]);
        return mma32<kF16>(a, z, acc);
    }
};

template <> struct ProbTile<kBF16> {
    // p = hi + lo with both parts bf16: the pair carries ~16 significant bits, so the bf16 path
    // keeps the probabilities as precise as the fp16 path does.
    static constexpr int kStride = kTile + 8;
    uint16_t hi[kMaxHeads * kStride];
    uint16_t lo[kMaxHeads * kStride];
    __device__ void zero(int tid, int nthreads) {
        for (int i = tid; i < kMaxHeads * kStride; i += nthreads) { hi[i] = 0; lo[i] = 0; }
    }
    __device__ void store(int h, int t, float v) {
        uint16_t a = float_to_bf16_bits(v);
        hi[h * kStride + t] = a;
        lo[h * kStride + t] = float_to_bf16_bits(v - bf16_bits_to_float(a));
    }
    __device__ f32x16 mma(int row, int tcol, const bf16x8& z, f32x16 acc) const {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(&hi[row * kStride + tcol]);
        bf16x8 b = *reinterpret_cast<const bf16x8*>(&lo[row * kStride + tcol]);
        acc = mma32<kBF16>(a, z, acc);
        return mma32<kBF16>(b, z, acc);
    }
};

template <> struct ProbTile<kF32> {
    static constexpr int kStride = kTile + 4;
    float p[kMaxHeads * kStride];
    __device__ void zero(int tid, int nthreads) {
        for (int i = tid; i < kMaxHeads * kStride; i += nthreads) p[i] = 0.0f;
    }
    __device__ void store(int h, int t, float v) { p[h * kStride + t] = v; }
    __device__ f32x16 mma(int row, int tcol, const f32x8& z, f32x16 acc) const {
        const f32x4* src = reinterpret_cast<const f32x4*>(&p[row * kStride + tcol]);
        f32x4 a0 = src[0], a1 = src[1];
        f32x8 a;
        for (int i = 0; i < 4; ++i) { a[i] = a0[i]; a[4 + i] = a1[i]; }
        return mma32<kF32>(a, z, acc);
    }
};

// ------------------------------------------------------------------------------------------------
// Kernel 1
// ------------------------------------------------------------------------------------------------
template <int D, int NTV, int K>
__global__ __launch_bounds__(512, 1) void latent_decode_split(const LatentDecodeParams p) {
    constexpr int MT = D / 32;          // 32-row tiles of head dims
    constexpr int HMT = MT / 2;         // tiles holding the first half of the dims
    constexpr int NF = D / 2;           // RoPE frequencies
    constexpr int TRIG_STRIDE = 2 * NF + 4;
    constexpr int SC_STRIDE = kTile + 4;
    using Fr = typename Elem<K>::frag;

    __shared__ __attribute__((aligned(16))) float s_trig[kTile * TRIG_STRIDE];
    __shared__ __attribute__((aligned(16))) float s_q[kMaxHeads * D];
    __shared__ __attribute__((aligned(16))) float s_score[kMaxHeads * SC_STRIDE];
    __shared__ __attribute__((aligned(16))) float s_alpha[kMaxHeads];
    __shared__ __attribute__((aligned(16))) ProbTile<K> s_p;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int split = blockIdx.x;
    const int b = blockIdx.y;
    const int H = p.H, rv = p.rv;
    const int ntiles = (p.seq_len + kTile - 1) / kTile;
    const int tile_begin = split * p.tiles_per_split;
    const int tile_end = min(ntiles, tile_begin + p.tiles_per_split);

    for (int i = tid; i < H * D; i += 512) s_q[i] = p.q[(size_t)b * H * D + i] * p.q_scale;
    s_p.zero(tid, 512);
    if (tid < kMaxHeads) s_alpha[tid] = 1.0f;

    float m_run[4], l_run[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { m_run[j] = -INFINITY; l_run[j] = 0.0f; }
    f32x16 accv[NTV];
#pragma unroll
    for (int k = 0; k < NTV; ++k)
        for (int r = 0; r < 16; ++r) accv[k][r] = 0.0f;
    __syncthreads();

    const int st = wave / kKeyWaveGroups;     // key sub-tile (32 tokens)
    const int grp = wave % kKeyWaveGroups;
    const int nsched = p.sched_n[grp];
    const int tok = 32 * st + (lane & 31);    // this lane's token inside the tile (key phase)
    const size_t nblk = (size_t)p.cap / kTile;

    for (int tile = tile_begin; tile < tile_end; ++tile) {
        const int t0 = tile * kTile;

        // ---- RoPE table for positions t0 .. t0+63 ----
        for (int e = tid; e < kTile * NF; e += 512) {
            const int j = e / NF, i = e - j * NF;
            const double rev = (double)(t0 + j) * p.rope_rev[i];
            const float x = (float)(rev - floor(rev));
            float c, s;
            sincos_rev(x, &c, &s);
            s_trig[j * TRIG_STRIDE + 2 * i] = c;
            s_trig[j * TRIG_STRIDE + 2 * i + 1] = s;
        }
        __syncthreads();

        // ---- key phase ----
        {
            float tc[HMT][4][4], ts[HMT][4][4];
#pragma unroll
            for (int mt = 0; mt < HMT; ++mt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4* row = reinterpret_cast<const f32x4*>(
                        &s_trig[tok * TRIG_STRIDE + 2 * (32 * mt + 8 * g + 4 * half)]);
                    const f32x4 v0 = row[0], v1 = row[1];
                    tc[mt][g][0] = v0[0]; ts[mt][g][0] = v0[1];
                    tc[mt][g][1] = v0[2]; ts[mt][g][1] = v0[3];
                    tc[mt][g][2] = v1[0]; ts[mt][g][2] = v1[1];
                    tc[mt][g][3] = v1[2]; ts[mt][g][3] = v1[3];
                }
            const bool valid = (t0 + tok) < p.seq_len;
            const size_t zrow = ((size_t)b * p.cap + t0 + tok) * p.Rk;
            for (int si = 0; si < nsched; ++si) {
                const int h = p.sched[grp][si];
                const int ko = p.koff[h];
                const int nks = p.rank[h] >> 4;
                f32x16 acc[MT];
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    for (int r = 0; r < 16; ++r) acc[mt][r] = 0.0f;
                const size_t fbase = (size_t)ko * D;
                for (int ks = 0; ks < nks; ++ks) {
                    const Fr bz = load_frag<K>(p.zk, zrow + ko + 16 * ks + 8 * half);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const Fr a = load_frag<K>(p.bkt, fbase + ((size_t)(mt * nks + ks) * 64 + lane) * 8);
                        acc[mt] = mma32<K>(a, bz, acc[mt]);
                    }
                }
                const float* qh = &s_q[h * D];
                float sc = 0.0f;
#pragma unroll
                for (int mt = 0; mt < HMT; ++mt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int i0 = 32 * mt + 8 * g + 4 * half;
                        const f32x4 q1 = *reinterpret_cast<const f32x4*>(&qh[i0]);
                        const f32x4 q2 = *reinterpret_cast<const f32x4*>(&qh[i0 + NF]);
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) {
                            const float a = acc[mt][4 * g + r4], bb = acc[mt + HMT][4 * g + r4];
                            const float c = tc[mt][g][r4], s = ts[mt][g][r4];
                            sc += q1[r4] * (a * c - bb * s) + q2[r4] * (bb * c + a * s);
                        }
                    }
                sc += __shfl_xor(sc, 32, 64);
                if (lane < 32) s_score[h * SC_STRIDE + tok] = valid ? sc : -INFINITY;
            }
        }
        __syncthreads();

        // ---- softmax phase: wave w owns heads w, w+8, w+16, w+24 ----
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int h = wave + 8 * j;
            if (h < H) {
                const float v = s_score[h * SC_STRIDE + lane];
                const float m_new = fmaxf(m_run[j], wave_max(v));
                const float alpha = __builtin_amdgcn_exp2f(m_run[j] - m_new);
                const float pr = __builtin_amdgcn_exp2f(v - m_new);
                l_run[j] = l_run[j] * alpha + wave_sum(pr);
                m_run[j] = m_new;
                s_p.store(h, lane, pr);
                if (lane == 0) s_alpha[h] = alpha;
            }
        }
        __syncthreads();

        // ---- value phase ----
        const bool partial = (t0 + kTile) > p.seq_len;
#pragma unroll
        for (int k = 0; k < NTV; ++k) {
            const int nt = wave + 8 * k;
            if (nt * 32 < rv) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 al = *reinterpret_cast<const f32x4*>(&s_alpha[8 * g + 4 * half]);
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) accv[k][4 * g + r4] *= al[r4];
                }
                const int ch = nt * 32 + (lane & 31);
                const bool ch_ok = ch < rv;
                const size_t zvb = (((size_t)b * nblk + tile) * rv + (ch_ok ? ch : 0)) * kTile;
#pragma unroll
                for (int ks = 0; ks < kTile / 16; ++ks) {
                    const int tt = 16 * ks + 8 * half;
                    Fr z = ch_ok ? load_frag<K>(p.zv, zvb + tt) : zero_frag<K>();
                    if (partial) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (t0 + tt + e >= p.seq_len) z[e] = 0;
                    }
                    accv[k] = s_p.mma(lane & 31, tt, z, accv[k]);
                }
            }
        }
    }

    // ---- partial results of this split ----
    const size_t part = (size_t)b * p.S + split;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int h = wave + 8 * j;
        if (h < H && lane == 0) {
            p.ws_ml[(part * H + h) * 2 + 0] = m_run[j];
            p.ws_ml[(part * H + h) * 2 + 1] = l_run[j];
        }
    }
#pragma unroll
    for (int k = 0; k < NTV; ++k) {
        const int nt = wave + 8 * k;
        const int ch = nt * 32 + (lane & 31);
        if (nt * 32 < rv && ch < rv) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int h = acc_row(r, lane);
                if (h < H) p.ws_acc[(part * H + h) * rv + ch] = accv[k][r];
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Kernel 2: log-sum-exp merge of the splits, one workgroup per (b, h). Row width W.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_splits(const MergeParams p) {
    __shared__ float s_w[256];
    __shared__ float s_inv_l;
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh - b * p.H;
    const int S = p.active_splits;
    if (threadIdx.x == 0) {
        float M = -INFINITY;
        for (int s = 0; s < S; ++s) M = fmaxf(M, p.ws_ml[(((size_t)b * p.S + s) * p.H + h) * 2]);
        float L = 0.0f;
        for (int s = 0; s < S; ++s) {
            const size_t o = (((size_t)b * p.S + s) * p.H + h) * 2;
            const float w = __builtin_amdgcn_exp2f(p.ws_ml[o] - M);
            s_w[s] = w;
            L += w * p.ws_ml[o + 1];
        }
        s_inv_l = 1.0f / L;
    }
    __syncthreads();
    const float inv_l = s_inv_l;
    for (int c = threadIdx.x; c < p.W; c += 256) {
        float a = 0.0f;
        for (int s = 0; s < S; ++s) a += s_w[s] * p.ws_acc[(((size_t)b * p.S + s) * p.H + h) * p.W + c];
        p.ws_a[((size_t)b * p.H + h) * p.W + c] = a * inv_l;
    }
}

// ------------------------------------------------------------------------------------------------
// Kernel 3: out[b][h][j0..j0+15] = sum_c a[b][h][c] * B_v[c][h*D + j], all b (chunks of 32).
// Thread (cs = tid / 16, jj = tid % 16) sums channels c = cs + 16*k; LDS reduces over cs.
// ------------------------------------------------------------------------------------------------
template <int K>
__device__ __forceinline__ float load_scalar(const void* base, size_t i);
template <> __device__ __forceinline__ float load_scalar<kF32>(const void* base, size_t i) {
    return static_cast<const float*>(base)[i];
}
template <> __device__ __forceinline__ float load_scalar<kF16>(const void* base, size_t i) {
    return (float)static_cast<const _Float16*>(base)[i];
}
template <> __device__ __forceinline__ float load_scalar<kBF16>(const void* base, size_t i) {
    return bf16_bits_to_float(static_cast<const uint16_t*>(base)[i]);
}

template <int K>
__global__ __launch_bounds__(256) void project_heads(const ProjectParams p) {
    constexpr int BCH = 32;
    __shared__ float s_red[16][BCH][17];
    const int h = blockIdx.x;
    const int j0 = blockIdx.y * 16;
    const int tid = threadIdx.x;
    const int jj = tid & 15, cs = tid >> 4;
    const size_t HD = (size_t)p.H * p.D;
    for (int b0 = 0; b0 < p.B; b0 += BCH) {
        const int nb = min(BCH, p.B - b0);
        float acc[BCH];
#pragma unroll
        for (int i = 0; i < BCH; ++i) acc[i] = 0.0f;
        for (int c = cs; c < p.rv; c += 16) {
            const float w = load_scalar<K>(p.bv, (size_t)c * HD + (size_t)h * p.D + j0 + jj);
            const float* arow = p.ws_a + ((size_t)b0 * p.H + h) * p.rv + c;
#pragma unroll
            for (int i = 0; i < BCH; ++i)
                if (i < nb) acc[i] += arow[(size_t)i * p.H * p.rv] * w;
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) s_red[cs][i][jj] = acc[i];
        __syncthreads();
        for (int e = tid; e < nb * 16; e += 256) {
            const int i = e >> 4, j = e & 15;
            float v = 0.0f;
            for (int k = 0; k < 16; ++k) v += s_red[k][i][j];
            p.out[((size_t)(b0 + i) * p.H + h) * p.D + j0 + j] = v;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------------
// Packing of the key factors into MFMA A-operand fragments: for head h (rank r, offset ko),
// fragment (mt, ks) lane l holds B_k[ko + 16*ks + 8*(l/32) + j][32*mt + l%32], j = 0..7, stored
// at ((ko*D) + ((mt*(r/16) + ks)*64 + l)*8 + j). One workgroup per head.
// ------------------------------------------------------------------------------------------------
struct PackParams {
    const void* bk;
    void* bkt;
    int D, H;
    int16_t koff[kMaxHeads + 1];
    int16_t rank[kMaxHeads];
};

template <int K>
__global__ __launch_bounds__(256) void pack_key_factors(const PackParams p) {
    using T = typename Elem<K>::storage;
    const int h = blockIdx.x;
    const int ko = p.koff[h], nks = p.rank[h] >> 4;
    const int total = p.D * p.rank[h];
    const T* src = static_cast<const T*>(p.bk);
    T* dst = static_cast<T*>(p.bkt) + (size_t)ko * p.D;
    for (int idx = threadIdx.x; idx < total; idx += 256) {
        const int j = idx & 7;
        const int l = (idx >> 3) & 63;
        const int frag = idx >> 9;           // mt * nks + ks
        const int mt = frag / nks, ks = frag - mt * nks;
        const int dim = 32 * mt + (l & 31);
        const int rr = 16 * ks + 8 * (l >> 5) + j;
        dst[idx] = src[(size_t)(ko + rr) * p.D + dim];
    }
}

// ------------------------------------------------------------------------------------------------
// Host launchers
// ------------------------------------------------------------------------------------------------
template <int D, int NTV, int K>
static hipError_t launch_split_t(const LatentDecodeParams& p, hipStream_t st) {
    hipLaunchKernelGGL((latent_decode_split<D, NTV, K>), dim3(p.S, p.B), dim3(512), 0, st, p);
    return hipGetLastError();
}

template <int D, int K>
static hipError_t launch_split_d(const LatentDecodeParams& p, int ntv, hipStream_t st) {
    switch (ntv) {
    case 1: return launch_split_t<D, 1, K>(p, st);
    case 2: return launch_split_t<D, 2, K>(p, st);
    case 3: return launch_split_t<D, 3, K>(p, st);
    case 4: return launch_split_t<D, 4, K>(p, st);
    case 5: return launch_split_t<D, 5, K>(p, st);
    default: return hipErrorInvalidValue;
    }
}

template <int K>
static hipError_t launch_split_k(const LatentDecodeParams& p, int ntv, hipStream_t st) {
    if (p.D == 128) return launch_split_d<128, K>(p, ntv, st);
    if (p.D == 64) return launch_split_d<64, K>(p, ntv, st);
    return hipErrorInvalidValue;
}

hipError_t launch_latent_split(const LatentDecodeParams& p, int elem, int ntv, hipStream_t st) {
    switch (elem) {
    case kF32: return launch_split_k<kF32>(p, ntv, st);
    case kF16: return launch_split_k<kF16>(p, ntv, st);
    case kBF16: return launch_split_k<kBF16>(p, ntv, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_merge(const MergeParams& p, hipStream_t st) {
    hipLaunchKernelGGL(merge_splits, dim3(p.B * p.H), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_project(const ProjectParams& p, int elem, hipStream_t st) {
    const dim3 grid(p.H, p.D / 16);
    switch (elem) {
    case kF32: hipLaunchKernelGGL(project_heads<kF32>, grid, dim3(256), 0, st, p); break;
    case kF16: hipLaunchKernelGGL(project_heads<kF16>, grid, dim3(256), 0, st, p); break;
    case kBF16: hipLaunchKernelGGL(project_heads<kBF16>, grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pack_keys(const void* bk, void* bkt, int D, int H, const int16_t* koff,
                            const int16_t* rank, int elem, hipStream_t st) {
    PackParams p;
    p.bk = bk;
    p.bkt = bkt;
    p.D = D;
    p.H = H;
    for (int h = 0; h <= H; ++h) p.koff[h] = koff[h];
    for (int h = 0; h < H; ++h) p.rank[h] = rank[h];
    switch (elem) {
    case kF32: hipLaunchKernelGGL(pack_key_factors<kF32>, dim3(H), dim3(256), 0, st, p); break;
    case kF16: hipLaunchKernelGGL(pack_key_factors<kF16>, dim3(H), dim3(256), 0, st, p); break;
    case kBF16: hipLaunchKernelGGL(pack_key_factors<kBF16>, dim3(H), dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace starkv
