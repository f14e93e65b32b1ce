// prefill.hip -- key side of chunked (prefill) attention over the latent cache (gfx950).
//
// A chunk of queries per sequence attends causally to the latent cache (Zhou, STAR-KV reading
// notes, Algorithm 2 steps 4-7 applied to every query of the chunk; section 5.3): query l of
// sequence b, at position pos0 + l, scores every cached token n <= pos0 + l,
//   s_{l,h,n} = scale * q_{l,h} . RoPE_n(Z_k[h][n] B_k[h]).
// One workgroup takes 32 queries of one head of one sequence; its four waves walk the 32-token key
// tiles. For each key tile a wave
//   1. rebuilds K~^T = B_k^T Z_k^T on MFMA 32x32x16 (factor fragments staged in LDS once),
//   2. rotates each key to its position in fp32 (R_n = R_{n0} R_j: the lane's constant rotation by
//      j*theta from an LDS table, then the tile's rotation by n0*theta),
//   3. splits the rotated keys into binary16 hi + lo parts (scaled per tile by a power of two) and
//      forms S^T = K Q^T on MFMA as K_hi Q_hi + K_hi Q_lo + K_lo Q_hi, with the query tile staged
//      the same way in LDS: about 2^-22 relative error, the accuracy of the fp32 dot of the decode
//      kernel,
//   4. masks keys past each query's position, and writes the probabilities of the tile relative
//      to each query's tile maximum (rounded up to an integer in log2 units) plus the tile
//      statistics (m_t, l_t) -- the workspace layout the value kernel reads for query rows.
// The values then go through the value kernel (queries of a sequence stacked as query rows, the
// value latent streamed once per group of rows) and the per-head output step.

#include "common.hpp"

namespace starkv {

namespace {

constexpr int kPfWaves = 4;
constexpr int kPfQueries = 32;                 // queries per workgroup
constexpr int kPfMaxFrag = 128 * 128;          // B_k elements of one head (rank <= d <= 128)

__device__ __forceinline__ void pf_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// 2^e with max * 2^e in [2^13, 2^14) (1 for max == 0): binary16 hi + lo parts of values scaled
// so keep about 22 significant bits for every value above 2^-16 of the maximum
__device__ __forceinline__ int pf_scale_exp(float mx) {
    if (!(mx > 0.0f)) return 0;
    int e;
    frexpf(mx, &e);                             // mx in [2^(e-1), 2^e)
    return max(-120, min(120, 14 - e));
}

}  // namespace

template <int D, int K, bool QK>
__global__ __launch_bounds__(64 * kPfWaves, 2) void prefill_scores(const PrefillParams p) {
    constexpr int NF = D / 2;            // RoPE frequencies
    constexpr int HMT = D / 64;          // m-tile pairs (mt, mt + HMT)
    constexpr int MT = D / 32;           // m-tiles of the rebuilt keys
    constexpr int KSTEPS = D / 16;       // contraction steps of S^T = K Q^T
    constexpr int MAXKS = D / 16;        // rank steps (ranks <= d)
    using Fr = typename Elem<K>::frag;
    using T = typename Elem<K>::storage;

    __shared__ __attribute__((aligned(32))) T s_bk[kPfMaxFrag];
    // query fragments, B operand of S^T: lane l holds column (query) l % 32 and, for step ks =
    // 2*mt + s, dims 32*mt + 16*s + 4*(l/32) + {0..3} then 32*mt + 16*s + 8 + 4*(l/32) + {0..3}
    // (the rows a lane of the key rebuild holds, so the rebuilt keys are used in place)
    __shared__ __attribute__((aligned(16))) _Float16 s_qh[KSTEPS * 64 * 8], s_ql[KSTEPS * 64 * 8];
    // cos / sin of j*theta_i for lane l (j = l % 32), frequencies i = 32*pp + 8*g + 4*(l/32) + r:
    // entry [pp*4 + g][l] holds r = 0..3
    __shared__ __attribute__((aligned(16))) f32x4 s_cj[HMT * 4][64], s_sj[HMT * 4][64];
    __shared__ __attribute__((aligned(16))) float s_c0[kPfWaves][64], s_s0[kPfWaves][64];
    __shared__ double s_rev[64];
    __shared__ float s_qmax[kPfWaves];
    __shared__ int s_goff[QK ? MAXKS : 1], s_gn[QK ? MAXKS : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int j = lane & 31;
    const int l0 = blockIdx.x * kPfQueries;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int H = p.H;
    const int clen = p.chunk_lens ? min(max(p.chunk_lens[b], 0), p.chunk) : p.chunk;
    const int nq_here = max(0, min(kPfQueries, clen - l0));
    if (nq_here == 0) return;                   // every query row of the tile is empty
    const int lmax = p.pos0 + l0 + nq_here;     // the longest causal length in the tile
    const int nkb = (lmax + 63) >> 6;           // key blocks the tile's rows read
    const int rk = p.rank[h], sr = p.srank[h], so = p.soff[h], nks = rk >> 4;
    const int kgrp = p.koff[h] >> 4;
    const int Rk = p.Rk;
    const size_t kgroups = (size_t)(Rk >> 4);
    // mixed 4/3-bit cache: the sequence's complete groups below its fill are codes
    const int fill = p.pos0 + clen;
    const int full_blocks = QK ? fill >> 6 : nkb;
    const T* __restrict__ zk = static_cast<const T*>(p.zk);
    const T* __restrict__ bkg = static_cast<const T*>(p.bk);

    if (tid < 64) s_rev[tid] = tid < NF ? p.rope_rev[tid] : 0.0;
    if (QK && tid < MAXKS) {
        const int g16 = min(kgrp + tid, (int)kgroups - 1);
        s_goff[tid] = p.ql.goff[g16];
        s_gn[tid] = p.ql.gn[g16];
    }
    // largest |scaled query| of the tile (power-of-two scale of its hi / lo parts)
    {
        float m = 0.0f;
        for (int e = tid; e < nq_here * D; e += 64 * kPfWaves) {
            const int qc = e / D, dim = e - qc * D;
            m = fmaxf(m, fabsf(p.q[(((size_t)b * p.chunk + l0 + qc) * H + h) * D + dim] * p.q_scale));
        }
        m = wave_max(m);
        if (lane == 0) s_qmax[wave] = m;
    }
    __syncthreads();
    // the lane table of the constant rotation by j*theta
    for (int e = tid; e < HMT * 4 * 64 * 4; e += 64 * kPfWaves) {
        const int r = e & 3, l = (e >> 2) & 63, pg = e >> 8;
        const int i = 32 * (pg >> 2) + 8 * (pg & 3) + 4 * (l >> 5) + r;
        const double rev = (double)(l & 31) * s_rev[i];
        float c, sn;
        sincos_rev((float)(rev - floor(rev)), &c, &sn);
        s_cj[pg][l][r] = c;
        s_sj[pg][l][r] = sn;
    }
    // B_k rows of the head into MFMA A-operand fragment order (as the decode score kernel):
    // fragment f = mt*(rank/16) + ks, lane l holds rows 16*ks + 8*(l/32) + jj at column
    // 32*mt + l%32; rows past the head's true rank are zero
    for (int i = tid; i < (rk >> 3) * D; i += 64 * kPfWaves) {
        const int k8 = i / D, dim = i - k8 * D;
        struct __attribute__((aligned(16))) Run { T v[8]; } run;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int k = 8 * k8 + jj;
            run.v[jj] = k < sr ? bkg[(size_t)(so + k) * D + dim] : T(0);
        }
        *reinterpret_cast<Run*>(s_bk + (((dim >> 5) * nks + (k8 >> 1)) * 64 + (k8 & 1) * 32 + (dim & 31)) * 8) = run;
    }
    // query fragments, scaled and split
    float qmx = 0.0f;
#pragma unroll
    for (int w = 0; w < kPfWaves; ++w) qmx = fmaxf(qmx, s_qmax[w]);
    const int eq = pf_scale_exp(qmx);
    const float qs = ldexpf(p.q_scale, eq);
    for (int e = tid; e < KSTEPS * 64 * 8; e += 64 * kPfWaves) {
        const int slot = e & 7, l = (e >> 3) & 63, ks = e >> 9;
        const int qc = l & 31, hh = l >> 5, mt = ks >> 1, s = ks & 1;
        const int dim = 32 * mt + 16 * s + (slot < 4 ? 4 * hh + slot : 8 + 4 * hh + slot - 4);
        const float v = qc < nq_here ? p.q[(((size_t)b * p.chunk + l0 + qc) * H + h) * D + dim] * qs : 0.0f;
        const _Float16 hi = (_Float16)v;
        s_qh[e] = hi;
        s_ql[e] = (_Float16)(v - (float)hi);
    }
    __syncthreads();

    const uint32_t* __restrict__ qcodes = static_cast<const uint32_t*>(p.zk);
    const uint16_t* __restrict__ qmeta = static_cast<const uint16_t*>(p.zk_meta);
    const _Float16* __restrict__ qtail = static_cast<const _Float16*>(p.zk_tail);
    const size_t qblock_words = (size_t)(p.ql.block_bytes >> 2);
    _Float16* __restrict__ Pout = static_cast<_Float16*>(p.P);
    const int qc = lane & 31;                   // this lane's query column in S^T
    const int lq = l0 + qc;
    const int qlen = lq < clen ? p.pos0 + lq + 1 : 0;
    const size_t prow = ((size_t)b * p.chunk + lq) * H + h;     // (query row, head)

    for (int kt = wave; kt < 2 * nkb; kt += kPfWaves) {
        const int blk = kt >> 1, nt = kt & 1, n0 = 32 * kt;
        if (lane < NF) {
            const double rev = (double)n0 * s_rev[lane];
            float c, sn;
            sincos_rev((float)(rev - floor(rev)), &c, &sn);
            s_c0[wave][lane] = c;
            s_s0[wave][lane] = sn;
        }
        pf_wave_sync();
        // the 32 keys' latent fragments: lane column j = key n0 + j, eight ranks per lane
        Fr z[MAXKS];
        if constexpr (QK) {
            if (blk >= full_blocks) {
                // partial last group of a mixed cache: binary16 rows of the tail [B][64][Rk]
                const _Float16* rowp = qtail + ((size_t)b * 64 + 32 * nt + j) * Rk + 16 * kgrp + 8 * half;
#pragma unroll
                for (int ks = 0; ks < MAXKS; ++ks)
                    z[ks] = load_frag<kF16>(rowp, (size_t)16 * min(ks, nks - 1));
            } else {
                const size_t bid = block_id(p.pages, p.nblk_cap, b, blk);
                const uint32_t* blkw = qcodes + bid * qblock_words;
                const uint16_t* meta = qmeta + bid * 2 * (size_t)Rk;
#pragma unroll
                for (int ks = 0; ks < MAXKS; ++ks) {
                    const int kk = min(ks, nks - 1);
                    const int n = s_gn[kk];
                    const int c0 = 16 * (kgrp + kk) + 8 * half;
                    const u32x4 sc = *reinterpret_cast<const u32x4*>(meta + c0);
                    const u32x4 zc = *reinterpret_cast<const u32x4*>(meta + Rk + c0);
                    const int rb = 8 * s_goff[kk] + (32 * nt + j) * (48 + n);
                    const uint32_t* wp = blkw + (rb >> 5);
                    z[ks] = q43_key_frag(wp[0], wp[1], wp[2], rb & 31, n, half, sc, zc);
                }
            }
        } else {
            const size_t base = (block_id(p.pages, p.nblk_cap, b, blk) * kgroups + kgrp) * 1024 + (size_t)j * 16 +
                                8 * half + nt * 512;
#pragma unroll
            for (int ks = 0; ks < MAXKS; ++ks) z[ks] = load_frag<K>(zk, base + (size_t)min(ks, nks - 1) * 1024);
        }
        // rebuild and rotate
        f32x16 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mt][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < MAXKS; ++ks) {
            if (ks < nks) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt] = mma32<K>(*reinterpret_cast<const Fr*>(s_bk + ((mt * nks + ks) * 64 + lane) * 8), z[ks], acc[mt]);
            }
        }
        float mx = 0.0f;
#pragma unroll
        for (int pp = 0; pp < HMT; ++pp)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int i0 = 32 * pp + 8 * g + 4 * half;
                const f32x4 cj = s_cj[pp * 4 + g][lane], sj = s_sj[pp * 4 + g][lane];
                const f32x4 c0 = *reinterpret_cast<const f32x4*>(&s_c0[wave][i0]);
                const f32x4 s0 = *reinterpret_cast<const f32x4*>(&s_s0[wave][i0]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float a = acc[pp][4 * g + r], bb = acc[pp + HMT][4 * g + r];
                    // by j*theta, then by n0*theta: the key at position n0 + j
                    const float a1 = fmaf(-bb, sj[r], a * cj[r]), b1 = fmaf(a, sj[r], bb * cj[r]);
                    const float a2 = fmaf(-b1, s0[r], a1 * c0[r]), b2 = fmaf(a1, s0[r], b1 * c0[r]);
                    acc[pp][4 * g + r] = a2;
                    acc[pp + HMT][4 * g + r] = b2;
                    mx = fmaxf(mx, fmaxf(fabsf(a2), fabsf(b2)));
                }
            }
        mx = wave_max(mx);
        const int ek = pf_scale_exp(mx);
        const float ks_ = ldexpf(1.0f, ek);
        // S^T = K Q^T: keys on rows, the tile's queries on columns
        f32x16 st;
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = 0.0f;
#pragma unroll
        for (int step = 0; step < KSTEPS; ++step) {
            const int mt = step >> 1, s = step & 1;
            f16x8 kh, kl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = acc[mt][8 * s + e] * ks_;
                kh[e] = (_Float16)v;
                kl[e] = (_Float16)(v - (float)kh[e]);
            }
            const f16x8 qh = *reinterpret_cast<const f16x8*>(s_qh + (step * 64 + lane) * 8);
            const f16x8 ql = *reinterpret_cast<const f16x8*>(s_ql + (step * 64 + lane) * 8);
            st = mma32<kF16>(kh, qh, st);
            st = mma32<kF16>(kh, ql, st);
            st = mma32<kF16>(kl, qh, st);
        }
        const float unscale = ldexpf(1.0f, -ek - eq);
        // lane: query column qc, key rows 8*(r/4) + 4*half + r%4 of the tile
        float v[16];
        float m = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int n = n0 + 8 * (r >> 2) + 4 * half + (r & 3);
            v[r] = n < qlen ? st[r] * unscale : -INFINITY;
            m = fmaxf(m, v[r]);
        }
        {
            const LanePair pr = swap32(m);
            m = fmaxf(pr.a, pr.b);
        }
        // the tile's maximum rounded up to an integer (log2 units): the value kernel's rescaling
        // 2^(m_t - M) of these probabilities is then an exact power of two, so the binary16
        // operand it feeds to the matrix cores carries only the rounding of the stored value
        if (m != -INFINITY) m = ceilf(m);
        float l = 0.0f;
        _Float16 pv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float e = m != -INFINITY ? __builtin_amdgcn_exp2f(v[r] - m) : 0.0f;
            pv[r] = (_Float16)e;
            l += (float)pv[r];          // the sum of the stored values, so that the normaliser
                                        // carries the same rounding as the weights
        }
        l = add_xor32(l);
        if (lq < p.chunk) {
            _Float16* prow_p = Pout + prow * p.Tp + n0 + 4 * half;
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
                const f16x4 w4 = {pv[4 * rg], pv[4 * rg + 1], pv[4 * rg + 2], pv[4 * rg + 3]};
                *reinterpret_cast<f16x4*>(prow_p + 8 * rg) = w4;
            }
            p.stats[(prow * 2 * p.nblk + kt) * 2 + half] = half ? l : m;
        }
        pf_wave_sync();
    }
}

template <int D, int K, bool QK>
static hipError_t launch_prefill_d(const PrefillParams& p, hipStream_t st) {
    const dim3 grid((p.chunk + kPfQueries - 1) / kPfQueries, p.H, p.B);
    hipLaunchKernelGGL((prefill_scores<D, K, QK>), grid, dim3(64 * kPfWaves), 0, st, p);
    return hipGetLastError();
}

// elem: kF16 / kBF16, or -1 for a mixed 4/3-bit key cache (binary16 factors)
hipError_t launch_prefill_scores(const PrefillParams& p, int elem, hipStream_t st) {
    if (p.D == 128) {
        if (elem == kF16) return launch_prefill_d<128, kF16, false>(p, st);
        if (elem == kBF16) return launch_prefill_d<128, kBF16, false>(p, st);
        if (elem == -1) return launch_prefill_d<128, kF16, true>(p, st);
    } else if (p.D == 64) {
        if (elem == kF16) return launch_prefill_d<64, kF16, false>(p, st);
        if (elem == kBF16) return launch_prefill_d<64, kBF16, false>(p, st);
        if (elem == -1) return launch_prefill_d<64, kF16, true>(p, st);
    }
    return hipErrorInvalidValue;
}

// Value side for query rows stacked four at a time (Zhou notes, Algorithm 2 step 6 per query;
// section 5.3: all heads in one operand): Acc[row][h][c] = sum_n p_{row,h,n} 2^(m_t - M) Z_v[n][c]
// over the split's blocks. One workgroup takes four query rows of one sequence and 512 value
// channels; its eight waves own 64 channels each. Per 64-token block the probabilities of the four
// rows (all heads) are rescaled by 2^(m_t - M) once and staged in LDS in MFMA operand order
// (double-buffered), so every wave feeds them to its own channel tiles without repeating the
// rescaling. The tile maxima are integers, so the rescaled binary16 probability is exact (one
// operand); a bfloat16 operand takes it as a hi + lo pair (two MFMAs per fragment). Writes
// (M, L, Acc) per split in the decode workspace layout, read by the output step.
constexpr int kPvWaves = 8;
constexpr int kPvRows = 4;
constexpr int kPvTiles = 2;                            // 32-channel tiles per wave
constexpr int kPvChannels = 32 * kPvTiles * kPvWaves;

template <int K>
__global__ __launch_bounds__(64 * kPvWaves, 1) void prefill_values(const ValueParams p) {
    using Fr = typename Elem<K>::frag;
    using T = typename Elem<K>::storage;
    constexpr bool LO = K == kBF16;                     // a second (lo) operand part
    // [buffer][row][ks][lane][8]: lane l holds head l % 32, tokens 16*ks + 8*(l/32) + 0..7
    __shared__ __attribute__((aligned(16))) T s_ph[2][kPvRows * 4 * 64 * 8], s_pl[2][LO ? kPvRows * 4 * 64 * 8 : 8];
    __shared__ float s_M[kPvRows][kMaxHeads], s_L[kPvRows][kMaxHeads];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int split = blockIdx.x;
    const int chunk = blockIdx.y;
    const int grp = blockIdx.z;
    const int H = p.H;
    const int row0 = grp * kPvRows;
    int seq_len = 0;
#pragma unroll
    for (int qi = 0; qi < kPvRows; ++qi) seq_len = max(seq_len, seq_length(p.seq_lens, row0 + qi, p.seq_len));
    const int bc = cache_seq(p.seq_map, grp, p.cache_batch);
    const int blk_begin = split * p.blocks_per_split;
    const int blk_end = max(blk_begin, min((seq_len + 63) >> 6, blk_begin + p.blocks_per_split));
    const int nb = blk_end - blk_begin;

    // split statistics per (row, head) from the 32-token tile statistics
    for (int hq = wave; hq < kPvRows * H; hq += kPvWaves) {
        const int qi = hq / H, h = hq - qi * H;
        const float* st = p.stats + (((size_t)(row0 + qi) * H + h) * 2 * p.nblk + 2 * blk_begin) * 2;
        float M = -INFINITY;
        for (int i = lane; i < 2 * nb; i += 64) M = fmaxf(M, st[2 * i]);
        M = wave_max(M);
        const float Mc = M != -INFINITY ? M : 0.0f;
        float L = 0.0f;
        for (int i = lane; i < 2 * nb; i += 64) L += tile_factor(st[2 * i] - Mc) * st[2 * i + 1];
        L = wave_sum(L);
        if (lane == 0) { s_M[qi][h] = M; s_L[qi][h] = L; }
    }
    __syncthreads();

    // staging of one block's operands: 512 threads, two 8-token runs each (row, head, run)
    auto stage = [&](int buf, int blk) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int e = tid + it * 64 * kPvWaves;             // (qi, h, u) with u < 8 runs
            const int u = e & 7, h = (e >> 3) & 31, qi = e >> 8;
            const int hh = min(h, H - 1);
            const size_t prow = ((size_t)(row0 + qi) * H + hh) * p.Tp + (size_t)blk * 64 + 8 * u;
            const f16x8 pv = *reinterpret_cast<const f16x8*>(static_cast<const _Float16*>(p.P) + prow);
            const float m = p.stats[(((size_t)(row0 + qi) * H + hh) * 2 * p.nblk + 2 * blk + (u >> 2)) * 2];
            const float M = s_M[qi][hh];
            const float f = h < H ? tile_factor(m - M) : 0.0f;
            const int ks = u >> 1, l = h + 32 * (u & 1);
            const int at = ((qi * 4 + ks) * 64 + l) * 8;
            if constexpr (LO) {
                struct __attribute__((aligned(16))) Run { T v[8]; } rh, rl;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float v = (float)pv[k] * f;
                    const uint16_t hb = float_to_bf16_bits(v);
                    rh.v[k] = hb;
                    rl.v[k] = float_to_bf16_bits(v - bf16_bits_to_float(hb));
                }
                *reinterpret_cast<Run*>(&s_ph[buf][at]) = rh;
                *reinterpret_cast<Run*>(&s_pl[buf][at]) = rl;
            } else {
                const _Float16 fh = (_Float16)f;
                *reinterpret_cast<f16x8*>(&s_ph[buf][at]) = pv * (f16x8){fh, fh, fh, fh, fh, fh, fh, fh};
            }
        }
    };

    // this wave's channels (channels past r_v read a clamped channel and are never stored)
    int ch[kPvTiles];
    size_t zoff[kPvTiles];
    const int cgroups = p.rv >> 4;
#pragma unroll
    for (int k = 0; k < kPvTiles; ++k) {
        ch[k] = ((chunk * kPvWaves + wave) * kPvTiles + k) * 32 + (lane & 31);
        const int cc = min(ch[k], p.rv - 1);
        zoff[k] = (size_t)(cc >> 4) * 1024 + (cc & 15) * 16 + 8 * half;
    }
    f32x16 acc[kPvRows][kPvTiles];
#pragma unroll
    for (int qi = 0; qi < kPvRows; ++qi)
#pragma unroll
        for (int k = 0; k < kPvTiles; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qi][k][r] = 0.0f;

    if (nb > 0) stage(0, blk_begin);
    for (int i = 0; i < nb; ++i) {
        const int blk = blk_begin + i, buf = i & 1;
        __syncthreads();                     // block i staged; block i - 1's operands consumed
        if (i + 1 < nb) stage(buf ^ 1, blk + 1);
        const size_t bbase = block_id(p.pages, p.nblk_cap, bc, blk) * cgroups * 1024;
        Fr z[kPvTiles][4];
#pragma unroll
        for (int k = 0; k < kPvTiles; ++k)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) z[k][ks] = load_frag<K>(p.zv, bbase + zoff[k] + ks * 256);
        if ((blk + 1) * 64 > seq_len) {
            // the group's last block: tokens past its longest row may hold anything (their
            // probabilities are 0, but 0 * NaN is not): zero them
#pragma unroll
            for (int k = 0; k < kPvTiles; ++k)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (blk * 64 + 16 * ks + 8 * half + e >= seq_len) z[k][ks][e] = 0;
        }
#pragma unroll
        for (int qi = 0; qi < kPvRows; ++qi)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int at = ((qi * 4 + ks) * 64 + lane) * 8;
                const Fr ph = *reinterpret_cast<const Fr*>(&s_ph[buf][at]);
#pragma unroll
                for (int k = 0; k < kPvTiles; ++k) acc[qi][k] = mma32<K>(ph, z[k][ks], acc[qi][k]);
                if constexpr (LO) {
                    const Fr pl = *reinterpret_cast<const Fr*>(&s_pl[buf][at]);
#pragma unroll
                    for (int k = 0; k < kPvTiles; ++k) acc[qi][k] = mma32<K>(pl, z[k][ks], acc[qi][k]);
                }
            }
    }

    // (M, L) of the split (one writer per (row, head)), then the wave's channels of Acc
    if (chunk == 0 && tid < kPvRows * H) {
        const int qi = tid / H, h = tid - qi * H;
        float* ml = p.ws_ml + (((size_t)(row0 + qi) * p.S + split) * H + h) * 2;
        ml[0] = s_M[qi][h];
        ml[1] = s_L[qi][h];
    }
#pragma unroll
    for (int k = 0; k < kPvTiles; ++k) {
        if (ch[k] >= p.rv) continue;
#pragma unroll
        for (int qi = 0; qi < kPvRows; ++qi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int h = 8 * (r >> 2) + 4 * half + (r & 3);
                if (h < H) p.ws_acc[(((size_t)(row0 + qi) * p.S + split) * H + h) * p.rv + ch[k]] = acc[qi][k][r];
            }
    }
}

hipError_t launch_prefill_values(const ValueParams& p, int elem, hipStream_t st) {
    const dim3 grid(p.S, (p.rv + kPvChannels - 1) / kPvChannels, p.B / kPvRows);
    if (elem == kF16) hipLaunchKernelGGL(prefill_values<kF16>, grid, dim3(64 * kPvWaves), 0, st, p);
    else if (elem == kBF16) hipLaunchKernelGGL(prefill_values<kBF16>, grid, dim3(64 * kPvWaves), 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// Output step for many query rows (Zhou notes, Algorithm 2 step 7 per row): out[r][h] =
// (sum_s w_{r,h,s} Acc_s[r][h]) B_v[:, h*d:(h+1)*d] with the log-sum-exp split weights w
// (normalised). One workgroup takes 128 rows of one head: wave w owns rows 32w .. 32w+31 and
// all d output columns (d/32 MFMA accumulators). The head's B_v slice is staged in LDS per chunk
// of 32 value channels (read once per 128 rows); each lane forms its row's merged latent values in
// fp32 and feeds them as binary16 hi + lo parts (two MFMAs per fragment: fp32 accuracy).
constexpr int kPpRows = 128;
constexpr int kPpChunk = 32;
constexpr int kPpMaxSplits = 64;

template <int D, int K>
__global__ __launch_bounds__(256, 2) void prefill_project(const ProjectParams p) {
    constexpr int NT = D / 32;
    using T = typename Elem<K>::storage;
    using Fr = typename Elem<K>::frag;
    // B_v rows of the chunk in B-operand fragment order: [nt][step][lane][8]
    __shared__ __attribute__((aligned(16))) T s_bv[NT * 2 * 64 * 8];
    __shared__ float s_w[kPpRows][kPpMaxSplits];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int r0 = blockIdx.x * kPpRows;
    const int h = blockIdx.y;
    const int S = p.S;
    const size_t HD = (size_t)p.H * D;

    // split weights of each row: w_s = 2^(M_s - M) / sum_s 2^(M_s - M) L_s (zeros for an empty row)
    for (int rr = tid; rr < kPpRows; rr += 256) {
        const int row = min(r0 + rr, p.B - 1);
        const float* ml = p.ws_ml + ((size_t)row * S * p.H + h) * 2;
        float M = -INFINITY;
        for (int s = 0; s < S; ++s) M = fmaxf(M, ml[(size_t)s * p.H * 2]);
        if (M == -INFINITY) M = 0.0f;
        float L = 0.0f;
        for (int s = 0; s < S; ++s) L += __builtin_amdgcn_exp2f(ml[(size_t)s * p.H * 2] - M) * ml[(size_t)s * p.H * 2 + 1];
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        for (int s = 0; s < S; ++s) s_w[rr][s] = __builtin_amdgcn_exp2f(ml[(size_t)s * p.H * 2] - M) * inv;
    }

    const int rr = 32 * wave + (lane & 31);          // this lane's row of the A operand
    const int row = min(r0 + rr, p.B - 1);
    f32x16 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;

    for (int c0 = 0; c0 < p.rv; c0 += kPpChunk) {
        __syncthreads();                              // the previous chunk's fragments are read
        // stage B_v[c0 .. c0+31][h*d .. h*d + d): fragment (nt, step), lane l holds column
        // 32*nt + l%32 and channels c0 + 16*step + 8*(l/32) + jj; channels past rv_src are zero
        for (int e = tid; e < NT * 2 * 64; e += 256) {
            const int l = e & 63, st = (e >> 6) & 1, nt = e >> 7;
            const int col = 32 * nt + (l & 31);
            struct __attribute__((aligned(16))) Run { T v[8]; } run;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int c = c0 + 16 * st + 8 * (l >> 5) + jj;
                run.v[jj] = c < p.rv_src ? static_cast<const T*>(p.bv)[(size_t)c * HD + (size_t)h * D + col] : T(0);
            }
            *reinterpret_cast<Run*>(&s_bv[e * 8]) = run;
        }
        __syncthreads();
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            // the lane's row: merged latent values of channels c0 + 16*st + 8*half .. + 7
            const int cb = c0 + 16 * st + 8 * half;
            f32x4 a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = {0.0f, 0.0f, 0.0f, 0.0f};
            if (cb < p.rv) {
                for (int s = 0; s < S; ++s) {
                    const f32x4* src = reinterpret_cast<const f32x4*>(p.ws_acc + (((size_t)row * S + s) * p.H + h) * p.rv + cb);
                    const float w = s_w[rr][s];
                    a0 += w * src[0];
                    a1 += w * src[1];
                }
            }
            Fr ahi, alo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = e < 4 ? a0[e] : a1[e - 4];
                if constexpr (K == kBF16) {
                    const uint16_t hb = float_to_bf16_bits(v);
                    ahi[e] = __builtin_bit_cast(__bf16, hb);
                    alo[e] = __builtin_bit_cast(__bf16, float_to_bf16_bits(v - bf16_bits_to_float(hb)));
                } else {
                    ahi[e] = (_Float16)v;
                    alo[e] = (_Float16)(v - (float)ahi[e]);
                }
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const Fr bf = *reinterpret_cast<const Fr*>(&s_bv[((nt * 2 + st) * 64 + lane) * 8]);
                acc[nt] = mma32<K>(ahi, bf, acc[nt]);
                acc[nt] = mma32<K>(alo, bf, acc[nt]);
            }
        }
    }
    // acc[nt]: rows 32*wave + 8*(r/4) + 4*half + r%4, column 32*nt + lane%32
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int orow = r0 + 32 * wave + 8 * (r >> 2) + 4 * half + (r & 3);
            if (orow < p.B) p.out[((size_t)orow * p.H + h) * D + 32 * nt + (lane & 31)] = acc[nt][r];
        }
}

hipError_t launch_prefill_project(const ProjectParams& p, int elem, hipStream_t st) {
    if (p.S > kPpMaxSplits) return hipErrorInvalidValue;
    const dim3 grid((p.B + kPpRows - 1) / kPpRows, p.H);
    if (p.D == 128) {
        if (elem == kF16) hipLaunchKernelGGL((prefill_project<128, kF16>), grid, dim3(256), 0, st, p);
        else if (elem == kBF16) hipLaunchKernelGGL((prefill_project<128, kBF16>), grid, dim3(256), 0, st, p);
        else return hipErrorInvalidValue;
    } else if (p.D == 64) {
        if (elem == kF16) hipLaunchKernelGGL((prefill_project<64, kF16>), grid, dim3(256), 0, st, p);
        else if (elem == kBF16) hipLaunchKernelGGL((prefill_project<64, kBF16>), grid, dim3(256), 0, st, p);
        else return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void prefill_rows(const PrefillRowsParams p) {
    const int row = blockIdx.x * 256 + threadIdx.x;
    if (row >= p.B * p.chunk) return;
    const int b = row / p.chunk, l = row - b * p.chunk;
    const int clen = p.chunk_lens ? min(max(p.chunk_lens[b], 0), p.chunk) : p.chunk;
    p.row_len[row] = l < clen ? p.pos0 + l + 1 : 0;
    p.row_fill[row] = p.pos0 + clen;
    if (row % p.nq == 0) p.group_seq[row / p.nq] = b;
}

hipError_t launch_prefill_rows(const PrefillRowsParams& p, hipStream_t st) {
    const int rows = p.B * p.chunk;
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_rows, dim3((rows + 255) / 256), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace starkv
