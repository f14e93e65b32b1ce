// latent_decode.hip -- decode attention straight from a low-rank latent KV cache (gfx950).
//
// Computes, for every sequence b and head h (Zhou, STAR-KV reading notes, Algorithm 2 steps 4-7
// and section 5.3):
//   s_n   = scale * q_h . RoPE_n(Z_k[h][n] B_k[h])        keys rebuilt per tile in registers
//   p     = softmax_n(s)
//   out_h = (sum_n p_n Z_v[n]) B_v[:, h*d:(h+1)*d]        values summed in latent space
// No full-width K or V is ever written to memory.
//
// Three kernels per call:
//  1. latent_scores: one workgroup per (split of the sequence, head group, sequence). The group's
//     B_k rows are staged once in LDS in MFMA fragment order (zero rows where a rank was rounded
//     up to 16); each wave walks 64-token blocks and, per head,
//     rebuilds K~^T (d x 64 tokens) = B_k^T Z_k^T on MFMA 32x32x16 (A = factor fragments from
//     LDS, B = latent fragments streamed from HBM one unit ahead in registers), applies RoPE and
//     the dot with q in registers, and writes the probabilities p = exp2(s - m_t) of each
//     32-token tile (relative to the tile maximum) plus (m_t, sum p). RoPE at position n0 + j
//     (n0 = first token of a 32-token MFMA column tile, j = lane's column) is split as
//     R_{n0+j} = R_{n0} R_j: the query is rotated back by n0 once per (head, tile) and the
//     constant rotation by j*theta is kept in registers, so no per-token trigonometry runs in
//     the hot loop.
//  2. latent_values: one workgroup per (split, channel chunk, sequence): per-head split maximum
//     M and sum L from the tile statistics, then Acc[H x r_v] += (p * 2^(m_t - M)) Z_v on MFMA
//     with all heads stacked into one 32-row operand (notes, section 5.3), Z_v fragments
//     streamed one block ahead in registers. Writes (M, L, Acc) per split.
//  3. project_heads: merges the splits per (b, h) (log-sum-exp weights, normalised) while it
//     loads them, then out[b][h] = a[b][h] . B_v[:, h*d:(h+1)*d] for a batch of sequences.
//  merge_splits (the same merge as a kernel of its own) finishes the exempt-layer path.

#include <type_traits>

#include "common.hpp"

namespace starkv {

// ------------------------------------------------------------------------------------------------
// 2. Scores.
// ------------------------------------------------------------------------------------------------
template <int K> struct PStore;
template <> struct PStore<kF32> { using T = float; };
template <> struct PStore<kF16> { using T = _Float16; };
template <> struct PStore<kBF16> { using T = _Float16; };

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Latent fragments of one unit held in registers (the paths that load a whole unit at once).
template <int K, int MAXKS> struct KeyBuf {
    typename Elem<K>::frag z[2][MAXKS];
};

// Waves per score workgroup: twelve (three per SIMD, at most 168 VGPRs each) for 16-bit and
// mixed 4/3-bit latents, else eight with a two-deep register pipeline over units.
#ifndef STARKV_Q43_STAGE_WAVES
#define STARKV_Q43_STAGE_WAVES 12
#endif
template <int K, int MAXKS, bool QK>
constexpr int score_waves() { return K == kF32 ? 8 : (QK && MAXKS <= 4) ? STARKV_Q43_STAGE_WAVES : 12; }
// With ranks above 64 (or code windows plus scales and zero points) at twelve waves, a unit's
// latents for both 32-token column tiles do not fit the register budget: the second tile's
// fragments are loaded once the first tile's MFMAs have consumed theirs.
template <int K, int MAXKS, bool QK>
constexpr bool score_split_loads() { return QK || (score_waves<K, MAXKS, QK>() == 12 && MAXKS > 4); }
// NQ queries of one sequence share each rebuilt, rotated key: eight waves (the per-query sums and
// query tiles need the larger register budget), a smaller factor budget in LDS to make room for
// NQ rotated queries per wave, and head groups of at most kMaxGroupHeadsMQ heads.
template <int K, int MAXKS, bool QK, int NQ>
constexpr int score_waves_q() { return NQ > 1 ? 8 : score_waves<K, MAXKS, QK>(); }
// (mixed 4/3-bit codes are only ever read by the per-fragment loads of the split path)
template <int K, int MAXKS, bool QK, int NQ>
constexpr bool score_split_q() { return NQ == 1 ? score_split_loads<K, MAXKS, QK>() : QK; }
static_assert(score_split_q<kF16, 4, true, 1>() && score_split_q<kF16, 8, true, 1>() &&
              score_split_q<kF16, 4, true, 2>() && score_split_q<kF16, 8, true, 4>(),
              "mixed 4/3-bit caches must take the per-fragment load path");

template <int D, int K, int MAXKS, bool QK, int NQ>
__global__ __launch_bounds__((64 * score_waves_q<K, MAXKS, QK, NQ>()), 1) void latent_scores(const ScoreParams p) {
    constexpr int NW = score_waves_q<K, MAXKS, QK, NQ>();
    constexpr int NF = D / 2;           // RoPE frequencies
    constexpr int HMT = D / 64;         // m-tile pairs (mt, mt + HMT)
    using Fr = typename Elem<K>::frag;
    using T = typename Elem<K>::storage;
    using PT = typename PStore<K>::T;
    using Buf = KeyBuf<K, MAXKS>;

    __shared__ __attribute__((aligned(32))) T s_bk[(NQ > 1 ? kFragLdsBytesMQ : kFragLdsBytes) / sizeof(T)];
    __shared__ __attribute__((aligned(16))) float s_q[(NQ > 1 ? kMaxGroupHeadsMQ : kMaxHeads) * NQ * D];
    __shared__ __attribute__((aligned(16))) float s_qr[NW][NQ][2][D];
    __shared__ int s_slot[kMaxHeads + 1];

    // small per-layer tables, copied out of the kernel arguments so that every dynamic index
    // reads LDS (indexing the by-value argument block would make the compiler copy it to scratch)
    __shared__ double s_rev[64];
    __shared__ int s_head[kMaxHeads], s_rank[kMaxHeads], s_kgrp[kMaxHeads];
    __shared__ int s_srank[kMaxHeads], s_soff[kMaxHeads];
    __shared__ int s_goff[QK ? kMaxHeads : 1][8], s_gn[QK ? kMaxHeads : 1][8];
    // Mixed 4/3-bit codes, heads of rank <= 64: one unit's code run (at most 2048 bytes, read from
    // the 16-byte boundary at or below its start, so at most 2056 bytes) and the head's scale and
    // zero-point words, staged in a wave-private buffer one unit ahead.
    constexpr bool STAGE = QK && MAXKS <= 4;
    constexpr int kStCodeWords = 516, kStWords = kStCodeWords + 64;
    __shared__ __attribute__((aligned(16))) uint32_t s_stage[STAGE ? NW : 1][STAGE ? kStWords : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int half = lane >> 5;
    const int j = lane & 31;
    const int split = blockIdx.x;
    const int grp = blockIdx.y;
    const int b = blockIdx.z;
    const int hs0 = p.gstart[grp];
    const int ng = p.gstart[grp + 1] - hs0;
    const int H = p.H;
    // query rows row0 .. row0 + NQ - 1 read cache sequence b; the blocks cover the longest
    int qlen[NQ];
    const int row0 = b * NQ;
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) qlen[qi] = seq_length(p.seq_lens, row0 + qi, p.seq_len);
    int seq_len = qlen[0];
#pragma unroll
    for (int qi = 1; qi < NQ; ++qi) seq_len = max(seq_len, qlen[qi]);
    const int Tp = p.Tp;
    const int nblk = p.nblk;                                     // stride of the statistics
    const int my_nblk = (seq_len + 63) >> 6;
    // quantised groups of a mixed cache: the complete groups below the sequence's fill (the
    // longest length of the rows that read it; the rows of this workgroup, else row_fill)
    const int fill = (QK && p.row_fill) ? max(seq_len, p.row_fill[row0]) : seq_len;
    const int full_blocks = QK ? fill >> 6 : my_nblk;
    const float q_scale = p.q_scale;
    const T* __restrict__ zk = static_cast<const T*>(p.zk);
    const T* __restrict__ bkg = static_cast<const T*>(p.bk);
    const float* __restrict__ qg = p.q;
    PT* __restrict__ Pout = static_cast<PT*>(p.P);
    float* __restrict__ stats = p.stats;
    const int Rk = p.Rk;
    const size_t kgroups = (size_t)(Rk >> 4);
    const int bc = cache_seq(p.seq_map, b, p.cache_batch);      // the cache sequence read
    const uint32_t* __restrict__ qcodes = static_cast<const uint32_t*>(p.zk);
    const uint16_t* __restrict__ qmeta = static_cast<const uint16_t*>(p.zk_meta);
    const T* __restrict__ qtail = static_cast<const T*>(p.zk_tail);
    const size_t qblock_words = (size_t)(p.ql.block_bytes >> 2);

    if (tid < 64) s_rev[tid] = tid < NF ? p.rope_rev[tid] : 0.0;
    if (tid < ng) {
        const int h = p.order[hs0 + tid];
        s_head[tid] = h;
        s_rank[tid] = p.rank[h];
        s_kgrp[tid] = p.koff[h] >> 4;
        s_srank[tid] = p.srank[h];
        s_soff[tid] = p.soff[h];
    }
    if (QK && tid < 8 * ng) {
        const int sl = tid >> 3, k = tid & 7;
        const int h = p.order[hs0 + sl];
        const int g16 = min((p.koff[h] >> 4) + k, (int)kgroups - 1);
        s_goff[sl][k] = p.ql.goff[g16];
        s_gn[sl][k] = p.ql.gn[g16];
    }
    // ---- stage the group's factor fragments and (scaled) queries ----
    if (tid == 0) {
        int off = 0;
        for (int s = 0; s < ng; ++s) {
            s_slot[s] = off;
            off += p.rank[p.order[hs0 + s]] * D;
        }
        s_slot[ng] = off;
    }
    __syncthreads();
    for (int s = 0; s < ng; ++s) {
        const int h = s_head[s];
        // B_k rows of the head into MFMA A-operand fragment order: fragment f = mt*(rank/16) + ks,
        // lane l holds rows 16*ks + 8*(l/32) + jj (jj < 8) at column 32*mt + l%32, elements
        // (f*64 + l)*8 + jj of the head's slot. Rows past the head's true rank (the rounding of
        // its rank up to 16) are zero. Thread per (8 rows, column): the eight row reads are
        // coalesced across the wave's consecutive columns, and the eight values are one
        // contiguous LDS store (consecutive columns write consecutive 16-byte runs).
        const int rk = s_rank[s], sr = s_srank[s], so = s_soff[s], nks = rk >> 4;
        T* dst = &s_bk[s_slot[s]];
        for (int i = tid; i < (rk >> 3) * D; i += 64 * NW) {
            const int k8 = i / D, dim = i - k8 * D;
            struct __attribute__((aligned(16))) Run { T v[8]; } run;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int k = 8 * k8 + jj;
                run.v[jj] = k < sr ? bkg[(size_t)(so + k) * D + dim] : T(0);
            }
            *reinterpret_cast<Run*>(dst + (((dim >> 5) * nks + (k8 >> 1)) * 64 + (k8 & 1) * 32 + (dim & 31)) * 8) = run;
        }
        for (int i = tid; i < NQ * D; i += 64 * NW) {
            const int qi = i / D, e = i - qi * D;
            s_q[(s * NQ + qi) * D + e] = qg[((size_t)(row0 + qi) * H + h) * D + e] * q_scale;
        }
    }

    // ---- constant rotation by j*theta_i for this lane's column j and its frequencies ----
    // Frequencies held by the lane: i = 32*pp + 8*g + 4*half + r, pp < HMT, g < 4, r < 4.
    // One query row: the rotation is kept in tangent form, (cos, tan = sin / cos), so that the
    // rotate-and-dot of a rotary pair takes five operations instead of six:
    // q1 (a c - b s) + q2 (a s + b c) = c (q1 (a - t b) + q2 (b + t a)). A cosine of exactly 0
    // (or below 2^-60) is moved to +-2^-60, which changes the rotated pair by at most 2^-60 of it.
    constexpr bool TANGENT = NQ == 1;
    float cj[HMT][4][4], sj[HMT][4][4];
#pragma unroll
    for (int pp = 0; pp < HMT; ++pp)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 32 * pp + 8 * g + 4 * half + r;
                const double rev = (double)j * s_rev[i];
                sincos_rev((float)(rev - floor(rev)), &cj[pp][g][r], &sj[pp][g][r]);
                if constexpr (TANGENT) {
                    if (fabsf(cj[pp][g][r]) < 0x1p-60f) cj[pp][g][r] = copysignf(0x1p-60f, cj[pp][g][r]);
                    sj[pp][g][r] = sj[pp][g][r] / cj[pp][g][r];
                }
            }
    __syncthreads();

    const int blk_begin = split * p.blocks_per_wg;
    const int blk_end = min(my_nblk, blk_begin + p.blocks_per_wg);
    // the pipelined loop covers the blocks stored in the main layout (all blocks for binary16 /
    // bf16 / fp32 caches; the quantised groups for a mixed-precision cache, whose partial last
    // block is read from the binary16 tail afterwards)
    const int main_end = QK ? min(blk_end, full_blocks) : blk_end;
    const int my_blocks = blk_begin + wave < main_end ? (main_end - blk_begin - wave + NW - 1) / NW : 0;
    const int nunits = my_blocks * ng;

    auto load_unit = [&](Buf& z, int u) __attribute__((always_inline)) {
        const int blk = blk_begin + wave + NW * (u / ng);
        const int s = u - (u / ng) * ng;
        const int nks = s_rank[s] >> 4;
        // Every slot is loaded (steps past the head's rank repeat its last step, a cache hit), so
        // the number of loads in flight is static and the compiler's wait counts stay exact:
        // loads are retired in order, and a data-dependent count would force a full drain.
        const size_t base = (block_id(p.pages, p.nblk_cap, bc, blk) * kgroups + s_kgrp[s]) * 1024 + (size_t)j * 16 + 8 * half;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int ks = 0; ks < MAXKS; ++ks)
                z.z[nt][ks] = load_frag<K>(zk, base + (size_t)min(ks, nks - 1) * 1024 + nt * 512);
    };

    float cb[2] = {1.0f, 1.0f}, sb[2] = {0.0f, 0.0f};     // rotation by n0*theta_lane (lane < NF)

    // One unit: head slot s over 64-token block blk. frag(nt, ks) supplies the latent operand.
    auto unit = [&](int blk, int s, auto&& frag) __attribute__((always_inline)) {
        const int h = __builtin_amdgcn_readfirstlane(s_head[s]);   // s is wave-uniform
        const int nks = s_rank[s] >> 4;
        if (s == 0 && lane < NF) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const double rev = (double)(blk * 64 + 32 * nt) * s_rev[lane];
                sincos_rev((float)(rev - floor(rev)), &cb[nt], &sb[nt]);
            }
        }
        // q' = R_{n0}^T q for both column tiles and every query, wave-private LDS
        if (lane < NF) {
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                const float q1 = s_q[(s * NQ + qi) * D + lane], q2 = s_q[(s * NQ + qi) * D + lane + NF];
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    s_qr[wave][qi][nt][lane] = q1 * cb[nt] + q2 * sb[nt];
                    s_qr[wave][qi][nt][lane + NF] = q2 * cb[nt] - q1 * sb[nt];
                }
            }
        }
        wave_sync_lds();
        const T* fr = &s_bk[s_slot[s]];
        float sc[NQ][2];
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) sc[qi][0] = sc[qi][1] = 0.0f;
        // Key rebuild + RoPE + dot for a head of NKS rank steps, as straight-line code: the rank
        // is dispatched once per unit, so no branch separates the MFMA chains from the RoPE
        // arithmetic and the scheduler can overlap one pass's MFMAs with another's VALU work.
        auto core = [&](auto nks_c) __attribute__((always_inline)) {
            constexpr int NKS = decltype(nks_c)::value;
            // heads of at most four rank steps load both column tiles up front even where the
            // instantiation's larger ranks need the split (their fragments fit the same registers)
            constexpr bool SPLIT = score_split_q<K, MAXKS, QK, NQ>() && (QK || NKS > 4);
            Fr z[2][NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) z[0][ks] = frag(0, ks);
            if constexpr (!SPLIT) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) z[1][ks] = frag(1, ks);
            }
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
                for (int pp = 0; pp < HMT; ++pp) {
                    f32x16 acc0, acc1;
#pragma unroll
                    for (int r = 0; r < 16; ++r) { acc0[r] = 0.0f; acc1[r] = 0.0f; }
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        const Fr a0 = *reinterpret_cast<const Fr*>(fr + ((pp * NKS + ks) * 64 + lane) * 8);
                        const Fr a1 = *reinterpret_cast<const Fr*>(fr + (((pp + HMT) * NKS + ks) * 64 + lane) * 8);
                        acc0 = mma32<K>(a0, z[nt][ks], acc0);
                        acc1 = mma32<K>(a1, z[nt][ks], acc1);
                    }
                    if (SPLIT && nt == 0 && pp == HMT - 1) {
                        // the first tile's fragments are dead: load the second tile's here, and
                        // keep the scheduler from hoisting the loads above this point
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) z[1][ks] = frag(1, ks);
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int i0 = 32 * pp + 8 * g + 4 * half;
                        f32x4 q1[NQ], q2[NQ];
#pragma unroll
                        for (int qi = 0; qi < NQ; ++qi) {
                            q1[qi] = *reinterpret_cast<const f32x4*>(&s_qr[wave][qi][nt][i0]);
                            q2[qi] = *reinterpret_cast<const f32x4*>(&s_qr[wave][qi][nt][i0 + NF]);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float a = acc0[4 * g + r], bb = acc1[4 * g + r];
                            const float c = cj[pp][g][r], sn = sj[pp][g][r];
                            if constexpr (TANGENT) {
                                // c (q1 (a - t b) + q2 (b + t a)), t = tan(j theta) in sj
                                const float u = fmaf(-bb, sn, a), v = fmaf(a, sn, bb);
                                sc[0][nt] = fmaf(c, fmaf(q1[0][r], u, q2[0][r] * v), sc[0][nt]);
                            } else {
                                // the key rotated by j*theta, then its dot with each query
                                const float ra = fmaf(-bb, sn, a * c), rb = fmaf(a, sn, bb * c);
#pragma unroll
                                for (int qi = 0; qi < NQ; ++qi) {
                                    sc[qi][nt] = fmaf(q1[qi][r], ra, sc[qi][nt]);
                                    sc[qi][nt] = fmaf(q2[qi][r], rb, sc[qi][nt]);
                                }
                            }
                        }
                    }
                    // consume the dot here, so the compiler cannot sink every pass's RoPE
                    // arithmetic past all the MFMA chains (all accumulators would stay live)
#pragma unroll
                    for (int qi = 0; qi < NQ; ++qi) asm volatile("" : "+v"(sc[qi][nt]));
                }
            }
        };
        switch (nks) {
        case 1: core(std::integral_constant<int, 1>{}); break;
        case 2: core(std::integral_constant<int, (MAXKS >= 2 ? 2 : 1)>{}); break;
        case 3: core(std::integral_constant<int, (MAXKS >= 3 ? 3 : 1)>{}); break;
        case 4: core(std::integral_constant<int, (MAXKS >= 4 ? 4 : 1)>{}); break;
        case 5: core(std::integral_constant<int, (MAXKS >= 5 ? 5 : 1)>{}); break;
        case 6: core(std::integral_constant<int, (MAXKS >= 6 ? 6 : 1)>{}); break;
        case 7: core(std::integral_constant<int, (MAXKS >= 7 ? 7 : 1)>{}); break;
        default: core(std::integral_constant<int, MAXKS>{}); break;
        }
        const int tok = blk * 64 + lane;
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) sc[qi][nt] = add_xor32(sc[qi][nt]);
            // lane = token of the block, so each half holds one 32-token tile
            float my = half ? sc[qi][1] : sc[qi][0];
            if (tok >= qlen[qi]) my = -INFINITY;
            // the tile maximum rounded up to an integer: rescaling a stored probability by
            // 2^(m - M) between tiles is then exact; the tile sum adds the stored (rounded) values,
            // so that numerator and denominator hold the same probabilities
            const float m = ceilf(half_max(my));          // -inf stays -inf
            // a tile wholly past the query's end: p = 0, l = 0
            const PT pst = (PT)(m != -INFINITY ? __builtin_amdgcn_exp2f(my - m) : 0.0f);
            const float l = half_sum((float)pst);
            // row and block are wave-uniform: the addresses are a scalar base plus the lane
            const size_t row = (size_t)(row0 + qi) * H + h;
            (Pout + (row * Tp + (size_t)blk * 64))[lane] = pst;
            // every lane stores (even lanes m, odd lanes l, to the same two words of its tile): no
            // branch, so the count of memory operations in flight stays static
            (stats + (row * 2 * nblk + 2 * (size_t)blk) * 2)[2 * half + (lane & 1)] = (lane & 1) ? l : m;
        }
        wave_sync_lds();
    };

    auto compute_unit = [&](const Buf& z, int u) __attribute__((always_inline)) {
        const int blk = blk_begin + wave + NW * (u / ng);
        const int s = u - (u / ng) * ng;
        unit(blk, s, [&](int nt, int ks) __attribute__((always_inline)) { return z.z[nt][ks]; });
    };

    if constexpr (score_split_q<K, MAXKS, QK, NQ>() && !QK) {
        // One unit at a time, latent fragments loaded inside the unit, per column tile.
        for (int u = 0; u < nunits; ++u) {
            const int blk = blk_begin + wave + NW * (u / ng);
            const int s = u - (u / ng) * ng;
            const size_t base = (block_id(p.pages, p.nblk_cap, bc, blk) * kgroups + s_kgrp[s]) * 1024 + (size_t)j * 16 + 8 * half;
            unit(blk, s, [&](int nt, int ks) __attribute__((always_inline)) {
                return load_frag<K>(zk, base + (size_t)ks * 1024 + nt * 512);
            });
        }
    } else if constexpr (STAGE) {
        // Mixed 4/3-bit codes, ranks <= 64: the next unit's code run and scale / zero-point words
        // are loaded into registers before the current unit runs and written to the wave's LDS
        // buffer after it, so the current unit decodes its fragments from LDS and waits on no
        // global load. Every lane loads (indexes past the run are clamped to its last 16 bytes or
        // word, inside the block's codes or the buffer's end padding), so the count of loads in
        // flight is static.
        struct Staged { u32x4 c0, c1; uint32_t tail, meta; int off0; };
        auto stage_load = [&](int u) __attribute__((always_inline)) {
            const int blk = blk_begin + wave + NW * (u / ng);
            const int s = u - (u / ng) * ng;
            const int nks = s_rank[s] >> 4;
            const size_t bid = block_id(p.pages, p.nblk_cap, bc, blk);
            const size_t start = bid * (size_t)p.ql.block_bytes + (size_t)s_goff[s][0];
            const size_t end = bid * (size_t)p.ql.block_bytes + (size_t)(s_goff[s][nks - 1] + 8 * (48 + s_gn[s][nks - 1]));
            const size_t c16 = start >> 4, last16 = (end - 1) >> 4;
            const u32x4* code16 = reinterpret_cast<const u32x4*>(qcodes);
            Staged st;
            st.c0 = code16[min(c16 + (size_t)lane, last16)];
            st.c1 = code16[min(c16 + 64 + (size_t)lane, last16)];
            st.tail = qcodes[min(4 * c16 + 512 + (size_t)(lane & 3), (end - 1) >> 2)];
            const uint32_t* mw = reinterpret_cast<const uint32_t*>(qmeta) + bid * (size_t)Rk;
            st.meta = mw[(lane < 32 ? 0 : (Rk >> 1)) + 8 * s_kgrp[s] + min(lane & 31, 8 * nks - 1)];
            st.off0 = (int)(start & 15);
            return st;
        };
        // buffer words: [0, 516) codes from the 16-byte boundary, [516, 548) scales and
        // [548, 580) zero points of the head's channels (two binary16 values per word)
        auto stage_store = [&](const Staged& st) __attribute__((always_inline)) {
            uint32_t* buf = s_stage[wave];
            *reinterpret_cast<u32x4*>(buf + 4 * lane) = st.c0;
            *reinterpret_cast<u32x4*>(buf + 256 + 4 * lane) = st.c1;
            buf[512 + (lane & 3)] = st.tail;     // lanes with equal (lane & 3) store the same word
            buf[kStCodeWords + lane] = st.meta;
        };
        int off0 = 0;    // the staged unit's start within its first 16 bytes (0 or 8)
        if (nunits > 0) {
            const Staged st = stage_load(0);
            stage_store(st);
            off0 = st.off0;
        }
        for (int u = 0; u < nunits; ++u) {
            const Staged nx = stage_load(min(u + 1, nunits - 1));
            const int blk = blk_begin + wave + NW * (u / ng);
            const int s = u - (u / ng) * ng;
            const uint32_t* buf = s_stage[wave];
            const int g0 = s_goff[s][0];
            unit(blk, s, [&](int nt, int ks) __attribute__((always_inline)) {
                const int n = s_gn[s][ks];
                const u32x4 sc = *reinterpret_cast<const u32x4*>(buf + kStCodeWords + 8 * ks + 4 * half);
                const u32x4 zc = *reinterpret_cast<const u32x4*>(buf + kStCodeWords + 32 + 8 * ks + 4 * half);
                const int rb = 8 * (off0 + s_goff[s][ks] - g0) + (int)__umul24(32 * nt + j, 48 + n);
                const uint32_t* wp = buf + (rb >> 5);
                return q43_key_frag(wp[0], wp[1], wp[2], rb & 31, n, half, sc, zc);
            });
            stage_store(nx);
            off0 = nx.off0;
        }
    } else if constexpr (score_split_q<K, MAXKS, QK, NQ>()) {
        // Mixed 4/3-bit codes: the code window, scales and zero points of each fragment are
        // loaded inside the unit, per column tile, and dequantised in registers.
        for (int u = 0; u < nunits; ++u) {
            const int blk = blk_begin + wave + NW * (u / ng);
            const int s = u - (u / ng) * ng;
            const size_t bid = block_id(p.pages, p.nblk_cap, bc, blk);
            const uint32_t* blkw = qcodes + bid * qblock_words;
            const uint16_t* meta = qmeta + bid * 2 * (size_t)Rk;
            unit(blk, s, [&](int nt, int ks) __attribute__((always_inline)) {
                const int n = s_gn[s][ks];
                const int c0 = 16 * (s_kgrp[s] + ks) + 8 * half;
                const u32x4 sc = *reinterpret_cast<const u32x4*>(meta + c0);
                const u32x4 zc = *reinterpret_cast<const u32x4*>(meta + Rk + c0);
                const int rb = 8 * s_goff[s][ks] + (32 * nt + j) * (48 + n);
                const uint32_t* wp = blkw + (rb >> 5);
                return q43_key_frag(wp[0], wp[1], wp[2], rb & 31, n, half, sc, zc);
            });
        }
    } else if constexpr (NW == 12) {
        // One unit at a time: its loads are waited for inside it, and the other two waves of the
        // SIMD cover the latency (a second register buffer would cost a wave per SIMD).
        Buf zA;
        for (int u = 0; u < nunits; ++u) {
            load_unit(zA, u);
            compute_unit(zA, u);
        }
    } else {
        // Two-deep software pipeline over units. Prefetches past the last unit reload the last
        // one (a cache hit) instead of being skipped, for the same reason as in load_unit.
        Buf zA, zB;
        if (nunits > 0) load_unit(zA, 0);
        for (int u = 0; u < nunits; u += 2) {
            load_unit(zB, min(u + 1, nunits - 1));
            compute_unit(zA, u);
            load_unit(zA, min(u + 2, nunits - 1));
            if (u + 1 < nunits) compute_unit(zB, u + 1);
        }
    }

    if constexpr (QK) {
        // the partial last block of a mixed-precision cache: its rows are still binary16 in the
        // tail buffer [B][64][Rk], token-major
        const int tb = full_blocks;
        if (tb < blk_end && tb >= blk_begin && (tb - blk_begin) % NW == wave) {
            for (int s = 0; s < ng; ++s) {
                const T* rowp = qtail + ((size_t)bc * 64 + j) * Rk + 16 * s_kgrp[s] + 8 * half;
                unit(tb, s, [&](int nt, int ks) __attribute__((always_inline)) {
                    return load_frag<K>(rowp, (size_t)(32 * nt) * Rk + 16 * ks);
                });
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// 3. Values. Wave w of workgroup (split, chunk, b) owns channel tiles nt = (chunk*kValueWaves + w)
// * NTW + k, k < NTW (32 channels each). A operand = probabilities (row = head), B operand = Z_v.
// ------------------------------------------------------------------------------------------------
template <int K> struct ProbFrag;

// The tile maxima are integers, so the factor f = 2^(m_t - M) that brings a tile's stored
// probabilities to the split's maximum is a power of two and the rescaled binary16 value is exact
// (short of the subnormal range, where it is rounded once): one binary16 operand.
template <> struct ProbFrag<kF16> {
    using Raw = f16x8;
    __device__ static Raw load(const void* P, size_t i) { return *reinterpret_cast<const f16x8*>(static_cast<const _Float16*>(P) + i); }
    __device__ static Raw zero() { Raw r; for (int e = 0; e < 8; ++e) r[e] = (_Float16)0.0f; return r; }
    struct Op { f16x8 v; };
    __device__ static Op scale(const Raw& r, float f) {
        const _Float16 h = (_Float16)f;
        Op o;
        o.v = r * (f16x8){h, h, h, h, h, h, h, h};
        return o;
    }
    __device__ static f32x16 mma(const Op& a, const f16x8& z, f32x16 acc) { return mma32<kF16>(a.v, z, acc); }
};

template <> struct ProbFrag<kBF16> {
    // probabilities are stored as fp16; the bf16 operand is split into hi + lo so that the pair
    // keeps the ~16 significant bits of the scaled probability.
    using Raw = f16x8;
    __device__ static Raw load(const void* P, size_t i) { return *reinterpret_cast<const f16x8*>(static_cast<const _Float16*>(P) + i); }
    __device__ static Raw zero() { Raw r; for (int e = 0; e < 8; ++e) r[e] = (_Float16)0.0f; return r; }
    struct Op { bf16x8 hi, lo; };
    __device__ static Op scale(const Raw& r, float f) {
        Op o;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = (float)r[e] * f;
            const uint16_t hb = float_to_bf16_bits(v);
            const uint16_t lb = float_to_bf16_bits(v - bf16_bits_to_float(hb));
            o.hi[e] = __builtin_bit_cast(__bf16, hb);
            o.lo[e] = __builtin_bit_cast(__bf16, lb);
        }
        return o;
    }
    __device__ static f32x16 mma(const Op& a, const bf16x8& z, f32x16 acc) {
        acc = mma32<kBF16>(a.hi, z, acc);
        return mma32<kBF16>(a.lo, z, acc);
    }
};

template <> struct ProbFrag<kF32> {
    using Raw = f32x8;
    __device__ static Raw load(const void* P, size_t i) {
        const f32x4* s = reinterpret_cast<const f32x4*>(static_cast<const float*>(P) + i);
        const f32x4 a = s[0], c = s[1];
        Raw r;
        for (int e = 0; e < 4; ++e) { r[e] = a[e]; r[4 + e] = c[e]; }
        return r;
    }
    __device__ static Raw zero() { Raw r; for (int e = 0; e < 8; ++e) r[e] = 0.0f; return r; }
    struct Op { f32x8 v; };
    __device__ static Op scale(const Raw& r, float f) {
        Op o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o.v[e] = r[e] * f;
        return o;
    }
    __device__ static f32x16 mma(const Op& a, const f32x8& z, f32x16 acc) { return mma32<kF32>(a.v, z, acc); }
};

// Eight mixed 4/3-bit value codes (tokens 16*ks + 8*half .. +7 of one channel) to an fp16 MFMA
// operand fragment. run: the channel's 64 codes as eight words (4-bit: eight tokens per word;
// 3-bit: words 0..3 the low two bits of sixteen tokens each, words 4..5 the third bit of 32), each
// word holding the even tokens of its span in its low 16 bits and the odd tokens in its high 16
// bits, so that one shift and mask leave tokens 2k and 2k+1 of the fragment in the two halves of
// a word; s2 / z2: the channel's scale and zero point in both halves. Each value is
// binary16(q*s + z) rounded once; q is formed exactly as binary16(1024 + q) - 1024.
__device__ __forceinline__ f16x8 q43_value_frag(const uint32_t (&run)[8], bool hi4, int ks, int half,
                                               uint32_t s2, uint32_t z2) {
    uint32_t bits[4];
    if (hi4) {
        const uint32_t w = half ? run[2 * ks + 1] : run[2 * ks];   // static register indices
#pragma unroll
        for (int k = 0; k < 4; ++k) bits[k] = ((w >> (4 * k)) & 0x000F000Fu) | 0x64006400u;
    } else {
        const uint32_t w2 = run[ks] >> (8 * half);
        const uint32_t w1 = (run[4 + (ks >> 1)] >> (8 * (ks & 1) + 4 * half)) << 2;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            bits[k] = ((w2 >> (2 * k)) & 0x00030003u) | (((w1 >> k) & 0x00040004u) | 0x64006400u);
    }
    f16x8 out;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f16x2 qv = __builtin_bit_cast(f16x2, bits[k]) - (f16x2){(_Float16)1024.0f, (_Float16)1024.0f};
        const f16x2 r = __builtin_elementwise_fma(qv, __builtin_bit_cast(f16x2, s2), __builtin_bit_cast(f16x2, z2));
        out[2 * k] = r[0];
        out[2 * k + 1] = r[1];
    }
    return out;
}

template <int K, int MAXC, bool QV> struct ValBuf;
template <int K, int NTW> struct ValBuf<K, NTW, false> {
    typename Elem<K>::frag z[NTW][4];
};
template <int K, int NTW> struct ValBuf<K, NTW, true> {
    uint32_t run[NTW][8];
    uint32_t s2[NTW], z2[NTW];
};

// NQ query rows of one cache sequence (row0 = b * NQ ...): each latent fragment feeds NQ stacked
// 32-row operands (one per query row's heads), so the value latent is streamed once for all.
template <int K, int NTW, bool QV, int NQ>
__global__ __launch_bounds__(256, 2) void latent_values(const ValueParams p) {
    using Fr = typename Elem<K>::frag;
    using Buf = ValBuf<K, NTW, QV>;
    using PF = ProbFrag<K>;
    constexpr int BPS = kMaxBlocksPerSplit / NQ;      // the planner caps splits at this many blocks
    __shared__ float s_f[NQ][kMaxHeads][2 * BPS];       // per 32-token tile
    __shared__ float s_M[NQ][kMaxHeads], s_L[NQ][kMaxHeads];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int split = blockIdx.x;
    const int chunk = blockIdx.y;
    const int b = blockIdx.z;
    const int H = p.H;
    const int row0 = b * NQ;                                     // this workgroup's query rows
    int seq_len = seq_length(p.seq_lens, row0, p.seq_len);      // the longest of their lengths
#pragma unroll
    for (int qi = 1; qi < NQ; ++qi) seq_len = max(seq_len, seq_length(p.seq_lens, row0 + qi, p.seq_len));
    const int bc = cache_seq(p.seq_map, b, p.cache_batch);      // the cache sequence read
    const int blk_begin = split * p.blocks_per_split;
    // a split past this sequence's end is empty (blk_end == blk_begin): (M, L, Acc) = (-inf, 0, 0)
    const int blk_end = max(blk_begin, min((seq_len + 63) >> 6, blk_begin + p.blocks_per_split));
    const int nb = blk_end - blk_begin;

    // ---- split statistics per (query row, head) from the 32-token tile statistics (m, l):
    // M = max m, f_tile = 2^(m - M), L = sum f l
    for (int hq = wave; hq < NQ * H; hq += kValueWaves) {
        const int qi = hq / H, h = hq - qi * H;
        const float* st = p.stats + (((size_t)(row0 + qi) * H + h) * 2 * p.nblk + 2 * blk_begin) * 2;
        float M = -INFINITY;
        for (int i = lane; i < 2 * nb; i += 64) M = fmaxf(M, st[2 * i]);
        M = wave_max(M);
        // a row whose tiles here all lie past its own end: every f is 0 (no -inf - -inf)
        const float Mc = M != -INFINITY ? M : 0.0f;
        float L = 0.0f;
        for (int i = lane; i < 2 * nb; i += 64) {
            const float f = tile_factor(st[2 * i] - Mc);
            s_f[qi][h][i] = f;
            L += f * st[2 * i + 1];
        }
        L = wave_sum(L);
        if (lane == 0) { s_M[qi][h] = M; s_L[qi][h] = L; }
    }
    __syncthreads();

    // Rows (heads) >= H and channels >= r_v only feed output rows / columns that are never
    // stored, so their operands are loaded from a clamped valid address without masking; all
    // loads are unconditional, which keeps the compiler's in-order wait counts exact.
    const int hrow = lane & 31;
    const bool hvalid = hrow < H;
    const int cgroups = p.rv >> 4;
    int ch[NTW];
    bool chok[NTW];
    size_t zoff[NTW];
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
        ch[k] = ((chunk * kValueWaves + wave) * NTW + k) * 32 + (lane & 31);
        chok[k] = ch[k] < p.rv;
        const int cc = min(ch[k], p.rv - 1);
        zoff[k] = (size_t)(cc >> 4) * 1024 + (cc & 15) * 16 + 8 * half;
    }
    f32x16 acc[NQ][NTW];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
        for (int k = 0; k < NTW; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qi][k][r] = 0.0f;

    typename PF::Raw pA[NQ][4], pB[NQ][4];
    Buf zA, zB;
    // probability row of this lane's head for query row qi: prow + qi * qstride
    const size_t prow = ((size_t)row0 * H + min(hrow, H - 1)) * p.Tp + 8 * half;
    const size_t qstride = (size_t)H * p.Tp;
    // mixed 4/3-bit cache: per lane, the channel's run offset and width are fixed
    const uint8_t* __restrict__ qcodes = static_cast<const uint8_t*>(p.zv);
    const uint16_t* __restrict__ qmeta = static_cast<const uint16_t*>(p.zv_meta);
    int roff[NTW];
    bool hi4[NTW];
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
        const int cc = min(ch[k], p.rv - 1);
        hi4[k] = cc < p.n_hi;
        roff[k] = cc < p.n_hi ? 32 * cc : 32 * p.n_hi + 24 * (cc - p.n_hi);
    }
    // mixed cache: blocks [blk_begin, main_end) are quantised; a block main_end < blk_end is the
    // partial last group, read from the binary16 tail
    const int fill = (QV && p.row_fill) ? max(seq_len, p.row_fill[row0]) : seq_len;
    const int main_end = QV ? max(blk_begin, min(blk_end, fill >> 6)) : blk_end;

    auto load_blk = [&](typename PF::Raw (&pr)[NQ][4], Buf& z, int blk) __attribute__((always_inline)) {
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) pr[qi][ks] = PF::load(p.P, prow + qi * qstride + (size_t)blk * 64 + 16 * ks);
        if constexpr (!QV) {
            const size_t bbase = block_id(p.pages, p.nblk_cap, bc, blk) * cgroups * 1024;
#pragma unroll
            for (int k = 0; k < NTW; ++k)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) z.z[k][ks] = load_frag<K>(p.zv, bbase + zoff[k] + ks * 256);
        } else {
            const size_t bb = block_id(p.pages, p.nblk_cap, bc, blk);
            const uint8_t* blkp = qcodes + bb * p.block_bytes;
            const uint16_t* meta = qmeta + bb * 2 * p.rv;
#pragma unroll
            for (int k = 0; k < NTW; ++k) {
                // the 3-bit runs are 24 bytes; the eight-word window may read into the next run or
                // the buffer's padding, which is never used
                const uint2* w = reinterpret_cast<const uint2*>(blkp + roff[k]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint2 v = w[i];
                    z.run[k][2 * i] = v.x;
                    z.run[k][2 * i + 1] = v.y;
                }
                const int cc = min(ch[k], p.rv - 1);
                const uint32_t sv = meta[cc], zv = meta[p.rv + cc];
                z.s2[k] = sv | (sv << 16);
                z.z2[k] = zv | (zv << 16);
            }
        }
    };
    // Fr frag(k, ks) of the block's latent operand; zero past the sequence end
    auto accumulate = [&](const typename PF::Raw (&pr)[NQ][4], int blk, auto&& frag) __attribute__((always_inline)) {
        float f[NQ][2];                                   // per 32-token tile of the block
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
            for (int t = 0; t < 2; ++t) f[qi][t] = hvalid ? s_f[qi][hrow][2 * (blk - blk_begin) + t] : 0.0f;
        const bool ragged = (blk + 1) * 64 > seq_len;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            typename PF::Op a[NQ];
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) a[qi] = PF::scale(pr[qi][ks], f[qi][ks >> 1]);
#pragma unroll
            for (int k = 0; k < NTW; ++k) {
                Fr zf = frag(k, ks);
                if (ragged) {                              // ragged last block: zero the tail
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (blk * 64 + 16 * ks + 8 * half + e >= seq_len) zf[e] = 0;
                }
#pragma unroll
                for (int qi = 0; qi < NQ; ++qi) acc[qi][k] = PF::mma(a[qi], zf, acc[qi][k]);
            }
        }
    };
    auto compute_blk = [&](const typename PF::Raw (&pr)[NQ][4], const Buf& z, int blk) __attribute__((always_inline)) {
        if constexpr (!QV) {
            accumulate(pr, blk, [&](int k, int ks) __attribute__((always_inline)) { return z.z[k][ks]; });
        } else {
            accumulate(pr, blk, [&](int k, int ks) __attribute__((always_inline)) {
                return q43_value_frag(z.run[k], hi4[k], ks, half, z.s2[k], z.z2[k]);
            });
        }
    };

    if (main_end > blk_begin) load_blk(pA, zA, blk_begin);
    for (int blk = blk_begin; blk < main_end; blk += 2) {
        load_blk(pB, zB, min(blk + 1, main_end - 1));
        compute_blk(pA, zA, blk);
        load_blk(pA, zA, min(blk + 2, main_end - 1));
        if (blk + 1 < main_end) compute_blk(pB, zB, blk + 1);
    }
    if constexpr (QV) {
        // the partial last block of a mixed-precision cache: binary16 rows in the tail [B][64][rv]
        if (main_end < blk_end) {
            const int blk = main_end;
            typename PF::Raw pr[NQ][4];
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) pr[qi][ks] = PF::load(p.P, prow + qi * qstride + (size_t)blk * 64 + 16 * ks);
            const _Float16* tail = static_cast<const _Float16*>(p.zv_tail) + (size_t)bc * 64 * p.rv;
            accumulate(pr, blk, [&](int k, int ks) __attribute__((always_inline)) {
                const int cc = min(ch[k], p.rv - 1);
                Fr zf;
#pragma unroll
                for (int e = 0; e < 8; ++e) zf[e] = tail[(size_t)(16 * ks + 8 * half + e) * p.rv + cc];
                return zf;
            });
        }
    }

#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        const size_t part = (size_t)(row0 + qi) * p.S + split;
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
            if (!chok[k]) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int h = acc_row(r, lane);
                if (h < H) p.ws_acc[(part * H + h) * p.rv + ch[k]] = acc[qi][k][r];
            }
        }
    }
    if (chunk == 0 && tid < NQ * H) {
        const int qi = tid / H, h = tid - qi * H;
        const size_t part = (size_t)(row0 + qi) * p.S + split;
        p.ws_ml[(part * H + h) * 2 + 0] = s_M[qi][h];
        p.ws_ml[(part * H + h) * 2 + 1] = s_L[qi][h];
    }
}

// ------------------------------------------------------------------------------------------------
// 4. Log-sum-exp merge of the splits: thread per (b, h, 4 channels); the split weights
// w_s = 2^(M_s - M) / sum_s 2^(M_s - M) L_s are recomputed per thread from the (small) split
// statistics. Row width W (a multiple of 4).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_splits(const MergeParams p) {
    const int W4 = p.W >> 2;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.B * p.H * W4) return;
    const int c4 = (int)(idx % W4);
    const int bh = (int)(idx / W4);
    const int b = bh / p.H, h = bh - b * p.H;
    const int S = p.active_splits;
    const float* ml = p.ws_ml + ((size_t)b * p.S * p.H + h) * 2;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[(size_t)s * p.H * 2]);
    if (M == -INFINITY) M = 0.0f;                  // every split empty (a length-0 sequence): zeros
    float L = 0.0f;
    for (int s = 0; s < S; ++s) L += __builtin_amdgcn_exp2f(ml[(size_t)s * p.H * 2] - M) * ml[(size_t)s * p.H * 2 + 1];
    const float inv_l = L > 0.0f ? 1.0f / L : 0.0f;
    const f32x4* acc = reinterpret_cast<const f32x4*>(p.ws_acc + ((size_t)b * p.S * p.H + h) * p.W) + c4;
    const size_t sstride = (size_t)p.H * W4;
    f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int s = 0; s < S; ++s) {
        const float w = __builtin_amdgcn_exp2f(ml[(size_t)s * p.H * 2] - M) * inv_l;
        const f32x4 v = acc[s * sstride];
        a += w * v;
    }
    reinterpret_cast<f32x4*>(p.ws_a + ((size_t)b * p.H + h) * p.W)[c4] = a;
}

// ------------------------------------------------------------------------------------------------
// 5. Output projection: out[b][h][j] = sum_c a[b][h][c] * B_v[c][h*D + j], where a is the split
// merge a = sum_s 2^(M_s - M) Acc_s / sum_s 2^(M_s - M) L_s formed while loading. Workgroup (h,
// 64-column tile, chunk of 4 sequences), 16 waves; wave w sums the channels c = w + 16*i with lane = column
// (coalesced 128-byte rows of B_v) and the 4 sequences' a[.][h][c] broadcast from LDS; the waves'
// partial sums are reduced through LDS.
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

constexpr int kProjBatch = 4;     // sequences per workgroup (a multiple of 4)
constexpr int kProjMaxRv = 2048;
constexpr int kProjWaves = 16;
constexpr int kMaxProjSplits = 256;   // value splits merged while loading

template <int K>
__global__ __launch_bounds__(1024) void project_heads(const ProjectParams p) {
    __shared__ __attribute__((aligned(16))) float s_a[kProjMaxRv * kProjBatch];
    __shared__ float s_red[kProjWaves][kProjBatch][64];
    __shared__ float s_w[kProjBatch][kMaxProjSplits];
    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = blockIdx.y * 64 + lane;
    const int b0 = blockIdx.z * kProjBatch;
    const int nb = min(kProjBatch, p.B - b0);
    // split weights w_s = 2^(M_s - M) / sum_s 2^(M_s - M) L_s for each of the batch's sequences
    // (wave bi, lanes over the splits)
    if (wave < kProjBatch) {
        const int bi = wave;
        const float* ml = p.ws_ml + ((size_t)(b0 + min(bi, nb - 1)) * p.S * p.H + h) * 2;
        const size_t sstride = (size_t)p.H * 2;
        float M = -INFINITY;
        for (int s = lane; s < p.S; s += 64) M = fmaxf(M, ml[s * sstride]);
        M = wave_max(M);
        if (M == -INFINITY) M = 0.0f;              // every split empty (a length-0 sequence): zeros
        float L = 0.0f;
        for (int s = lane; s < p.S; s += 64) L += __builtin_amdgcn_exp2f(ml[s * sstride] - M) * ml[s * sstride + 1];
        L = wave_sum(L);
        const float inv_l = L > 0.0f ? 1.0f / L : 0.0f;
        for (int s = lane; s < p.S; s += 64)
            s_w[bi][s] = bi < nb ? __builtin_amdgcn_exp2f(ml[s * sstride] - M) * inv_l : 0.0f;
    }
    __syncthreads();
    // merged, normalised latent output a[b][h][c] of the batch's sequences, channel-major in LDS
    // four channels per thread (16-byte loads), four splits in flight per step
    const size_t sacc4 = (size_t)p.H * p.rv / 4;
    const int rv4 = p.rv >> 2;
    for (int e = tid; e < kProjBatch * rv4; e += 1024) {
        const int bi = e / rv4, c4 = e - bi * rv4;
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
        if (bi < nb) {
            const f32x4* acc = reinterpret_cast<const f32x4*>(
                p.ws_acc + ((size_t)(b0 + bi) * p.S * p.H + h) * p.rv) + c4;
            int s = 0;
            for (; s + 4 <= p.S; s += 4) {
                const f32x4 v0 = acc[(s + 0) * sacc4], v1 = acc[(s + 1) * sacc4];
                const f32x4 v2 = acc[(s + 2) * sacc4], v3 = acc[(s + 3) * sacc4];
                a += s_w[bi][s] * v0 + s_w[bi][s + 1] * v1 + s_w[bi][s + 2] * v2 + s_w[bi][s + 3] * v3;
            }
            for (; s < p.S; ++s) a += s_w[bi][s] * acc[s * sacc4];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) s_a[(4 * c4 + k) * kProjBatch + bi] = a[k];
    }
    __syncthreads();
    float acc[kProjBatch];
#pragma unroll
    for (int i = 0; i < kProjBatch; ++i) acc[i] = 0.0f;
    const bool colok = col < p.D;
    const size_t HD = (size_t)p.H * p.D;
    const size_t cbase = (size_t)h * p.D + (colok ? col : 0);
#pragma unroll 8
    for (int c = wave; c < p.rv_src; c += kProjWaves) {     // stored channels past rv_src are zero
        const float w = load_scalar<K>(p.bv, (size_t)c * HD + cbase);
#pragma unroll
        for (int k4 = 0; k4 < kProjBatch / 4; ++k4) {
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(&s_a[c * kProjBatch + 4 * k4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * k4 + e] += a4[e] * w;
        }
    }
#pragma unroll
    for (int i = 0; i < kProjBatch; ++i) s_red[wave][i][lane] = acc[i];
    __syncthreads();
    if (tid < kProjBatch * 64) {
        const int i = tid >> 6, jc = tid & 63;
        const int c2 = blockIdx.y * 64 + jc;
        if (i < nb && c2 < p.D) {
            float v = 0.0f;
#pragma unroll
            for (int k = 0; k < kProjWaves; ++k) v += s_red[k][i][jc];
            p.out[((size_t)(b0 + i) * p.H + h) * p.D + c2] = v;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Host launchers
// ------------------------------------------------------------------------------------------------
// grid.z = cache sequences (each workgroup serves its sequence's NQ query rows)
template <int D, int K, int MAXKS, bool QK, int NQ>
static hipError_t launch_scores_t(const ScoreParams& p, int groups, int splits, hipStream_t st) {
    hipLaunchKernelGGL((latent_scores<D, K, MAXKS, QK, NQ>), dim3(splits, groups, p.B / NQ),
                       dim3(64 * score_waves_q<K, MAXKS, QK, NQ>()), 0, st, p);
    return hipGetLastError();
}

template <int D, int K, bool QK, int NQ>
static hipError_t launch_scores_d(const ScoreParams& p, int groups, int splits, int maxks, hipStream_t st) {
    if (maxks <= 4) return launch_scores_t<D, K, 4, QK, NQ>(p, groups, splits, st);
    if (D == 128 && maxks <= 8) return launch_scores_t<D, K, (D == 128 ? 8 : 4), QK, NQ>(p, groups, splits, st);
    return hipErrorInvalidValue;
}

template <int K, bool QK, int NQ>
static hipError_t launch_scores_k(const ScoreParams& p, int groups, int splits, int maxks, hipStream_t st) {
    if (p.D == 128) return launch_scores_d<128, K, QK, NQ>(p, groups, splits, maxks, st);
    if (p.D == 64) return launch_scores_d<64, K, QK, NQ>(p, groups, splits, maxks, st);
    return hipErrorInvalidValue;
}

template <int NQ>
static hipError_t launch_scores_q(const ScoreParams& p, int elem, int groups, int splits, int maxks,
                                  hipStream_t st) {
    switch (elem) {
    case kF16: return launch_scores_k<kF16, false, NQ>(p, groups, splits, maxks, st);
    case kBF16: return launch_scores_k<kBF16, false, NQ>(p, groups, splits, maxks, st);
    case -1: return launch_scores_k<kF16, true, NQ>(p, groups, splits, maxks, st);
    default: return hipErrorInvalidValue;
    }
}

// elem: kF32 / kF16 / kBF16, or -1 for a mixed 4/3-bit key cache (binary16 factors). nq: query
// rows per cache sequence (p.B rows in all); 2 and 4 share each key between the rows (16-bit and
// mixed caches).
hipError_t launch_latent_scores(const ScoreParams& p, int elem, int groups, int splits, int maxks,
                                int nq, hipStream_t st) {
    if (nq == 2) return launch_scores_q<2>(p, elem, groups, splits, maxks, st);
    if (nq == 4) return launch_scores_q<4>(p, elem, groups, splits, maxks, st);
    if (nq != 1) return hipErrorInvalidValue;
    if (elem == kF32) return launch_scores_k<kF32, false, 1>(p, groups, splits, maxks, st);
    return launch_scores_q<1>(p, elem, groups, splits, maxks, st);
}

// 32-channel tiles per value wave: four where r_v fills whole 512-channel chunks (each probability
// fragment a wave loads and scales then feeds 16 MFMAs, and a block's probabilities are read by
// half as many waves), two where that would leave a partly empty chunk (e.g. r_v = 768, 1280).
int value_tiles_per_wave(int rv) {
    const int tiles = (rv + 31) / 32;
    const int waste4 = ((tiles + 4 * kValueWaves - 1) / (4 * kValueWaves)) * 4 * kValueWaves - tiles;
    const int waste2 = ((tiles + 2 * kValueWaves - 1) / (2 * kValueWaves)) * 2 * kValueWaves - tiles;
    return waste2 < waste4 ? 2 : 4;
}

// grid.z = cache sequences; NQ query rows each (p.B rows in all)
template <int NTW, int NQ>
static hipError_t launch_values_t(const ValueParams& p, int elem, int chunks, hipStream_t st) {
    const dim3 grid(p.S, chunks, p.B / NQ);
    switch (elem) {
    case kF16: hipLaunchKernelGGL((latent_values<kF16, NTW, false, NQ>), grid, dim3(256), 0, st, p); break;
    case kBF16: hipLaunchKernelGGL((latent_values<kBF16, NTW, false, NQ>), grid, dim3(256), 0, st, p); break;
    case -1: hipLaunchKernelGGL((latent_values<kF16, NTW, true, NQ>), grid, dim3(256), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ntw channel tiles per wave (nq query rows per sequence: 2 and 4 use ntw = 4 / nq, so the
// accumulators stay at four tiles' worth)
hipError_t launch_latent_values(const ValueParams& p, int elem, int chunks, int ntw, int nq, hipStream_t st) {
    if (nq == 2 && ntw == 2) return launch_values_t<2, 2>(p, elem, chunks, st);
    if (nq == 4 && ntw == 1) return launch_values_t<1, 4>(p, elem, chunks, st);
    if (nq != 1) return hipErrorInvalidValue;
    if (elem == kF32) {
        if (ntw != 2) return hipErrorInvalidValue;
        hipLaunchKernelGGL((latent_values<kF32, 2, false, 1>), dim3(p.S, chunks, p.B), dim3(256), 0, st, p);
        return hipGetLastError();
    }
    if (ntw == 4) return launch_values_t<4, 1>(p, elem, chunks, st);
    if (ntw == 2) return launch_values_t<2, 1>(p, elem, chunks, st);
    return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeParams& p, hipStream_t st) {
    const long long n = (long long)p.B * p.H * (p.W / 4);
    hipLaunchKernelGGL(merge_splits, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
    return hipGetLastError();
}

// One thread per query row: the largest clamped length among the rows that read its cache
// sequence (rows <= a few thousand, so the quadratic scan is a few microseconds at most).
__global__ __launch_bounds__(256) void row_fill_max(const RowFillParams p) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= p.rows) return;
    const int mine = cache_seq(p.seq_map, i, p.cache_batch);
    int m = 0;
    for (int r = 0; r < p.rows; ++r)
        if (cache_seq(p.seq_map, r, p.cache_batch) == mine) m = max(m, seq_length(p.seq_lens, r, p.max_len));
    p.row_fill[i] = m;
}

hipError_t launch_row_fill(const RowFillParams& p, hipStream_t st) {
    if (p.rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(row_fill_max, dim3((p.rows + 255) / 256), dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_project(const ProjectParams& p, int elem, hipStream_t st) {
    const dim3 grid(p.H, (p.D + 63) / 64, (p.B + kProjBatch - 1) / kProjBatch);
    switch (elem) {
    case kF32: hipLaunchKernelGGL(project_heads<kF32>, grid, dim3(1024), 0, st, p); break;
    case kF16: hipLaunchKernelGGL(project_heads<kF16>, grid, dim3(1024), 0, st, p); break;
    case kBF16: hipLaunchKernelGGL(project_heads<kBF16>, grid, dim3(1024), 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}


}  // namespace starkv
