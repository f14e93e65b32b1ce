// prefill.hip -- chunked (prefill) attention over the latent cache (gfx950).
//
// A chunk of queries per sequence attends causally to the latent cache (Zhou, STAR-KV reading
// notes, Algorithm 2 steps 4-7 applied to every query of the chunk; section 5.3): query l of
// sequence b, at position pos0 + l, attends to every cached token n <= pos0 + l with
//   s_{l,h,n} = scale * q_{l,h} . RoPE_n(Z_k[h][n] B_k[h]),   o_{l,h} = sum_n p_{l,h,n} Z_v[n] B_v^h.
// For one query the latent order pays (values summed in latent space, B_v applied once); for a
// chunk of queries it does not: the latent value sum costs 2 r_v flop per (query, key, head)
// against 2 d for values rebuilt once per key, V_h = Z_v B_v^h. So a call
//   1. copies the latent rows of tokens [0, pos0 + chunk) out of the cache (dequantising mixed
//      4/3-bit groups) -- api.cpp;
//   2. prefill_kv: per (sequence, head, 32-token tile) rebuilds the keys K~ = Z_k B_k on MFMA,
//      rotates each to its position in fp32 (R_n = R_{n0} R_j), and the values V = Z_v B_v^h on
//      MFMA; both are stored as binary16 hi + lo parts scaled by a power of two per tile, in the
//      MFMA operand order the attention kernel reads;
//   3. prefill_attend: per (sequence, head, 32 queries) one wave walks the key tiles up to the
//      diagonal: S^T = K Q^T as K_hi Q_hi + K_hi Q_lo + K_lo Q_hi (about 2^-22 relative error,
//      the accuracy of the decode kernel's fp32 dot), causal mask, an online softmax whose
//      running maximum is rounded up to an integer (log2 units) so that every rescaling is an
//      exact power of two, probabilities as binary16, O^T += V^T P^T (V as hi + lo parts), and
//      the normalised output written once. Neither the probabilities nor any per-query latent
//      sum goes to memory.

#include "common.hpp"
#include "prefill.hpp"

namespace starkv {

namespace {

constexpr int kPkWaves = 8;          // key tiles per preparation workgroup (one per wave)
constexpr int kPkChunk = 64;         // value-factor rows staged in LDS at a time
constexpr int kPaWaves = 4;          // query tiles per attention workgroup (one per wave)
constexpr int kPfMaxFrag = 128 * 128;   // B_k elements of one head (rank <= d <= 128)

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

// value ranks as staged for the preparation kernel: whole 64-rank chunks (B_v padded with zeros)
__host__ __device__ __forceinline__ int pf_padded_rank(int rv) { return (rv + kPkChunk - 1) / kPkChunk * kPkChunk; }

// tokens of sequence b that hold latents: [0, pos0 + chunk_len(b))
__device__ __forceinline__ int pf_fill(const int32_t* chunk_lens, int b, int chunk, int pos0) {
    return pos0 + (chunk_lens ? min(max(chunk_lens[b], 0), chunk) : chunk);
}

struct __attribute__((aligned(16))) Run16 { uint16_t v[8]; };

}  // namespace

// ------------------------------------------------------------------------------------------------
// Keys and values of 32-token tiles. Workgroup (tile group, head, sequence); wave w takes tile
// 8 * blockIdx.x + w. The head's B_k rows sit in LDS in MFMA A-operand order (as in the decode
// score kernel); B_v^h, already in B-operand fragment order (prefill_bv_frags), is copied into LDS
// 64 rows at a time and shared by the eight tiles.
// ------------------------------------------------------------------------------------------------
template <int D, int K>
__global__ __launch_bounds__(64 * kPkWaves, 4) void prefill_kv(const PrefillKVParams p) {
    constexpr int NF = D / 2;            // RoPE frequencies
    constexpr int HMT = D / 64;          // m-tile pairs (mt, mt + HMT) of the rebuilt keys
    constexpr int MT = D / 32;
    constexpr int KSTEPS = D / 16;       // steps of S^T = K Q^T
    constexpr int MAXKS = D / 16;        // rank steps (ranks <= d)
    constexpr int NT = D / 32;           // 32-dim tiles of the values
    using Fr = typename Elem<K>::frag;
    using T = typename Elem<K>::storage;

    // B_k of the head during the key stage; afterwards two buffers of B_v^h chunks, in which
    // rows c0 + 16*ks + 8*(l/32) + e of dim 32*n + l%32 sit at ((ks*NT + n)*64 + l)*8 + e
    __shared__ __attribute__((aligned(32))) T s_bk[kPfMaxFrag];
    static_assert(2 * kPkChunk * D <= kPfMaxFrag, "two value chunks fit where B_k was");
    // cos / sin of j*theta_i for lane l (j = l % 32), frequencies i = 32*pp + 8*g + 4*(l/32) + r:
    // entry [pp*4 + g][l] holds r = 0..3
    __shared__ __attribute__((aligned(16))) f32x4 s_cj[HMT * 4][64], s_sj[HMT * 4][64];
    __shared__ __attribute__((aligned(16))) float s_c0[kPkWaves][64], s_s0[kPkWaves][64];
    __shared__ double s_rev[64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int j = lane & 31;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int fill = pf_fill(p.chunk_lens, b, p.chunk, p.pos0);
    const int ntb = (fill + 31) >> 5;                          // this sequence's key tiles
    if (blockIdx.x * kPkWaves >= ntb) return;                  // the whole workgroup is past them
    const int tile = blockIdx.x * kPkWaves + wave;
    const bool active = tile < ntb;                            // wave-uniform
    const int n0 = 32 * tile;
    const bool tok_ok = n0 + j < fill;                         // this lane's key holds latents
    const int rk = p.rank[h], sr = p.srank[h], so = p.soff[h], nks = rk >> 4;
    const int kgrp = p.koff[h] >> 4;
    const T* __restrict__ zk = static_cast<const T*>(p.zk_rows) + (size_t)b * p.Tr * p.Rk;
    const T* __restrict__ zv = static_cast<const T*>(p.zv_rows) + (size_t)b * p.Tr * p.rv;
    const T* __restrict__ bkg = static_cast<const T*>(p.bk);
    const size_t rec = ((size_t)b * p.H + h) * p.ntiles + min(tile, p.ntiles - 1);
    _Float16* __restrict__ kout = reinterpret_cast<_Float16*>(static_cast<char*>(p.kv) + rec * (256 * D));
    _Float16* __restrict__ vout = kout + KSTEPS * 2 * 64 * 8;

    // Value-stage staging: chunk c of B_v^h (rows 64c ..) is CKS*NT*64 16-byte runs, ITER per
    // thread; the tile's Z_v fragments of chunk c are CKS per lane. Both are loaded one chunk
    // ahead of their use, so that their latency overlaps the previous chunk's products.
    constexpr int CKS = kPkChunk / 16;
    constexpr int RUNS = CKS * NT * 64;
    constexpr int ITER = RUNS / (64 * kPkWaves);
    static_assert(ITER * 64 * kPkWaves == RUNS, "whole runs per thread");
    const int nch = pf_padded_rank(p.rv) / kPkChunk;
    const u32x4* __restrict__ bvsrc = reinterpret_cast<const u32x4*>(static_cast<const T*>(p.bvf)) +
                                      (size_t)h * (pf_padded_rank(p.rv) >> 4) * NT * 64;
    // B_v^h is padded with zero rows to whole chunks: every chunk is RUNS runs, and the staging
    // needs neither bounds nor selects (either would let the compiler wait for the loads early).
    auto bv_load = [&](int c, u32x4 (&v)[ITER]) {
#pragma unroll
        for (int i = 0; i < ITER; ++i) v[i] = bvsrc[(size_t)c * RUNS + tid + i * 64 * kPkWaves];
    };
    auto bv_store = [&](int c, const u32x4 (&v)[ITER]) {
        u32x4* dst = reinterpret_cast<u32x4*>(s_bk) + (c & 1) * RUNS;
#pragma unroll
        for (int i = 0; i < ITER; ++i) dst[tid + i * 64 * kPkWaves] = v[i];
    };
    // The lane's key row, clamped into the fill: a key past the fill in the tile that holds the
    // fill's last key takes that key's values (so the tile's largest value, and its scale, are
    // those of its real keys) and is causally masked for every query (probability exactly 0); a
    // wave whose whole tile lies past the fill reads valid rows and stores nothing.
    // In the fragment-order rows, 8 ranks of a key are one 16-byte unit and the 32 keys of a tile
    // 512 contiguous bytes: each load of the wave reads 1 KB in two contiguous halves.
    const int zr = min(n0 + j, fill - 1);
    const T* __restrict__ zvrow = zv + (((size_t)(zr >> 5) * (p.rv >> 3) + half) * 32 + (zr & 31)) * 8;
    auto zv_load = [&](int c, Fr (&a)[CKS]) {
#pragma unroll
        for (int ks = 0; ks < CKS; ++ks)
            a[ks] = load_frag<K>(zvrow, (size_t)min(c * (kPkChunk / 8) + 2 * ks, (p.rv >> 3) - 2) * 256);
    };

    if (tid < 64) s_rev[tid] = tid < NF ? p.rope_rev[tid] : 0.0;
    __syncthreads();
    for (int e = tid; e < HMT * 4 * 64 * 4; e += 64 * kPkWaves) {
        const int r = e & 3, l = (e >> 2) & 63, pg = e >> 8;
        const int i = 32 * (pg >> 2) + 8 * (pg & 3) + 4 * (l >> 5) + r;
        const double rev = (double)(l & 31) * s_rev[i];
        float c, sn;
        sincos_rev((float)(rev - floor(rev)), &c, &sn);
        s_cj[pg][l][r] = c;
        s_sj[pg][l][r] = sn;
    }
    // B_k rows of the head in A-operand fragment order: fragment f = mt*(rank/16) + ks, lane l
    // holds rows 16*ks + 8*(l/32) + jj at column 32*mt + l%32; rows past the true rank are zero
    for (int i = tid; i < (rk >> 3) * D; i += 64 * kPkWaves) {
        const int k8 = i / D, dim = i - k8 * D;
        struct __attribute__((aligned(16))) Run { T v[8]; } run;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int k = 8 * k8 + jj;
            run.v[jj] = k < sr ? bkg[(size_t)(so + k) * D + dim] : T(0);
        }
        *reinterpret_cast<Run*>(s_bk + (((dim >> 5) * nks + (k8 >> 1)) * 64 + (k8 & 1) * 32 + (dim & 31)) * 8) = run;
    }
    __syncthreads();

    if (active) {
        if (lane < NF) {
            const double rev = (double)n0 * s_rev[lane];
            float c, sn;
            sincos_rev((float)(rev - floor(rev)), &c, &sn);
            s_c0[wave][lane] = c;
            s_s0[wave][lane] = sn;
        }
        pf_wave_sync();
        // latent fragments: lane column j = key n0 + j, eight ranks per lane (zero past the fill)
        Fr z[MAXKS];
        // the tile's 64-token block in the cache (a 32-token tile never straddles two)
        const size_t zblk = p.zk_cache ? block_id(p.pages, p.nblk_cap, b, n0 >> 6) : 0;
#pragma unroll
        for (int ks = 0; ks < MAXKS; ++ks) {
            if (tok_ok) {
                const int g = kgrp + min(ks, nks - 1);       // the 16-rank group
                if (p.zk_cache) {
                    // cache block layout: 16 ranks of each token contiguous, tokens in order
                    z[ks] = load_frag<K>(static_cast<const T*>(p.zk_cache),
                                         ((zblk * (p.Rk >> 4) + g) * 64 + ((n0 + j) & 63)) * 16 + 8 * half);
                } else {
                    // fragment-order rows: 8 ranks of key j are one 16-byte unit, 32 keys 512 bytes
                    z[ks] = load_frag<K>(zk, (((size_t)tile * (p.Rk >> 3) + 2 * g + half) * 32 + j) * 8);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) z[ks][e] = 0;
            }
        }
        // K~^T = B_k^T Z_k^T: lane holds key j, dims 32*mt + 8*(r/4) + 4*half + r%4
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
        // rotate-half RoPE to the key's position n0 + j: by j*theta (lane table), then by n0*theta
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
                    const float a1 = fmaf(-bb, sj[r], a * cj[r]), b1 = fmaf(a, sj[r], bb * cj[r]);
                    const float a2 = fmaf(-b1, s0[r], a1 * c0[r]), b2 = fmaf(a1, s0[r], b1 * c0[r]);
                    acc[pp][4 * g + r] = a2;
                    acc[pp + HMT][4 * g + r] = b2;
                    mx = fmaxf(mx, fmaxf(fabsf(a2), fabsf(b2)));
                }
            }
        mx = wave_max(mx);
        const int ek = pf_scale_exp(mx);
        const float ksc = ldexpf(1.0f, ek);
        // A operand of S^T = K Q^T, used in place: step (mt, s) takes acc[mt][8*s .. 8*s + 7]
#pragma unroll
        for (int step = 0; step < KSTEPS; ++step) {
            const int mt = step >> 1, s = step & 1;
            f16x8 kh, kl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = acc[mt][8 * s + e] * ksc;
                kh[e] = (_Float16)v;
                kl[e] = (_Float16)(v - (float)kh[e]);
            }
            *reinterpret_cast<f16x8*>(kout + ((2 * step) * 64 + lane) * 8) = kh;
            *reinterpret_cast<f16x8*>(kout + ((2 * step + 1) * 64 + lane) * 8) = kl;
        }
        if (lane == 0) p.exps[rec * 2] = ek;
    }

    // V = Z_v B_v^h: A = the tile's value-latent rows (lane row = key j), B = B_v^h from LDS.
    // The accumulator of dim tile n holds, in lane (dim 32*n + l%32, half), keys
    // 8*(r/4) + 4*half + r%4: registers 8*t .. 8*t + 7 are the A fragment of step t of
    // O^T = V^T P^T, stored as they are.
    f32x16 va[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) va[n][r] = 0.0f;
    // Two fragment buffers used in turn (the loop is unrolled by two), so that no register copy
    // makes the next chunk's loads wait; no branch inside the loop (the last step loads and
    // stages its clamped successor again, into the buffer nobody reads), so that the compiler's
    // wait counts let each load run for a whole chunk. A wave past the fill computes on clamped
    // rows and stores nothing.
    Fr a0[CKS], a1[CKS];
    u32x4 bq[ITER];
    bv_load(0, bq);
    zv_load(0, a0);
    __syncthreads();                                           // every wave is done with B_k
    bv_store(0, bq);
    bv_load(min(1, nch - 1), bq);
    __syncthreads();
    // chunk c: B_v rows in LDS buffer c & 1, the next chunk's rows in bq, the tile's latent
    // fragments in cur; the next chunk's fragments are loaded into nxt
    auto vstep = [&](int c, const Fr (&cur)[CKS], Fr (&nxt)[CKS]) __attribute__((always_inline)) {
        zv_load(min(c + 1, nch - 1), nxt);
        const T* buf = s_bk + (c & 1) * (kPkChunk * D);
#pragma unroll
        for (int ks = 0; ks < CKS; ++ks) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
                va[n] = mma32<K>(cur[ks], *reinterpret_cast<const Fr*>(buf + ((ks * NT + n) * 64 + lane) * 8), va[n]);
        }
        // the other buffer was last read in chunk c - 1, before the previous barrier
        bv_store(min(c + 1, nch - 1), bq);
        bv_load(min(c + 2, nch - 1), bq);
        __syncthreads();
    };
    for (int c = 0; c < nch; c += 2) {
        vstep(c, a0, a1);
        if (c + 1 < nch) vstep(c + 1, a1, a0);
    }
    if (active) {
        float mx = 0.0f;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(va[n][r]));
        mx = wave_max(mx);
        // values keep their own scale (exponent 0) unless the tile's largest would overflow the
        // binary16 hi part or leave its lo part in the subnormal range: the attention kernel then
        // rarely has to move its accumulators to another scale
        const int ev = (mx > 16384.0f || (mx > 0.0f && mx < 0x1p-10f)) ? pf_scale_exp(mx) : 0;
        const float vsc = ldexpf(1.0f, ev);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f16x8 vh, vl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = va[n][8 * t + e] * vsc;
                    vh[e] = (_Float16)v;
                    vl[e] = (_Float16)(v - (float)vh[e]);
                }
                *reinterpret_cast<f16x8*>(vout + (((n * 2 + t) * 2) * 64 + lane) * 8) = vh;
                *reinterpret_cast<f16x8*>(vout + (((n * 2 + t) * 2 + 1) * 64 + lane) * 8) = vl;
            }
        if (lane == 0) p.exps[rec * 2 + 1] = ev;
    }
}

// ------------------------------------------------------------------------------------------------
// Attention. Workgroup (128-query block, head, sequence); wave w takes queries 128*block + 32*w ..
// +31. The four waves share each key tile's record through LDS (double-buffered: the next record
// is loaded into registers while the current one is used). Lane l holds query l % 32 in S^T and in
// O^T (both halves of the wave hold the same queries), so the running maximum, sum and rescaling
// are per-lane scalars.
// Every query block of a (sequence, head) reads that pair's records up to its diagonal, so the
// grid is one-dimensional and laid out for the eight XCDs (workgroup i runs on XCD i mod 8): all
// query blocks of one pair land on the same XCD, consecutively and the longest first, so they
// stream the same records through that XCD's L2 at about the same time.
// ------------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * kPaWaves, 2) void prefill_attend(const PrefillFlashParams p) {
    constexpr int KSTEPS = D / 16;
    constexpr int NT = D / 32;
    constexpr int REC = 256 * D;                              // bytes per key tile record
    constexpr int LOADS = REC / (16 * 64 * kPaWaves);          // 16-byte loads per thread
    __shared__ __attribute__((aligned(16))) u32x4 s_rec[2][REC / 16];
    __shared__ int s_ex[2][2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int j = lane & 31;
    const int nqb = (p.chunk + 32 * kPaWaves - 1) / (32 * kPaWaves);
    const int xcd = blockIdx.x & 7, u = blockIdx.x >> 3;
    const int pair = (u / nqb) * 8 + xcd;                      // (sequence, head) = b * H + h
    if (pair >= p.B * p.H) return;                             // padding of the last round
    const int h = pair % p.H;
    const int b = pair / p.H;
    const int qb = nqb - 1 - u % nqb;
    const int clen = p.chunk_lens ? min(max(p.chunk_lens[b], 0), p.chunk) : p.chunk;
    const int L0 = 32 * kPaWaves * qb;                         // the workgroup's first query
    const int l0 = L0 + 32 * wave;                             // the wave's
    const int lq = l0 + j;                                     // this lane's
    const bool qvalid = lq < clen;
    const int qpos = p.pos0 + lq;
    const int wl = min(l0 + 31, clen - 1);                     // the wave's last valid query
    const int wtiles = wl >= l0 ? ((p.pos0 + wl) >> 5) + 1 : 0;
    const int bl = min(L0 + 32 * kPaWaves - 1, clen - 1);
    const int btiles = bl >= L0 ? ((p.pos0 + bl) >> 5) + 1 : 0;
    const u32x4* __restrict__ recs = reinterpret_cast<const u32x4*>(p.kv) + ((size_t)b * p.H + h) * p.ntiles * (REC / 16);
    const int32_t* __restrict__ ex = p.exps + ((size_t)b * p.H + h) * p.ntiles * 2;

    int eq;                              // the queries' power-of-two scale exponent
    // the wave's queries, scaled (softmax scale and log2 e, and a power of two for the 16-bit
    // parts) and split into the B operand of S^T: lane (query j, half), step (mt, s), entry e:
    // dim 32*mt + 16*s + 8*(e/4) + 4*half + e%4 (the key fragments' order)
    // The two lanes of a query hold all of its dims between them, so the scale exponent comes
    // from the loaded registers (all loads in flight at once) as the largest |q * scale| over
    // the wave's valid queries.
    f16x8 qh[KSTEPS], ql[KSTEPS];
    {
        const float* qrow = p.q + (((size_t)b * p.chunk + min(lq, p.chunk - 1)) * p.H + h) * D;
        f32x4 qv[KSTEPS][2];
#pragma unroll
        for (int step = 0; step < KSTEPS; ++step) {
            const int base = 32 * (step >> 1) + 16 * (step & 1) + 4 * half;
            qv[step][0] = *reinterpret_cast<const f32x4*>(qrow + base);
            qv[step][1] = *reinterpret_cast<const f32x4*>(qrow + base + 8);
        }
        float qm = 0.0f;
        if (qvalid) {
#pragma unroll
            for (int step = 0; step < KSTEPS; ++step)
#pragma unroll
                for (int e = 0; e < 8; ++e) qm = fmaxf(qm, fabsf(qv[step][e >> 2][e & 3] * p.q_scale));
        }
        qm = wave_max(qm);
        const int eq0 = pf_scale_exp(qm);
        const float qs = ldexpf(p.q_scale, eq0);
#pragma unroll
        for (int step = 0; step < KSTEPS; ++step)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = qvalid ? qv[step][e >> 2][e & 3] * qs : 0.0f;
                qh[step][e] = (_Float16)v;
                ql[step][e] = (_Float16)(v - (float)qh[step][e]);
            }
        eq = eq0;
    }

    float m = -INFINITY, l = 0.0f;       // running maximum (an integer, log2 units) and sum
    int E = 0;                           // acc holds O^T * 2^E
    f32x16 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[n][r] = 0.0f;

    // one key tile of the record in LDS buffer buf; masked: the tile reaches past the wave's first
    // query (or the wave holds queries past its chunk), so keys are compared with positions
    auto attend_tile = [&](int kt, int buf, bool masked) __attribute__((always_inline)) {
            const _Float16* kb = reinterpret_cast<const _Float16*>(s_rec[buf]);
            const _Float16* vb = kb + KSTEPS * 2 * 64 * 8;
            f32x16 st;
#pragma unroll
            for (int r = 0; r < 16; ++r) st[r] = 0.0f;
            // key fragments read one step ahead of their products
            f16x8 kf[2][2];
            kf[0][0] = *reinterpret_cast<const f16x8*>(kb + lane * 8);
            kf[0][1] = *reinterpret_cast<const f16x8*>(kb + (64 + lane) * 8);
#pragma unroll
            for (int step = 0; step < KSTEPS; ++step) {
                if (step + 1 < KSTEPS) {
                    kf[(step + 1) & 1][0] = *reinterpret_cast<const f16x8*>(kb + ((2 * step + 2) * 64 + lane) * 8);
                    kf[(step + 1) & 1][1] = *reinterpret_cast<const f16x8*>(kb + ((2 * step + 3) * 64 + lane) * 8);
                }
                __builtin_amdgcn_sched_barrier(0);             // keep the reads ahead of the products
                st = mma32<kF16>(kf[step & 1][0], qh[step], st);
                st = mma32<kF16>(kf[step & 1][0], ql[step], st);
                st = mma32<kF16>(kf[step & 1][1], qh[step], st);
            }
            const int ek = s_ex[buf][0], ev = s_ex[buf][1];
            // a power of two (scaling is exact), kept above 0 so that a masked -inf stays -inf
            const float un = ldexpf(1.0f, -min(ek + eq, 149));
            // lane: query j, keys 32*kt + 8*(r/4) + 4*half + r%4. A masked product becomes -inf,
            // whose weight below is exactly 0; only the wave's last tiles take this branch.
            if (masked) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kpos = 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
                    if (!(qvalid && kpos <= qpos)) st[r] = -INFINITY;
                }
            }
            float tm = st[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) tm = fmaxf(tm, st[r]);
            {
                const LanePair pr = swap32(tm);
                tm = fmaxf(pr.a, pr.b) * un;
            }
            // the new running maximum, rounded up to an integer: the factors below are exact
            const float mn = tm == -INFINITY ? m : fmaxf(m, ceilf(tm));
            const float fl = m == -INFINITY ? 0.0f : ldexpf(1.0f, (int)(m - mn));
            const float g = ldexpf(fl, ev - E);               // sums rescaled, values' frame moved to ev
            // with no key seen yet (mn = -inf) every product here is -inf: offset 0 keeps exp2 at 0
            const float mo = mn == -INFINITY ? 0.0f : mn;
            f16x8 pf[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (_Float16)__builtin_amdgcn_exp2f(fmaf(st[r], un, -mo));
            // the sum of the stored values (fp32 sums of binary16 pairs), so that the normaliser
            // carries the same rounding as the weights
            float ls = 0.0f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const f16x2 pr2 = {pf[t][2 * k], pf[t][2 * k + 1]};
                    ls = __builtin_amdgcn_fdot2(pr2, (f16x2){(_Float16)1.0f, (_Float16)1.0f}, ls, false);
                }
            ls = add_xor32(ls);
            l = l * fl + ls;
            m = mn;
            E = ev;
            if (__builtin_amdgcn_ballot_w64(g != 1.0f)) {      // some lane's sums move
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[n][r] *= g;
            }
            // value fragments, likewise one (dim tile, key half) ahead
            f16x8 vf[2][2];
            vf[0][0] = *reinterpret_cast<const f16x8*>(vb + lane * 8);
            vf[0][1] = *reinterpret_cast<const f16x8*>(vb + (64 + lane) * 8);
#pragma unroll
            for (int u = 0; u < 2 * NT; ++u) {
                if (u + 1 < 2 * NT) {
                    vf[(u + 1) & 1][0] = *reinterpret_cast<const f16x8*>(vb + ((2 * u + 2) * 64 + lane) * 8);
                    vf[(u + 1) & 1][1] = *reinterpret_cast<const f16x8*>(vb + ((2 * u + 3) * 64 + lane) * 8);
                }
                __builtin_amdgcn_sched_barrier(0);
                const int n = u >> 1, t = u & 1;               // u = n * 2 + t
                acc[n] = mma32<kF16>(vf[u & 1][0], pf[t], acc[n]);
                acc[n] = mma32<kF16>(vf[u & 1][1], pf[t], acc[n]);
            }
    };

    // Records are loaded one tile ahead: tile kt + 1's loads are issued (into registers) at the
    // start of tile kt and land in the other LDS buffer at its end.
    struct Pref { u32x4 r[LOADS]; int x; };
    auto issue = [&](int kt) __attribute__((always_inline)) {
        Pref f;
        const u32x4* src = recs + (size_t)kt * (REC / 16);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) f.r[i] = src[tid + i * 64 * kPaWaves];
        // every thread loads (one of the two exponents), so that the count of loads in flight is
        // static and the compiler's in-order wait counts stay exact
        f.x = ex[kt * 2 + (tid & 1)];
        return f;
    };
    auto land = [&](const Pref& f, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) s_rec[buf][tid + i * 64 * kPaWaves] = f.r[i];
        if (tid < 2) s_ex[buf][tid] = f.x;
    };
    if (btiles > 0) land(issue(0), 0);
    __syncthreads();
    for (int kt = 0; kt < btiles; ++kt) {
        const int buf = kt & 1;
        Pref nxt;
        if (kt + 1 < btiles) nxt = issue(kt + 1);
        if (kt < wtiles) {
            // a tile wholly below the wave's first query, with every query of the wave valid,
            // needs no mask (wave-uniform); only the wave's last tiles take the masked form
            attend_tile(kt, buf, !(32 * kt + 31 <= p.pos0 + l0 && l0 + 31 < clen));
        }
        if (kt + 1 < btiles) land(nxt, buf ^ 1);
        __syncthreads();
    }

    // O = O^T * 2^-E / l; a query past its sequence's chunk (l == 0) writes zeros
    if (lq < p.chunk) {
        const float inv = l > 0.0f ? ldexpf(1.0f, -E) / l : 0.0f;
        float* orow = p.out + (((size_t)b * p.chunk + lq) * p.H + h) * D;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 o = {acc[n][4 * g] * inv, acc[n][4 * g + 1] * inv, acc[n][4 * g + 2] * inv,
                                 acc[n][4 * g + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + 32 * n + 8 * g + 4 * half) = o;
            }
    }
}

// B_v^h in the B-operand fragment order of V = Z_v B_v^h, for every head: element
// ((h * (rv/16) + ks) * (D/32) + n) * 512 + l * 8 + e = B_v[16*ks + 8*(l/32) + e][h*D + 32*n + l%32]
// (zero for rows past rv_src). Thread per (h, ks, n, lane): eight rows, one 16-byte store.
template <int D>
__global__ __launch_bounds__(256) void prefill_bv_frags(const PrefillKVParams p) {
    constexpr int NT = D / 32;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const int kst = pf_padded_rank(p.rv) >> 4;       // rank steps, zero rows past r_v
    const long long n_items = (long long)p.H * kst * NT * 64;
    if (idx >= n_items) return;
    const int l = (int)(idx & 63);
    const long long f = idx >> 6;                     // (h, ks, n)
    const int n = (int)(f % NT);
    const int ks = (int)((f / NT) % kst);
    const int h = (int)(f / NT / kst);
    const uint16_t* bv = static_cast<const uint16_t*>(p.bv);
    const size_t col = (size_t)h * D + 32 * n + (l & 31);
    Run16 run;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int c = 16 * ks + 8 * (l >> 5) + e;
        run.v[e] = c < p.rv_src ? bv[(size_t)c * p.H * D + col] : (uint16_t)0;
    }
    reinterpret_cast<Run16*>(p.bvf)[idx] = run;
}

template <int D, int K>
static hipError_t launch_kv_d(const PrefillKVParams& p, hipStream_t st) {
    const long long n_items = (long long)p.H * (pf_padded_rank(p.rv) >> 4) * (D / 32) * 64;
    hipLaunchKernelGGL(prefill_bv_frags<D>, dim3((unsigned)((n_items + 255) / 256)), dim3(256), 0, st, p);
    const dim3 grid((p.ntiles + kPkWaves - 1) / kPkWaves, p.H, p.B);
    hipLaunchKernelGGL((prefill_kv<D, K>), grid, dim3(64 * kPkWaves), 0, st, p);
    return hipGetLastError();
}

// elem: kF16 / kBF16 (the latent rows' and factors' type)
hipError_t launch_prefill_kv(const PrefillKVParams& p, int elem, hipStream_t st) {
    if (p.D == 128) {
        if (elem == kF16) return launch_kv_d<128, kF16>(p, st);
        if (elem == kBF16) return launch_kv_d<128, kBF16>(p, st);
    } else if (p.D == 64) {
        if (elem == kF16) return launch_kv_d<64, kF16>(p, st);
        if (elem == kBF16) return launch_kv_d<64, kBF16>(p, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_attend(const PrefillFlashParams& p, hipStream_t st) {
    const long long nqb = (p.chunk + 32 * kPaWaves - 1) / (32 * kPaWaves);
    const long long pairs8 = ((long long)p.B * p.H + 7) / 8;   // (sequence, head) pairs per XCD
    const dim3 grid((unsigned)(pairs8 * nqb * 8));
    if (p.D == 128) hipLaunchKernelGGL(prefill_attend<128>, grid, dim3(64 * kPaWaves), 0, st, p);
    else if (p.D == 64) hipLaunchKernelGGL(prefill_attend<64>, grid, dim3(64 * kPaWaves), 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace starkv
