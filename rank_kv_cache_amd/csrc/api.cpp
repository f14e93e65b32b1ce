// api.cpp -- host side of the C ABI declared in include/starkv.h: argument validation (entirely
// before anything is enqueued), the split planner, workspace carving and kernel launches.

#include "starkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "prefill.hpp"

namespace starkv {
hipError_t launch_latent_scores(const ScoreParams& p, int elem, int groups, int splits, int maxks,
                                int nq, hipStream_t st);
hipError_t launch_latent_values(const ValueParams& p, int elem, int chunks, int ntw, int nq,
                                hipStream_t st);
int value_tiles_per_wave(int rv);
hipError_t launch_linear(const LinearParams& p, int elem, hipStream_t st);
int linear_rows_per_workgroup(int elem);
hipError_t launch_linear_store(const LinearStoreParams& p, int elem, hipStream_t st);
hipError_t launch_merge(const MergeParams& p, hipStream_t st);
hipError_t launch_project(const ProjectParams& p, int elem, hipStream_t st);
hipError_t launch_row_fill(const RowFillParams& p, hipStream_t st);
hipError_t launch_prefill_kv(const PrefillKVParams& p, int elem, hipStream_t st);
hipError_t launch_prefill_attend(const PrefillFlashParams& p, hipStream_t st);
hipError_t launch_dense_split(const DenseDecodeParams& p, int elem, hipStream_t st);

hipError_t launch_copy_rows(const RowCopyParams& p, int B, hipStream_t st);
hipError_t launch_block_transpose(const BlockXposeParams& p, int elem_bytes, hipStream_t st,
                                  bool frag_rows = false);
hipError_t launch_append_small(const AppendSmallParams& p, int elem_bytes, hipStream_t st);
hipError_t launch_padded_rows(const PaddedRowsParams& p, int elem_bytes, hipStream_t st);
hipError_t launch_paged_rows(const PagedRowsParams& p, hipStream_t st);
hipError_t launch_q43_quantize(const Q43QuantParams& p, int ngroups, hipStream_t st);
hipError_t launch_q43_readback(const Q43ReadParams& p, hipStream_t st, bool frag_rows = false);
hipError_t launch_hadamard_rotate(const HadamardParams& p, hipStream_t st);
}  // namespace starkv

using namespace starkv;

namespace {

constexpr int kTargetWorkgroups = 256;   // MI355X compute units: one score workgroup per CU
constexpr int kValueTargetWorkgroups = 512;   // two 4-wave value workgroups per CU
constexpr int kMaxScoreRounds = 4;
constexpr int kMaxSplits = 256;
constexpr size_t kAlign = 256;
constexpr int64_t kSmallAppend = 16;     // appends of up to this many tokens use one fused launch

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elem_bytes(int dt) { return dt == STARKV_F32 ? 4 : 2; }

inline int elem_kind(int dt) {
    return dt == STARKV_F32 ? kF32 : dt == STARKV_BF16 ? kBF16 : kF16;
}

// Ranks as stored (rounded up to the 16-channel tile: rv, Rk, koff, rank) and as the caller
// passes rows and factors (rv_src, Rk_src, soff, srank); `padded` when they differ.
struct LayerInfo {
    int H = 0, D = 0, rv = 0, Rk = 0;
    int rv_src = 0, Rk_src = 0;
    bool dense = false, q43 = false, padded = false;
    int cache_dt = 0, factor_dt = 0;
    double top_fraction = 0.0;
    int16_t koff[kMaxHeads + 1] = {0};
    int16_t rank[kMaxHeads] = {0};
    int16_t soff[kMaxHeads + 1] = {0};
    int16_t srank[kMaxHeads] = {0};
};

// Validates the layer descriptor (host arithmetic only).
starkv_status check_layer(const starkv_layer* L, LayerInfo* out) {
    if (!L) return STARKV_ERR_NULL;
    LayerInfo li;
    li.H = L->num_heads;
    li.D = L->head_dim;
    li.dense = L->dense != 0;
    li.cache_dt = L->cache_dtype;
    li.factor_dt = L->factor_dtype;
    if (li.H < 1 || li.D < 2 || (li.D & 1)) return STARKV_ERR_SHAPE;
    if (!(L->rope_base > 1.0) || !std::isfinite(L->rope_base)) return STARKV_ERR_SHAPE;
    if (std::isnan(L->sm_scale) || std::isinf(L->sm_scale)) return STARKV_ERR_SHAPE;
    if (li.cache_dt < STARKV_F32 || li.cache_dt > STARKV_Q43) return STARKV_ERR_DTYPE;
    if (li.H > kMaxHeads || (li.D != 64 && li.D != 128)) return STARKV_ERR_UNSUPPORTED;
    if (li.dense) {
        if (li.cache_dt == STARKV_Q43) return STARKV_ERR_DTYPE;
        *out = li;
        return STARKV_OK;
    }
    if (!L->key_ranks) return STARKV_ERR_NULL;
    const int want_factor = li.cache_dt == STARKV_Q43 ? STARKV_F16 : li.cache_dt;
    if (li.factor_dt != want_factor) return STARKV_ERR_DTYPE;
    // fp caches take any rank and store it rounded up to the 16-channel tile (zero channels);
    // the mixed 4/3-bit layout is built on whole 16-channel groups and needs multiples of 16
    const bool q43 = li.cache_dt == STARKV_Q43;
    int off = 0, soff = 0;
    for (int h = 0; h < li.H; ++h) {
        const int r = L->key_ranks[h];
        if (r < 1 || r > li.D || (q43 && r % 16)) return STARKV_ERR_RANK_ALIGN;
        const int rp = (r + 15) / 16 * 16;
        li.koff[h] = static_cast<int16_t>(off);
        li.rank[h] = static_cast<int16_t>(rp);
        li.soff[h] = static_cast<int16_t>(soff);
        li.srank[h] = static_cast<int16_t>(r);
        off += rp;
        soff += r;
    }
    li.koff[li.H] = static_cast<int16_t>(off);
    li.soff[li.H] = static_cast<int16_t>(soff);
    li.Rk = off;
    li.Rk_src = soff;
    li.rv_src = L->value_rank;
    if (li.rv_src < 1 || li.rv_src > 2048 || (q43 && li.rv_src % 16)) return STARKV_ERR_RANK_ALIGN;
    li.rv = (li.rv_src + 15) / 16 * 16;
    li.padded = li.Rk != li.Rk_src || li.rv != li.rv_src;
    if (li.cache_dt == STARKV_Q43) {
        li.q43 = true;
        if (L->q_group != 64) return STARKV_ERR_UNSUPPORTED;
        if (L->q_bits_hi != 4 || L->q_bits_lo != 3) return STARKV_ERR_UNSUPPORTED;
        if (!(L->q_top_fraction >= 0.0f && L->q_top_fraction <= 1.0f)) return STARKV_ERR_SHAPE;
        if (li.Rk > kMaxKeyGroups * 16) return STARKV_ERR_UNSUPPORTED;
        li.top_fraction = L->q_top_fraction;
    }
    *out = li;
    return STARKV_OK;
}

starkv_status check_cache(const starkv_cache* c, const LayerInfo& li) {
    if (!c) return STARKV_ERR_NULL;
    if (c->batch < 0 || c->capacity < 0) return STARKV_ERR_SHAPE;
    if (c->capacity == 0 || (c->capacity % kTile)) return STARKV_ERR_CAPACITY;
    if (c->batch == 0) return STARKV_OK;
    if (!c->zk || !c->zv) return STARKV_ERR_NULL;
    if (!aligned16(c->zk) || !aligned16(c->zv)) return STARKV_ERR_MISALIGNED;
    if (c->block_table) {
        if (c->table_stride < c->capacity / kTile) return STARKV_ERR_CAPACITY;
        if (reinterpret_cast<uintptr_t>(c->block_table) & 3) return STARKV_ERR_MISALIGNED;
    }
    if (li.q43) {
        if (!c->zk_meta || !c->zv_meta || !c->zk_tail || !c->zv_tail) return STARKV_ERR_NULL;
        if (!aligned16(c->zk_meta) || !aligned16(c->zv_meta) || !aligned16(c->zk_tail) ||
            !aligned16(c->zv_tail))
            return STARKV_ERR_MISALIGNED;
    }
    return STARKV_OK;
}

// Channels of a latent of width r kept at 4 bits: the leading ceil(top_fraction * r). The
// fraction arrives as binary32, so products within 1e-4 of an integer count as that integer
// (0.2f * 80 = 16.0000002 gives 16, not 17).
int q43_hi_channels(int r, double frac) {
    const int n = static_cast<int>(std::ceil(frac * r - 1e-4));
    return std::max(0, std::min(r, n));
}

void q43_layouts(const LayerInfo& li, Q43Layout* K, Q43Layout* V) {
    std::memset(K, 0, sizeof(*K));
    std::memset(V, 0, sizeof(*V));
    K->C = li.Rk;
    K->is_key = 1;
    int off = 0, g = 0;
    for (int h = 0; h < li.H; ++h) {
        const int r = li.rank[h];
        const int nh = q43_hi_channels(r, li.top_fraction);
        for (int k = 0; k < r / 16; ++k, ++g) {
            const int n = std::max(0, std::min(16, nh - 16 * k));
            K->gn[g] = static_cast<uint8_t>(n);
            K->goff[g] = off;
            off += 384 + 8 * n;
        }
    }
    K->block_bytes = off;
    V->C = li.rv;
    V->is_key = 0;
    V->n_hi = q43_hi_channels(li.rv, li.top_fraction);
    V->block_bytes = 32 * V->n_hi + 24 * (li.rv - V->n_hi);
}

constexpr size_t kQ43CodePad = 32;   // readers load aligned windows that may pass a block's end

// Score-kernel head groups: the heads are dealt to G groups with balanced rank sums
// (longest-processing-time-first greedy); G is the smallest count whose largest group's factor
// fragments fit the LDS budget of one workgroup.
struct ScorePlan {
    int G = 1, splits = 1, bpw = 1, maxks = 1;
    int8_t order[kMaxHeads] = {0};
    int8_t gstart[kMaxGroups + 1] = {0};
};

// nq query rows per sequence share the score workgroup: more than one leaves a smaller factor
// budget and at most kMaxGroupHeadsMQ heads per group
bool plan_groups(const LayerInfo& li, int G, ScorePlan* sp, int nq = 1) {
    std::vector<int> order(li.H);
    for (int h = 0; h < li.H; ++h) order[h] = h;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return li.rank[a] > li.rank[b]; });
    std::vector<std::vector<int>> groups(G);
    std::vector<int> load(G, 0);
    for (int h : order) {
        int g = 0;
        for (int k = 1; k < G; ++k)
            if (load[k] < load[g]) g = k;
        groups[g].push_back(h);
        load[g] += li.rank[h];
    }
    const int esz = elem_bytes(li.factor_dt);
    int pos = 0;
    const size_t budget = static_cast<size_t>(nq > 1 ? kFragLdsBytesMQ : kFragLdsBytes);
    for (int g = 0; g < G; ++g) {
        if (static_cast<size_t>(load[g]) * li.D * esz > budget) return false;
        if (nq > 1 && groups[g].size() > static_cast<size_t>(kMaxGroupHeadsMQ)) return false;
        sp->gstart[g] = static_cast<int8_t>(pos);
        for (int h : groups[g]) sp->order[pos++] = static_cast<int8_t>(h);
    }
    sp->gstart[G] = static_cast<int8_t>(pos);
    sp->G = G;
    return true;
}

// B: cache sequences (one workgroup each per group and split), whatever their query rows
ScorePlan plan_scores(const LayerInfo& li, int B, int nblk, int nq = 1) {
    ScorePlan sp;
    // one head per group always fits (a rank-d head needs at most d * d * 4 bytes of fragments)
    int G = 1;
    while (G < li.H && !plan_groups(li, G, &sp, nq)) ++G;
    if (G == li.H) plan_groups(li, G, &sp, nq);
    int maxr = 0;
    for (int h = 0; h < li.H; ++h) maxr = std::max(maxr, static_cast<int>(li.rank[h]));
    sp.maxks = maxr / 16;
    // One score workgroup fills a CU. Choose the split count so that the grid's last round of
    // workgroups is as full as possible, preferring fewer rounds (each workgroup pays a prologue).
    const int per = std::max(1, B) * sp.G;
    int S = 1;
    double best = -1.0;
    for (int rounds = 1; rounds <= kMaxScoreRounds; ++rounds) {
        const int s_try = std::max(1, std::min(nblk, rounds * kTargetWorkgroups / per));
        const int wgs = per * s_try;
        const int used = (wgs + kTargetWorkgroups - 1) / kTargetWorkgroups;
        const double eff = static_cast<double>(wgs) / (used * kTargetWorkgroups);
        if (eff > best + 0.02) {
            best = eff;
            S = s_try;
        }
    }
    sp.bpw = (nblk + S - 1) / S;
    sp.splits = (nblk + sp.bpw - 1) / sp.bpw;
    return sp;
}

struct ValuePlan {
    int chunks = 1, splits = 1, bps = 1, ntw = 4;
};

// B: cache sequences; nq query rows each share a workgroup (four channel tiles' accumulators in
// all: 4 / nq tiles per wave) and splits of at most kMaxBlocksPerSplit / nq blocks
ValuePlan plan_values(const LayerInfo& li, int B, int nblk, int requested, int nq = 1) {
    ValuePlan vp;
    vp.ntw = nq > 1 ? 4 / nq
                    : li.cache_dt == STARKV_F32 ? 2 : value_tiles_per_wave(li.rv);   // fp32 operands: 2 tiles fit
    const int chunk_channels = kValueWaves * vp.ntw * 32;
    vp.chunks = (li.rv + chunk_channels - 1) / chunk_channels;
    const int per = std::max(1, B) * vp.chunks;
    const int max_bps = kMaxBlocksPerSplit / nq;
    // The four-tile form (≤ 256 VGPRs: two workgroups per CU at most) streams binary16 / bf16 value
    // latents fastest as one long stream per CU (measured: LongChat layer, B = 16, T = 32768:
    // 182 µs with 256 workgroups vs 193-203 µs with 512); the two-tile form, the mixed 4/3-bit
    // form (dequantisation in registers) and the multi-query forms keep two or more per CU.
    const int target = (nq == 1 && !li.q43 && vp.ntw == 4) ? kValueTargetWorkgroups / 2
                                                          : kValueTargetWorkgroups;
    int S = requested > 0 ? requested : (target + per - 1) / per;
    S = std::max({1, std::min(S, nblk), (nblk + max_bps - 1) / max_bps});
    S = std::min(S, kMaxSplits);
    vp.bps = (nblk + S - 1) / S;
    vp.splits = (nblk + vp.bps - 1) / vp.bps;
    return vp;
}

// Exempt-layer splits: about three 4-wave workgroups per compute unit (the kernel's register
// use allows three waves per SIMD). Each split is a whole number of 64-token blocks and no split
// is empty.
constexpr int kDenseTargetWorkgroups = 768;

int plan_splits(int B, int64_t seq_len, int requested) {
    const int ntiles = static_cast<int>((seq_len + kTile - 1) / kTile);
    int S = requested > 0 ? requested
                          : (kDenseTargetWorkgroups + std::max(B, 1) - 1) / std::max(B, 1);
    S = std::max(1, std::min({S, ntiles, kMaxSplits}));
    const int tps = (ntiles + S - 1) / S;
    return (ntiles + tps - 1) / tps;
}

// Longest sequence a decode call takes: at most kMaxSplits splits, and for latent layers at most
// kMaxBlocksPerSplit / nq blocks per split (the value kernel keeps a per-split table of that many
// 32-token tile factors per query row and head in LDS).
int64_t max_decode_len(const LayerInfo& li, int nq) {
    const int64_t bps = li.dense ? kMaxBlocksPerSplit : kMaxBlocksPerSplit / std::max(1, nq);
    return static_cast<int64_t>(kMaxSplits) * bps * kTile;
}

struct WorkspaceLayout {
    size_t P = 0, stats = 0, ml = 0, acc = 0, fill = 0, total = 0;
    int S = 1, tps = 1, nblk = 1;
    ScorePlan sp;
    ValuePlan vp;
};

// B: query rows (nq per cache sequence)
WorkspaceLayout workspace_layout(const LayerInfo& li, int B, int64_t seq_len, int requested, int nq = 1) {
    WorkspaceLayout w;
    const int nblk = static_cast<int>((seq_len + kTile - 1) / kTile);
    w.nblk = nblk;
    size_t off = 0;
    if (li.dense) {
        w.S = plan_splits(B, seq_len, requested);
        w.tps = (nblk + w.S - 1) / w.S;
        w.ml = off;
        off += align_up(static_cast<size_t>(B) * w.S * li.H * 2 * sizeof(float));
        w.acc = off;
        off += align_up(static_cast<size_t>(B) * w.S * li.H * li.D * sizeof(float));
        w.total = off;
        return w;
    }
    w.sp = plan_scores(li, B / nq, nblk, nq);
    w.vp = plan_values(li, B / nq, nblk, requested, nq);
    w.S = w.vp.splits;
    w.tps = w.vp.bps;
    const size_t Tp = static_cast<size_t>(nblk) * kTile;
    const size_t pesz = li.cache_dt == STARKV_F32 ? 4 : 2;
    w.P = off;
    off += align_up(static_cast<size_t>(B) * li.H * Tp * pesz);
    w.stats = off;                      // (m, l) per 32-token tile
    off += align_up(static_cast<size_t>(B) * li.H * 2 * nblk * 2 * sizeof(float));
    w.ml = off;
    off += align_up(static_cast<size_t>(B) * w.S * li.H * 2 * sizeof(float));
    w.acc = off;
    off += align_up(static_cast<size_t>(B) * w.S * li.H * li.rv * sizeof(float));
    w.fill = off;                       // per query row: its cache sequence's fill (mixed caches)
    off += align_up(static_cast<size_t>(B) * sizeof(int32_t));
    w.total = off;
    return w;
}

// Prefill: query rows b * chunk + l, grouped nq at a time for the value kernel (4, 2 or 1: the
// largest that divides the chunk, so that no group straddles two sequences); the decode workspace
// of those rows plus per-row lengths, per-row fills and the group-to-sequence map.
// Prefill workspace: the latent rows of tokens [0, pos0 + chunk) (binary16, or bfloat16 for a
// bfloat16 cache), B_v in MFMA fragment order, then one key/value record of 256 * d bytes and two
// exponents per (sequence, head, 32-token tile).
struct PrefillLayout {
    int64_t Tk = 0;
    int ntiles = 0;
    size_t zk_rows = 0, zv_rows = 0, bvf = 0, kv = 0, exps = 0, total = 0;
};

PrefillLayout prefill_layout(const LayerInfo& li, int B, int64_t pos0, int chunk) {
    PrefillLayout pl;
    pl.Tk = pos0 + chunk;
    pl.ntiles = static_cast<int>((pl.Tk + 31) / 32);
    const size_t b = static_cast<size_t>(B);
    size_t off = 0;
    // latent rows in fragment order: whole 32-token tiles per sequence
    const size_t T32 = static_cast<size_t>(pl.ntiles) * 32;
    pl.zk_rows = off;                               // 16-bit caches: keys read from the cache
    if (li.q43) off += align_up(b * T32 * li.Rk * 2);
    pl.zv_rows = off;
    off += align_up(b * T32 * li.rv * 2);
    pl.bvf = off;                                   // ranks padded with zero rows to a multiple of 64
    off += align_up(static_cast<size_t>((li.rv + 63) / 64 * 64) * li.H * li.D * 2);
    pl.kv = off;
    off += align_up(b * li.H * pl.ntiles * 256 * static_cast<size_t>(li.D));
    pl.exps = off;
    off += align_up(b * li.H * pl.ntiles * 2 * sizeof(int32_t));
    pl.total = off;
    return pl;
}

void fill_rope(double base, int D, double* rev) {
    for (int i = 0; i < D / 2; ++i)
        rev[i] = std::pow(base, (-2.0 * i) / D) / (2.0 * M_PI);
}

float q_scale_of(const starkv_layer* L, int D) {
    const double scale = L->sm_scale > 0.0f ? static_cast<double>(L->sm_scale) : 1.0 / std::sqrt(D);
    return static_cast<float>(scale * 1.4426950408889634);   // log2(e): softmax done in base 2
}

inline starkv_status dev(hipError_t e) { return e == hipSuccess ? STARKV_OK : STARKV_ERR_DEVICE; }

BlockMap pages_of(const starkv_cache* c) {
    BlockMap m;
    m.table = c->block_table;
    m.stride = c->table_stride;
    return m;
}

// Dense rows of a paged cache: rows [B][n][H*d] <-> tokens t0 .. t0 + n - 1 (or positions[b])
starkv_status dense_paged(const LayerInfo& li, const starkv_cache* cache, const void* k_rows,
                          const void* v_rows, int to_cache, int64_t t0, int64_t n,
                          hipStream_t st, const int32_t* positions = nullptr) {
    for (int which = 0; which < 2; ++which) {
        const void* rows = which ? v_rows : k_rows;
        if (!rows) continue;
        PagedRowsParams p;
        p.rows = static_cast<const char*>(rows);
        p.cache = static_cast<char*>(which ? cache->zv : cache->zk);
        p.row_bytes = static_cast<long long>(li.H) * li.D * elem_bytes(li.cache_dt);
        p.t0 = t0;
        p.n = n;
        p.B = cache->batch;
        p.nblk_cap = static_cast<int>(cache->capacity / kTile);
        p.to_cache = to_cache;
        p.positions = positions;
        p.pages = pages_of(cache);
        const starkv_status s = dev(launch_paged_rows(p, st));
        if (s != STARKV_OK) return s;
    }
    return STARKV_OK;
}

PadMap pad_map(const LayerInfo& li) {
    PadMap m;
    std::memset(&m, 0, sizeof(m));
    m.H = li.H;
    m.rv = li.rv;
    m.rv_src = li.rv_src;
    for (int h = 0; h <= li.H; ++h) {
        m.koff[h] = li.koff[h];
        m.soff[h] = li.soff[h];
    }
    for (int h = 0; h < li.H; ++h) m.srank[h] = li.srank[h];
    return m;
}

// Rows [B][n][C_src] of the key latent (zk_rows) and value latent (zv_rows) to or from cache
// tokens t0 .. t0 + n - 1 of a layer whose ranks were rounded up (either pointer may be NULL).
starkv_status copy_padded(const LayerInfo& li, const starkv_cache* cache, const void* zk_rows,
                          const void* zv_rows, int to_cache, int64_t t0, int64_t n,
                          hipStream_t st, const int32_t* positions = nullptr) {
    for (int which = 0; which < 2; ++which) {
        const void* rows = which ? zv_rows : zk_rows;
        if (!rows) continue;
        PaddedRowsParams p;
        p.rows = rows;
        p.cache = which ? cache->zv : cache->zk;
        p.B = cache->batch;
        p.nblk_cap = static_cast<int>(cache->capacity / kTile);
        p.which = which;
        p.C = which ? li.rv : li.Rk;
        p.C_src = which ? li.rv_src : li.Rk_src;
        p.to_cache = to_cache;
        p.t0 = t0;
        p.n = n;
        p.positions = positions;
        p.pages = pages_of(cache);
        p.map = pad_map(li);
        const starkv_status s = dev(launch_padded_rows(p, elem_bytes(li.cache_dt), st));
        if (s != STARKV_OK) return s;
    }
    return STARKV_OK;
}

// ---- rows x output-major weights (token down-projection, output projection) ----
constexpr int kLinearTargetWorkgroups = 512;   // two 4-wave workgroups per CU
constexpr int kLinearMaxRows = 1024;           // rows per launch (32 row tiles)

// Splits of Kd: about two workgroups per CU, every wave of a workgroup with at least one 64-wide
// K tile.
int linear_splits(int64_t M, int N, int Kd, int elem) {
    const int rows = linear_rows_per_workgroup(elem);
    const int64_t tiles = ((N + rows - 1) / rows) * ((M + 31) / 32);
    const int64_t s = (kLinearTargetWorkgroups + tiles - 1) / tiles;
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, std::max(1, Kd / 64 / 4))));
}

// Partial-sum bytes of the largest launch over up to `rows` rows (launches never exceed
// kLinearMaxRows rows; within a 32-row tile count the split count is fixed).
size_t linear_workspace_bound(int64_t rows, int N, int Kd, int elem) {
    const int64_t mmax = std::min<int64_t>(rows, kLinearMaxRows);
    size_t best = 0;
    for (int64_t tm = 1; tm <= (mmax + 31) / 32; ++tm) {
        const int64_t m = std::min<int64_t>(32 * tm, mmax);
        best = std::max(best, static_cast<size_t>(linear_splits(m, N, Kd, elem)) * m * N * sizeof(float));
    }
    return align_up(best);
}

struct LinearRun {
    const float* x = nullptr;
    int64_t x_tokens = 1;          // rows of x per sequence
    const void* w0 = nullptr;      // output rows [0, N0)
    const void* w1 = nullptr;      // output rows [N0, N)
    int N0 = 0, N = 0, Kd = 0;
    int elem = kF16;               // weight type
    float* part = nullptr;         // workspace
    int kind = 0;                  // store (see LinearStoreParams)
    int store_elem = kF32;
    void* dst0 = nullptr;
    void* dst1 = nullptr;
    int64_t pos = 0, cap = 0;
    bool padded = false;           // kind 1: stored ranks rounded up (see PadMap)
    PadMap map{};
    BlockMap pages;                // kinds 1 and 2: the cache's block table
};

// Rows (b, t) for every sequence b < B and tokens t0 <= t < t0 + tl, at most kLinearMaxRows rows
// per launch pair.
starkv_status run_linear(const LinearRun& r, int B, int64_t t0, int64_t tl, hipStream_t st) {
    const int64_t tchunk = std::min<int64_t>(tl, kLinearMaxRows);
    for (int64_t tc = t0; tc < t0 + tl; tc += tchunk) {
        const int tn = static_cast<int>(std::min<int64_t>(tchunk, t0 + tl - tc));
        const int bchunk = std::max(1, kLinearMaxRows / tn);
        for (int b0 = 0; b0 < B; b0 += bchunk) {
            const int nb = std::min(bchunk, B - b0);
            LinearParams p;
            p.x = r.x;
            p.w0 = r.w0;
            p.w1 = r.w1;
            p.part = r.part;
            p.M = nb * tn;
            p.N = r.N;
            p.N0 = r.N0;
            p.Kd = r.Kd;
            p.S = linear_splits(p.M, r.N, r.Kd, r.elem);
            p.b0 = b0;
            p.t0 = static_cast<int>(tc);
            p.tl = tn;
            p.x_tokens = static_cast<int>(r.x_tokens);
            starkv_status s = dev(launch_linear(p, r.elem, st));
            if (s != STARKV_OK) return s;
            LinearStoreParams q;
            q.part = r.part;
            q.dst0 = r.dst0;
            q.dst1 = r.dst1;
            q.M = p.M;
            q.N = p.N;
            q.N0 = p.N0;
            q.S = p.S;
            q.b0 = p.b0;
            q.t0 = p.t0;
            q.tl = p.tl;
            q.x_tokens = p.x_tokens;
            q.kind = r.kind;
            q.pos = r.pos;
            q.cap = r.cap;
            q.padded = r.padded ? 1 : 0;
            q.map = r.map;
            q.pages = r.pages;
            if ((s = dev(launch_linear_store(q, r.store_elem, st))) != STARKV_OK) return s;
        }
    }
    return STARKV_OK;
}

}  // namespace

extern "C" {

int32_t starkv_version(void) { return 100; }

const char* starkv_status_string(starkv_status s) {
    switch (s) {
    case STARKV_OK: return "ok";
    case STARKV_ERR_NULL: return "a required pointer is NULL";
    case STARKV_ERR_SHAPE: return "a size is out of range or inconsistent";
    case STARKV_ERR_RANK_ALIGN: return "a rank is not a multiple of 16 or exceeds its bound";
    case STARKV_ERR_DTYPE: return "unknown dtype or unsupported cache/factor dtype combination";
    case STARKV_ERR_MISALIGNED: return "a bulk pointer is not 16-byte aligned";
    case STARKV_ERR_CAPACITY: return "capacity not a multiple of 64, or a range beyond capacity";
    case STARKV_ERR_WORKSPACE: return "workspace missing or too small";
    case STARKV_ERR_UNSUPPORTED: return "request outside what the kernels implement";
    case STARKV_ERR_DEVICE: return "a HIP call or kernel launch failed";
    }
    return "unknown status";
}

starkv_status starkv_cache_bytes(const starkv_layer* layer, int32_t batch, int32_t capacity,
                                 size_t out_bytes[6]) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if (!out_bytes) return STARKV_ERR_NULL;
    if (batch < 0 || capacity < 0) return STARKV_ERR_SHAPE;
    if (capacity == 0 || capacity % kTile) return STARKV_ERR_CAPACITY;
    for (int i = 0; i < 6; ++i) out_bytes[i] = 0;
    const size_t Bc = static_cast<size_t>(batch) * capacity;
    if (li.dense) {
        out_bytes[0] = out_bytes[1] = Bc * li.H * li.D * elem_bytes(li.cache_dt);
        return STARKV_OK;
    }
    if (!li.q43) {
        out_bytes[0] = Bc * li.Rk * elem_bytes(li.cache_dt);
        out_bytes[1] = Bc * li.rv * elem_bytes(li.cache_dt);
        return STARKV_OK;
    }
    Q43Layout K, V;
    q43_layouts(li, &K, &V);
    const size_t nb = static_cast<size_t>(batch) * (capacity / kTile);
    out_bytes[0] = nb * K.block_bytes + kQ43CodePad;
    out_bytes[1] = nb * V.block_bytes + kQ43CodePad;
    out_bytes[2] = nb * li.Rk * 4;
    out_bytes[3] = nb * li.rv * 4;
    out_bytes[4] = static_cast<size_t>(batch) * kTile * li.Rk * 2;
    out_bytes[5] = static_cast<size_t>(batch) * kTile * li.rv * 2;
    return STARKV_OK;
}

size_t starkv_decode_workspace_bytes(const starkv_layer* layer, int32_t batch, int64_t seq_len,
                                     int32_t num_splits) {
    LayerInfo li;
    if (check_layer(layer, &li) != STARKV_OK || batch < 0 || seq_len < 1 || num_splits < 0)
        return 0;
    if (seq_len > max_decode_len(li, 1)) return 0;
    return workspace_layout(li, batch, seq_len, num_splits).total;
}

starkv_status starkv_append_latents(const starkv_layer* layer, const starkv_cache* cache,
                                    int64_t pos, int64_t n_new, const void* zk_new,
                                    const void* zv_new, void* stream) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if ((s = check_cache(cache, li)) != STARKV_OK) return s;
    if (pos < 0 || n_new < 0) return STARKV_ERR_SHAPE;
    if (pos + n_new > cache->capacity) return STARKV_ERR_CAPACITY;
    if (n_new == 0 || cache->batch == 0) return STARKV_OK;
    if (!zk_new || !zv_new) return STARKV_ERR_NULL;
    if (!aligned16(zk_new) || !aligned16(zv_new)) return STARKV_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int B = cache->batch;
    const int es = elem_bytes(li.cache_dt);
    if (li.q43) {
        // complete the groups this append finishes (quantise), then keep the rows of the
        // unfinished group in the tail
        Q43Layout K, V;
        q43_layouts(li, &K, &V);
        const int g_first = static_cast<int>(pos / kTile);
        const int ngroups = static_cast<int>((pos + n_new) / kTile) - g_first;
        for (int which = 0; which < 2; ++which) {
            Q43QuantParams q;
            q.pages = pages_of(cache);
            q.L = which ? V : K;
            q.src = which ? zv_new : zk_new;
            q.tail = which ? cache->zv_tail : cache->zk_tail;
            q.codes = which ? cache->zv : cache->zk;
            q.meta = which ? cache->zv_meta : cache->zk_meta;
            q.B = B;
            q.nblk_cap = cache->capacity / kTile;
            q.g_first = g_first;
            q.pos = pos;
            q.n = n_new;
            if ((s = dev(launch_q43_quantize(q, ngroups, st))) != STARKV_OK) return s;
        }
        const int64_t t_begin = std::max<int64_t>(pos, (pos + n_new) / kTile * kTile);
        const int64_t t_end = pos + n_new;
        if (t_end > t_begin) {
            for (int which = 0; which < 2; ++which) {
                const long long row = static_cast<long long>(which ? li.rv : li.Rk) * 2;
                RowCopyParams p;
                p.src = static_cast<const char*>(which ? zv_new : zk_new);
                p.dst = static_cast<char*>(which ? cache->zv_tail : cache->zk_tail);
                p.src_seq_stride = n_new * row;
                p.dst_seq_stride = kTile * row;
                p.src_off = (t_begin - pos) * row;
                p.dst_off = (t_begin % kTile) * row;
                p.bytes = (t_end - t_begin) * row;
                if ((s = dev(launch_copy_rows(p, B, st))) != STARKV_OK) return s;
            }
        }
        return STARKV_OK;
    }
    if (li.dense && cache->block_table) return dense_paged(li, cache, zk_new, zv_new, 1, pos, n_new, st);
    if (li.dense) {
        const long long cap = cache->capacity;
        const long long row = static_cast<long long>(li.H) * li.D * es;
        for (int which = 0; which < 2; ++which) {
            RowCopyParams p;
            p.src = static_cast<const char*>(which ? zv_new : zk_new);
            p.dst = static_cast<char*>(which ? cache->zv : cache->zk);
            p.src_seq_stride = n_new * row;
            p.dst_seq_stride = cap * row;
            p.src_off = 0;
            p.dst_off = pos * row;
            p.bytes = n_new * row;
            if ((s = dev(launch_copy_rows(p, B, st))) != STARKV_OK) return s;
        }
        return STARKV_OK;
    }
    if (li.padded) return copy_padded(li, cache, zk_new, zv_new, 1, pos, n_new, st);
    if (n_new <= kSmallAppend) {
        AppendSmallParams a;
        a.pages = pages_of(cache);
        a.zk_src = zk_new;
        a.zv_src = zv_new;
        a.zk = cache->zk;
        a.zv = cache->zv;
        a.B = B;
        a.Rk = li.Rk;
        a.rv = li.rv;
        a.nblk_cap = cache->capacity / kTile;
        a.pos = pos;
        a.n = n_new;
        return dev(launch_append_small(a, es, st));
    }
    for (int which = 0; which < 2; ++which) {
        BlockXposeParams x;
        x.pages = pages_of(cache);
        x.src = which ? zv_new : zk_new;
        x.dst = which ? cache->zv : cache->zk;
        x.B = B;
        x.C = which ? li.rv : li.Rk;
        x.nblk_cap = cache->capacity / kTile;
        x.t_begin = pos;
        x.t_end = pos + n_new;
        x.row0 = pos;
        x.rows_per_seq = n_new;
        x.blk_first = static_cast<int>(pos / kTile);
        x.to_blocks = 1;
        x.layout = which;
        if ((s = dev(launch_block_transpose(x, es, st))) != STARKV_OK) return s;
    }
    return STARKV_OK;
}

starkv_status starkv_append_latents_ragged(const starkv_layer* layer, const starkv_cache* cache,
                                           const int32_t* positions, const void* zk_new,
                                           const void* zv_new, void* stream) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if ((s = check_cache(cache, li)) != STARKV_OK) return s;
    if (cache->batch == 0) return STARKV_OK;
    if (!positions || !zk_new || !zv_new) return STARKV_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(positions) & 3) || !aligned16(zk_new) || !aligned16(zv_new))
        return STARKV_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int B = cache->batch;
    const int es = elem_bytes(li.cache_dt);
    if (li.dense && cache->block_table)
        return dense_paged(li, cache, zk_new, zv_new, 1, 0, 1, st, positions);
    if (li.q43 || li.dense) {
        // one row per sequence: dense rows at their position, mixed-cache rows into the tail at
        // position % 64 (then the groups that these tokens complete are quantised)
        for (int which = 0; which < 2; ++which) {
            const long long row = static_cast<long long>(li.dense ? li.H * li.D : which ? li.rv : li.Rk) *
                                  (li.dense ? es : 2);
            RowCopyParams p;
            p.src = static_cast<const char*>(which ? zv_new : zk_new);
            p.dst = static_cast<char*>(li.dense ? (which ? cache->zv : cache->zk)
                                                : (which ? cache->zv_tail : cache->zk_tail));
            p.src_seq_stride = row;
            p.dst_seq_stride = (li.dense ? cache->capacity : kTile) * row;
            p.src_off = 0;
            p.dst_off = 0;
            p.bytes = row;
            p.positions = positions;
            p.pos_mod = li.dense ? 0 : kTile;
            p.pos_limit = cache->capacity;
            if ((s = dev(launch_copy_rows(p, B, st))) != STARKV_OK) return s;
        }
        if (li.dense) return STARKV_OK;
        Q43Layout K, V;
        q43_layouts(li, &K, &V);
        for (int which = 0; which < 2; ++which) {
            Q43QuantParams q;
            q.pages = pages_of(cache);
            q.L = which ? V : K;
            q.src = which ? cache->zv_tail : cache->zk_tail;
            q.tail = q.src;
            q.codes = which ? cache->zv : cache->zk;
            q.meta = which ? cache->zv_meta : cache->zk_meta;
            q.B = B;
            q.nblk_cap = static_cast<int>(cache->capacity / kTile);
            q.g_first = 0;
            q.pos = 0;
            q.n = 0;
            q.positions = positions;
            if ((s = dev(launch_q43_quantize(q, 1, st))) != STARKV_OK) return s;
        }
        return STARKV_OK;
    }
    if (li.padded) return copy_padded(li, cache, zk_new, zv_new, 1, 0, 1, st, positions);
    AppendSmallParams a;
    a.pages = pages_of(cache);
    a.zk_src = zk_new;
    a.zv_src = zv_new;
    a.zk = cache->zk;
    a.zv = cache->zv;
    a.B = B;
    a.Rk = li.Rk;
    a.rv = li.rv;
    a.nblk_cap = static_cast<int>(cache->capacity / kTile);
    a.pos = 0;
    a.n = 1;
    a.positions = positions;
    return dev(launch_append_small(a, es, st));
}

// rows: query rows (q, out and the workspace are per row), -1 for one per cache sequence.
// seq_map: NULL (row b reads cache sequence b) or a device array of the cache sequence each row
// reads. seq_lens: NULL (every row attends to seq_len tokens) or a device array of per-row
// lengths, each clamped to [0, seq_len] in the kernels; seq_len then plans the splits.
static starkv_status decode_impl(const starkv_layer* layer, const starkv_cache* cache,
                                 int64_t seq_len, const int32_t* seq_lens, const float* q,
                                 const void* bk, const void* bv, float* out, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes, void* stream, void* ev0,
                                 void* evm, void* ev1, int rows = -1,
                                 const int32_t* seq_map = nullptr, int nq = 1) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if ((s = check_cache(cache, li)) != STARKV_OK) return s;
    if (seq_len < 1 || num_splits < 0) return STARKV_ERR_SHAPE;
    if (seq_len > cache->capacity) return STARKV_ERR_CAPACITY;
    if (seq_len > max_decode_len(li, nq)) return STARKV_ERR_UNSUPPORTED;
    const int B = rows < 0 ? cache->batch : rows;
    if (B == 0) return STARKV_OK;
    if (cache->batch == 0) return STARKV_ERR_SHAPE;          // query rows but no cache sequence
    if (!q || !out) return STARKV_ERR_NULL;
    if (!li.dense && (!bk || !bv)) return STARKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return STARKV_ERR_MISALIGNED;
    if (!li.dense && (!aligned16(bk) || !aligned16(bv))) return STARKV_ERR_MISALIGNED;
    const WorkspaceLayout w = workspace_layout(li, B, seq_len, num_splits, nq);
    if (!workspace || workspace_bytes < w.total) return STARKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return STARKV_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    if (li.dense) {
        const int active = (w.nblk + w.tps - 1) / w.tps;
        DenseDecodeParams p;
        p.pages = pages_of(cache);
        p.k = cache->zk;
        p.v = cache->zv;
        p.q = q;
        p.ws_ml = reinterpret_cast<float*>(ws + w.ml);
        p.ws_acc = reinterpret_cast<float*>(ws + w.acc);
        p.B = B;
        p.H = li.H;
        p.D = li.D;
        p.cap = cache->capacity;
        p.seq_len = static_cast<int>(seq_len);
        p.seq_lens = seq_lens;
        p.seq_map = seq_map;
        p.cache_batch = cache->batch;
        p.S = w.S;
        p.tiles_per_split = w.tps;
        p.q_scale = q_scale_of(layer, li.D);
        fill_rope(layer->rope_base, li.D, p.rope_rev);
        if (ev0 && (s = dev(hipEventRecord(static_cast<hipEvent_t>(ev0), st))) != STARKV_OK) return s;
        if ((s = dev(launch_dense_split(p, elem_kind(li.cache_dt), st))) != STARKV_OK) return s;
        if (evm && (s = dev(hipEventRecord(static_cast<hipEvent_t>(evm), st))) != STARKV_OK) return s;
        if (ev1 && (s = dev(hipEventRecord(static_cast<hipEvent_t>(ev1), st))) != STARKV_OK) return s;
        MergeParams m;
        m.ws_ml = p.ws_ml;
        m.ws_acc = p.ws_acc;
        m.ws_a = out;
        m.B = B;
        m.H = li.H;
        m.S = w.S;
        m.W = li.D;
        m.active_splits = active;
        return dev(launch_merge(m, st));
    }

    const int ek = elem_kind(li.cache_dt);
    ScoreParams sp;
    std::memset(&sp, 0, sizeof(sp));
    sp.pages = pages_of(cache);
    sp.zk = cache->zk;
    sp.bk = bk;
    sp.q = q;
    sp.P = ws + w.P;
    sp.stats = reinterpret_cast<float*>(ws + w.stats);
    sp.B = B;
    sp.H = li.H;
    sp.D = li.D;
    sp.Rk = li.Rk;
    sp.nblk_cap = cache->capacity / kTile;
    sp.seq_len = static_cast<int>(seq_len);
    sp.seq_lens = seq_lens;
    sp.seq_map = seq_map;
    sp.cache_batch = cache->batch;
    sp.nblk = w.nblk;
    sp.Tp = w.nblk * kTile;
    sp.blocks_per_wg = w.sp.bpw;
    sp.q_scale = q_scale_of(layer, li.D);
    for (int h = 0; h < li.H; ++h) sp.order[h] = w.sp.order[h];
    for (int g = 0; g <= w.sp.G; ++g) sp.gstart[g] = w.sp.gstart[g];
    for (int h = 0; h <= li.H; ++h) sp.koff[h] = li.koff[h];
    for (int h = 0; h < li.H; ++h) sp.rank[h] = li.rank[h];
    for (int h = 0; h <= li.H; ++h) sp.soff[h] = li.soff[h];
    for (int h = 0; h < li.H; ++h) sp.srank[h] = li.srank[h];
    fill_rope(layer->rope_base, li.D, sp.rope_rev);
    Q43Layout qk, qv;
    if (li.q43) {
        q43_layouts(li, &qk, &qv);
        sp.zk_meta = cache->zk_meta;
        sp.zk_tail = cache->zk_tail;
        sp.ql = qk;
    }
    const int stream_kind = li.q43 ? -1 : ek;     // -1: mixed 4/3-bit codes, dequantised in-kernel
    if (li.q43 && seq_map) {
        // rows mapped to one cache sequence may stop short of its fill: which of its groups are
        // quantised follows from the longest of them
        RowFillParams rf;
        rf.seq_map = seq_map;
        rf.seq_lens = seq_lens;
        rf.row_fill = reinterpret_cast<int32_t*>(ws + w.fill);
        rf.rows = B;
        rf.cache_batch = cache->batch;
        rf.max_len = static_cast<int>(seq_len);
        if ((s = dev(launch_row_fill(rf, st))) != STARKV_OK) return s;
        sp.row_fill = rf.row_fill;
    }
    if (ev0 && (s = dev(hipEventRecord(static_cast<hipEvent_t>(ev0), st))) != STARKV_OK) return s;
    if ((s = dev(launch_latent_scores(sp, stream_kind, w.sp.G, w.sp.splits, w.sp.maxks, nq, st))) != STARKV_OK)
        return s;
    if (evm && (s = dev(hipEventRecord(static_cast<hipEvent_t>(evm), st))) != STARKV_OK) return s;
    ValueParams vp;
    vp.pages = pages_of(cache);
    vp.zv = cache->zv;
    vp.P = sp.P;
    vp.stats = sp.stats;
    vp.ws_ml = reinterpret_cast<float*>(ws + w.ml);
    vp.ws_acc = reinterpret_cast<float*>(ws + w.acc);
    vp.B = B;
    vp.H = li.H;
    vp.rv = li.rv;
    vp.nblk_cap = sp.nblk_cap;
    vp.seq_len = sp.seq_len;
    vp.seq_lens = seq_lens;
    vp.seq_map = seq_map;
    vp.cache_batch = cache->batch;
    vp.nblk = w.nblk;
    vp.Tp = sp.Tp;
    vp.S = w.vp.splits;
    vp.blocks_per_split = w.vp.bps;
    vp.zv_meta = cache->zv_meta;
    vp.zv_tail = cache->zv_tail;
    vp.row_fill = sp.row_fill;
    vp.block_bytes = li.q43 ? qv.block_bytes : 0;
    vp.n_hi = li.q43 ? qv.n_hi : 0;
    if ((s = dev(launch_latent_values(vp, stream_kind, w.vp.chunks, w.vp.ntw, nq, st))) != STARKV_OK) return s;
    if (ev1 && (s = dev(hipEventRecord(static_cast<hipEvent_t>(ev1), st))) != STARKV_OK) return s;
    // the split merge happens inside the projection kernel, while it loads its inputs
    ProjectParams pr;
    pr.ws_ml = vp.ws_ml;
    pr.ws_acc = vp.ws_acc;
    pr.S = w.vp.splits;
    pr.bv = bv;
    pr.out = out;
    pr.B = B;
    pr.H = li.H;
    pr.D = li.D;
    pr.rv = li.rv;
    pr.rv_src = li.rv_src;
    return dev(launch_project(pr, ek, st));
}

starkv_status starkv_decode_attn(const starkv_layer* layer, const starkv_cache* cache,
                                 int64_t seq_len, const float* q, const void* bk, const void* bv,
                                 float* out, int32_t num_splits, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return decode_impl(layer, cache, seq_len, nullptr, q, bk, bv, out, num_splits, workspace,
                       workspace_bytes, stream, nullptr, nullptr, nullptr);
}

starkv_status starkv_decode_attn_ragged(const starkv_layer* layer, const starkv_cache* cache,
                                        int64_t max_seq_len, const int32_t* seq_lens,
                                        const float* q, const void* bk, const void* bv,
                                        float* out, int32_t num_splits, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    if (cache && cache->batch > 0) {
        if (!seq_lens) return STARKV_ERR_NULL;
        if (reinterpret_cast<uintptr_t>(seq_lens) & 3) return STARKV_ERR_MISALIGNED;
    }
    return decode_impl(layer, cache, max_seq_len, seq_lens, q, bk, bv, out, num_splits,
                       workspace, workspace_bytes, stream, nullptr, nullptr, nullptr);
}

starkv_status starkv_decode_attn_queries(const starkv_layer* layer, const starkv_cache* cache,
                                         int32_t num_queries, const int32_t* query_seq,
                                         const int32_t* query_len, int64_t max_len,
                                         const float* q, const void* bk, const void* bv,
                                         float* out, int32_t num_splits, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    if (num_queries < 0) return STARKV_ERR_SHAPE;
    if (num_queries > 0) {
        if (!query_seq || !query_len) return STARKV_ERR_NULL;
        if ((reinterpret_cast<uintptr_t>(query_seq) & 3) || (reinterpret_cast<uintptr_t>(query_len) & 3))
            return STARKV_ERR_MISALIGNED;
    }
    return decode_impl(layer, cache, max_len, query_len, q, bk, bv, out, num_splits, workspace,
                       workspace_bytes, stream, nullptr, nullptr, nullptr, num_queries, query_seq);
}

// ------------------------------------------------------------------------------------------------
// Prefill: a chunk of causal queries per sequence.
// ------------------------------------------------------------------------------------------------
static starkv_status prefill_check(const starkv_layer* layer, int32_t batch, int64_t pos0,
                                   int32_t chunk, LayerInfo* li) {
    starkv_status s = check_layer(layer, li);
    if (s != STARKV_OK) return s;
    if (batch < 0 || pos0 < 0 || chunk < 1) return STARKV_ERR_SHAPE;
    if (li->dense || li->cache_dt == STARKV_F32) return STARKV_ERR_UNSUPPORTED;
    if (pos0 + chunk > max_decode_len(*li, 1)) return STARKV_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(batch) * chunk > (int64_t{1} << 30)) return STARKV_ERR_UNSUPPORTED;
    return STARKV_OK;
}

size_t starkv_prefill_workspace_bytes(const starkv_layer* layer, int32_t batch, int64_t pos0,
                                      int32_t chunk) {
    LayerInfo li;
    if (prefill_check(layer, batch, pos0, chunk, &li) != STARKV_OK) return 0;
    return prefill_layout(li, batch, pos0, chunk).total;
}

starkv_status starkv_prefill_attn(const starkv_layer* layer, const starkv_cache* cache, int64_t pos0,
                                  int32_t chunk, const int32_t* chunk_lens, const float* q,
                                  const void* bk, const void* bv, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    LayerInfo li;
    if (!cache) return STARKV_ERR_NULL;
    starkv_status s = prefill_check(layer, cache->batch, pos0, chunk, &li);
    if (s != STARKV_OK) return s;
    if ((s = check_cache(cache, li)) != STARKV_OK) return s;
    if (pos0 + chunk > cache->capacity) return STARKV_ERR_CAPACITY;
    const int B = cache->batch;
    if (B == 0) return STARKV_OK;
    if (!q || !out || !bk || !bv) return STARKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(bk) || !aligned16(bv)) return STARKV_ERR_MISALIGNED;
    if (chunk_lens && (reinterpret_cast<uintptr_t>(chunk_lens) & 3)) return STARKV_ERR_MISALIGNED;
    const PrefillLayout pl = prefill_layout(li, B, pos0, chunk);
    if (!workspace || workspace_bytes < pl.total) return STARKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return STARKV_ERR_MISALIGNED;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    const int ek = elem_kind(li.cache_dt);

    // 1. latent rows of tokens [0, pos0 + chunk_len(b)) of each sequence, in MFMA fragment order
    //    (32-token tiles of 8-channel runs; mixed 4/3-bit groups dequantised to binary16 on the
    //    way); 16-bit key latents need no copy (the cache's key layout is already fragment order)
    for (int which = li.q43 ? 0 : 1; which < 2; ++which) {   // 16-bit keys: read in place
        void* rows = ws + (which ? pl.zv_rows : pl.zk_rows);
        if (li.q43) {
            Q43Layout K, V;
            q43_layouts(li, &K, &V);
            Q43ReadParams r;
            r.pages = pages_of(cache);
            r.L = which ? V : K;
            r.codes = which ? cache->zv : cache->zk;
            r.meta = which ? cache->zv_meta : cache->zk_meta;
            r.tail = which ? cache->zv_tail : cache->zk_tail;
            r.out = rows;
            r.B = B;
            r.nblk_cap = cache->capacity / kTile;
            r.t0 = 0;
            r.t1 = pl.Tk;
            r.full_tokens = pl.Tk / kTile * kTile;
            r.chunk_lens = chunk_lens;
            r.pos0 = pos0;
            r.chunk = chunk;
            if ((s = dev(launch_q43_readback(r, st, true))) != STARKV_OK) return s;
        } else {
            BlockXposeParams x;
            x.pages = pages_of(cache);
            x.src = which ? cache->zv : cache->zk;
            x.dst = rows;
            x.B = B;
            x.C = which ? li.rv : li.Rk;
            x.nblk_cap = cache->capacity / kTile;
            x.t_begin = 0;
            x.t_end = pl.Tk;
            x.row0 = 0;
            x.rows_per_seq = static_cast<long long>(pl.ntiles) * 32;
            x.blk_first = 0;
            x.to_blocks = 0;
            x.layout = which;
            x.chunk_lens = chunk_lens;
            x.pos0 = pos0;
            x.chunk = chunk;
            if ((s = dev(launch_block_transpose(x, elem_bytes(li.cache_dt), st, true))) != STARKV_OK) return s;
        }
    }

    // 2. keys (rotated) and values (per head) of every 32-token tile, once
    PrefillKVParams kp;
    std::memset(&kp, 0, sizeof(kp));
    kp.zk_rows = ws + pl.zk_rows;
    kp.zv_rows = ws + pl.zv_rows;
    if (!li.q43) {
        kp.zk_cache = cache->zk;
        kp.pages = pages_of(cache);
        kp.nblk_cap = cache->capacity / kTile;
    }
    kp.bk = bk;
    kp.bv = bv;
    kp.bvf = ws + pl.bvf;
    kp.kv = ws + pl.kv;
    kp.exps = reinterpret_cast<int32_t*>(ws + pl.exps);
    kp.chunk_lens = chunk_lens;
    kp.B = B;
    kp.H = li.H;
    kp.D = li.D;
    kp.Rk = li.Rk;
    kp.rv = li.rv;
    kp.rv_src = li.rv_src;
    kp.Tr = pl.ntiles * 32;
    kp.ntiles = pl.ntiles;
    kp.chunk = chunk;
    kp.pos0 = static_cast<int>(pos0);
    for (int h = 0; h <= li.H; ++h) kp.koff[h] = li.koff[h];
    for (int h = 0; h < li.H; ++h) kp.rank[h] = li.rank[h];
    for (int h = 0; h <= li.H; ++h) kp.soff[h] = li.soff[h];
    for (int h = 0; h < li.H; ++h) kp.srank[h] = li.srank[h];
    fill_rope(layer->rope_base, li.D, kp.rope_rev);
    // mixed 4/3-bit rows are binary16, with binary16 factors
    if ((s = dev(launch_prefill_kv(kp, li.q43 ? kF16 : ek, st))) != STARKV_OK) return s;

    // 3. causal attention, 32 queries per wave, output written once
    PrefillFlashParams fp;
    fp.q = q;
    fp.out = out;
    fp.kv = kp.kv;
    fp.exps = kp.exps;
    fp.chunk_lens = chunk_lens;
    fp.B = B;
    fp.H = li.H;
    fp.D = li.D;
    fp.chunk = chunk;
    fp.pos0 = static_cast<int>(pos0);
    fp.ntiles = pl.ntiles;
    fp.q_scale = q_scale_of(layer, li.D);
    return dev(launch_prefill_attend(fp, st));
}

size_t starkv_decode_multi_workspace_bytes(const starkv_layer* layer, int32_t batch, int32_t nq,
                                           int64_t max_len, int32_t num_splits) {
    LayerInfo li;
    if (check_layer(layer, &li) != STARKV_OK || li.dense || batch < 0 || max_len < 1 || num_splits < 0)
        return 0;
    if (nq != 1 && nq != 2 && nq != 4) return 0;
    if (max_len > max_decode_len(li, nq)) return 0;
    return workspace_layout(li, batch * nq, max_len, num_splits, nq).total;
}

starkv_status starkv_decode_attn_multi(const starkv_layer* layer, const starkv_cache* cache,
                                       int32_t nq, int64_t max_len, const int32_t* q_lens,
                                       const float* q, const void* bk, const void* bv, float* out,
                                       int32_t num_splits, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if (nq < 1) return STARKV_ERR_SHAPE;
    if (li.dense || (nq != 1 && nq != 2 && nq != 4) || (nq > 1 && li.cache_dt == STARKV_F32))
        return STARKV_ERR_UNSUPPORTED;
    if (q_lens && (reinterpret_cast<uintptr_t>(q_lens) & 3)) return STARKV_ERR_MISALIGNED;
    if (!cache) return STARKV_ERR_NULL;
    return decode_impl(layer, cache, max_len, q_lens, q, bk, bv, out, num_splits, workspace,
                       workspace_bytes, stream, nullptr, nullptr, nullptr, cache->batch * nq,
                       nullptr, nq);
}

starkv_status starkv_decode_attn_timed(const starkv_layer* layer, const starkv_cache* cache,
                                       int64_t seq_len, const float* q, const void* bk,
                                       const void* bv, float* out, int32_t num_splits,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       void* event_begin, void* event_mid, void* event_end) {
    return decode_impl(layer, cache, seq_len, nullptr, q, bk, bv, out, num_splits, workspace,
                       workspace_bytes, stream, event_begin, event_mid, event_end);
}

// ------------------------------------------------------------------------------------------------
// Decode without a caller workspace: for callers that cannot allocate device memory (code under
// graph capture, tight serving loops). The workspace is a fixed array in device memory, one per
// GPU, held until the process ends; calls on one GPU share it.
// ------------------------------------------------------------------------------------------------
}  // extern "C"

namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of `scratch` on the current device, looked up once per device. (In host code
// the array's name is only a stand-in for the symbol; its device address comes from the runtime.)
starkv_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
        return STARKV_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return STARKV_ERR_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return STARKV_OK;
}
}  // namespace

extern "C" {

size_t starkv_decode_attn_noalloc_max_bytes(void) { return kScratchBytes; }

starkv_status starkv_decode_attn_noalloc(const starkv_layer* layer, const starkv_cache* cache,
                                         int64_t seq_len, const float* q, const void* bk,
                                         const void* bv, float* out, int32_t num_splits,
                                         void* stream) {
    // a request whose workspace would not fit is refused before anything else is touched;
    // requests sized 0 (invalid, beyond the planner's limits, or an empty batch) get their status
    // from the shared validation without the array
    const int32_t batch = cache ? cache->batch : 0;
    const size_t need = layer ? starkv_decode_workspace_bytes(layer, batch, seq_len, num_splits) : 0;
    if (need > kScratchBytes) return STARKV_ERR_WORKSPACE;
    if (need == 0)
        return decode_impl(layer, cache, seq_len, nullptr, q, bk, bv, out, num_splits, nullptr, 0,
                           stream, nullptr, nullptr, nullptr);
    void* ws = nullptr;
    const starkv_status s = scratch_of_current_device(&ws);
    if (s != STARKV_OK) return s;
    return decode_impl(layer, cache, seq_len, nullptr, q, bk, bv, out, num_splits, ws,
                       kScratchBytes, stream, nullptr, nullptr, nullptr);
}

starkv_status starkv_dequant(const starkv_layer* layer, const starkv_cache* cache,
                             int64_t seq_len, int64_t t0, int64_t t1, void* zk_out, void* zv_out,
                             void* stream) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if ((s = check_cache(cache, li)) != STARKV_OK) return s;
    if (seq_len < 0 || t0 < 0 || t0 > t1) return STARKV_ERR_SHAPE;
    if (seq_len > cache->capacity || t1 > seq_len) return STARKV_ERR_CAPACITY;
    if ((zk_out && !aligned16(zk_out)) || (zv_out && !aligned16(zv_out))) return STARKV_ERR_MISALIGNED;
    if (cache->batch == 0 || t0 == t1) return STARKV_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int B = cache->batch;
    const int es = elem_bytes(li.cache_dt);
    const long long cap = cache->capacity, n = t1 - t0;
    if (li.q43) {
        Q43Layout K, V;
        q43_layouts(li, &K, &V);
        for (int which = 0; which < 2; ++which) {
            void* outp = which ? zv_out : zk_out;
            if (!outp) continue;
            Q43ReadParams r;
            r.pages = pages_of(cache);
            r.L = which ? V : K;
            r.codes = which ? cache->zv : cache->zk;
            r.meta = which ? cache->zv_meta : cache->zk_meta;
            r.tail = which ? cache->zv_tail : cache->zk_tail;
            r.out = outp;
            r.B = B;
            r.nblk_cap = cache->capacity / kTile;
            r.t0 = t0;
            r.t1 = t1;
            r.full_tokens = seq_len / kTile * kTile;
            if ((s = dev(launch_q43_readback(r, st))) != STARKV_OK) return s;
        }
        return STARKV_OK;
    }
    if (li.dense && cache->block_table) return dense_paged(li, cache, zk_out, zv_out, 0, t0, n, st);
    if (li.dense) {
        const long long row = static_cast<long long>(li.H) * li.D * es;
        for (int which = 0; which < 2; ++which) {
            void* outp = which ? zv_out : zk_out;
            if (!outp) continue;
            RowCopyParams p;
            p.src = static_cast<const char*>(which ? cache->zv : cache->zk);
            p.dst = static_cast<char*>(outp);
            p.src_seq_stride = cap * row;
            p.dst_seq_stride = n * row;
            p.src_off = t0 * row;
            p.dst_off = 0;
            p.bytes = n * row;
            if ((s = dev(launch_copy_rows(p, B, st))) != STARKV_OK) return s;
        }
        return STARKV_OK;
    }
    if (li.padded) return copy_padded(li, cache, zk_out, zv_out, 0, t0, n, st);
    for (int which = 0; which < 2; ++which) {
        void* outp = which ? zv_out : zk_out;
        if (!outp) continue;
        BlockXposeParams x;
        x.pages = pages_of(cache);
        x.src = which ? cache->zv : cache->zk;
        x.dst = outp;
        x.B = B;
        x.C = which ? li.rv : li.Rk;
        x.nblk_cap = cache->capacity / kTile;
        x.t_begin = t0;
        x.t_end = t1;
        x.row0 = t0;
        x.rows_per_seq = n;
        x.blk_first = static_cast<int>(t0 / kTile);
        x.to_blocks = 0;
        x.layout = which;
        if ((s = dev(launch_block_transpose(x, es, st))) != STARKV_OK) return s;
    }
    return STARKV_OK;
}

starkv_status starkv_hadamard_rotate(const starkv_layer* layer, int32_t which, int32_t kind,
                                     int64_t n, const void* src, void* dst, void* stream) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if (li.dense) return STARKV_ERR_UNSUPPORTED;
    if ((which != 0 && which != 1) || (kind != 0 && kind != 1) || n < 0) return STARKV_ERR_SHAPE;
    if (li.cache_dt != STARKV_F16 && li.cache_dt != STARKV_Q43) return STARKV_ERR_DTYPE;
    if (kind == 1 && n != (which == 0 ? li.D : static_cast<int64_t>(li.H) * li.D))
        return STARKV_ERR_SHAPE;
    if (n == 0) return STARKV_OK;
    if (!src || !dst) return STARKV_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(src) & 1) || (reinterpret_cast<uintptr_t>(dst) & 1))
        return STARKV_ERR_MISALIGNED;
    HadamardParams p;
    std::memset(&p, 0, sizeof(p));
    p.src = static_cast<const uint16_t*>(src);
    p.dst = static_cast<uint16_t*>(dst);
    p.n = n;
    p.kind = kind;
    p.C = which == 0 ? li.Rk_src : li.rv_src;
    // each latent splits into its leading 4-bit channels and the rest; each part of width w is
    // rotated in blocks of b = min(64, largest power of two dividing w)
    auto add = [&](int start, int w) {
        if (w <= 0) return;
        int b = 1;
        while (b < 64 && w % (2 * b) == 0) b *= 2;
        p.seg_start[p.nseg] = start;
        p.seg_width[p.nseg] = w;
        p.seg_block[p.nseg] = b;
        p.seg_inv[p.nseg] = 1.0 / std::sqrt(static_cast<double>(b));
        ++p.nseg;
    };
    if (which == 0) {
        for (int h = 0; h < li.H; ++h) {
            const int nh = q43_hi_channels(li.srank[h], li.top_fraction);
            add(li.soff[h], nh);
            add(li.soff[h] + nh, li.srank[h] - nh);
        }
    } else {
        const int nh = q43_hi_channels(li.rv_src, li.top_fraction);
        add(0, nh);
        add(nh, li.rv_src - nh);
    }
    return dev(launch_hadamard_rotate(p, static_cast<hipStream_t>(stream)));
}

size_t starkv_output_projection_workspace_bytes(const starkv_layer* layer, int32_t batch,
                                               int32_t hidden) {
    LayerInfo li;
    if (check_layer(layer, &li) != STARKV_OK || batch < 1 || hidden < 1) return 0;
    return linear_workspace_bound(batch, hidden, li.H * li.D,
                                  elem_kind(li.dense ? li.cache_dt : li.factor_dt));
}

starkv_status starkv_output_projection(const starkv_layer* layer, int32_t batch, const float* o,
                                      const void* wo, int32_t hidden, float* y, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if (batch < 0 || hidden < 1) return STARKV_ERR_SHAPE;
    if (batch == 0) return STARKV_OK;
    if (!o || !wo || !y || !workspace) return STARKV_ERR_NULL;
    if (!aligned16(o) || !aligned16(wo) || !aligned16(workspace) ||
        (reinterpret_cast<uintptr_t>(y) & 3))
        return STARKV_ERR_MISALIGNED;
    const int kd = li.H * li.D;
    const int wdt = li.dense ? li.cache_dt : li.factor_dt;    // the layer's weight type
    if (workspace_bytes < linear_workspace_bound(batch, hidden, kd, elem_kind(wdt)))
        return STARKV_ERR_WORKSPACE;
    LinearRun r;
    r.x = o;
    r.x_tokens = 1;
    r.w0 = wo;
    r.w1 = wo;
    r.N0 = hidden;
    r.N = hidden;
    r.Kd = kd;
    r.elem = elem_kind(wdt);
    r.kind = 0;
    r.dst0 = y;
    r.dst1 = y;
    r.part = static_cast<float*>(workspace);
    return run_linear(r, batch, 0, 1, static_cast<hipStream_t>(stream));
}

// Decode attention and the output projection in one call (Algorithm 2 steps 4-8): the heads'
// outputs stay in the workspace between the two.
static size_t decode_project_layout(const starkv_layer* layer, int32_t batch, int64_t seq_len,
                                    int32_t num_splits, int32_t hidden, size_t* o_off,
                                    size_t* part_off) {
    LayerInfo li;
    if (check_layer(layer, &li) != STARKV_OK || batch < 1 || hidden < 1) return 0;
    const size_t dec = starkv_decode_workspace_bytes(layer, batch, seq_len, num_splits);
    if (dec == 0) return 0;
    const size_t o_bytes = align_up(static_cast<size_t>(batch) * li.H * li.D * sizeof(float));
    const size_t part = starkv_output_projection_workspace_bytes(layer, batch, hidden);
    if (part == 0) return 0;
    *o_off = align_up(dec);
    *part_off = *o_off + o_bytes;
    return *part_off + part;
}

size_t starkv_decode_attn_project_workspace_bytes(const starkv_layer* layer, int32_t batch,
                                                  int64_t seq_len, int32_t num_splits,
                                                  int32_t hidden) {
    size_t o_off = 0, part_off = 0;
    return decode_project_layout(layer, batch, seq_len, num_splits, hidden, &o_off, &part_off);
}

starkv_status starkv_decode_attn_project(const starkv_layer* layer, const starkv_cache* cache,
                                         int64_t seq_len, const float* q, const void* bk,
                                         const void* bv, const void* wo, int32_t hidden, float* y,
                                         int32_t num_splits, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if (!cache) return STARKV_ERR_NULL;
    if (hidden < 1) return STARKV_ERR_SHAPE;
    if (cache->batch == 0) return STARKV_OK;
    if (!wo || !y) return STARKV_ERR_NULL;
    if (!aligned16(wo) || (reinterpret_cast<uintptr_t>(y) & 3)) return STARKV_ERR_MISALIGNED;
    size_t o_off = 0, part_off = 0;
    const size_t need = decode_project_layout(layer, cache->batch, seq_len, num_splits, hidden,
                                              &o_off, &part_off);
    if (need == 0) {
        // an invalid decode request: its own validation names the problem
        return decode_impl(layer, cache, seq_len, nullptr, q, bk, bv, nullptr, num_splits, nullptr, 0,
                           stream, nullptr, nullptr, nullptr);
    }
    if (!workspace || workspace_bytes < need) return STARKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return STARKV_ERR_MISALIGNED;
    char* ws = static_cast<char*>(workspace);
    float* o = reinterpret_cast<float*>(ws + o_off);
    if ((s = decode_impl(layer, cache, seq_len, nullptr, q, bk, bv, o, num_splits, ws, o_off,
                         stream, nullptr, nullptr, nullptr)) != STARKV_OK)
        return s;
    return starkv_output_projection(layer, cache->batch, o, wo, hidden, y, ws + part_off,
                                    need - part_off, stream);
}

size_t starkv_append_tokens_workspace_bytes(const starkv_layer* layer, int32_t batch,
                                            int64_t n_new, int32_t model_dim) {
    LayerInfo li;
    if (check_layer(layer, &li) != STARKV_OK || batch < 1 || n_new < 1 || model_dim < 64) return 0;
    const int n_out = li.dense ? 2 * li.H * li.D : li.Rk_src + li.rv_src;
    const int64_t rows = li.q43 ? static_cast<int64_t>(batch) * std::min<int64_t>(n_new, kTile)
                                : static_cast<int64_t>(batch) * n_new;
    return linear_workspace_bound(rows, n_out, model_dim,
                                  elem_kind(li.dense ? li.cache_dt : li.factor_dt));
}

starkv_status starkv_append_tokens(const starkv_layer* layer, const starkv_cache* cache,
                                   int64_t pos, int64_t n_new, const float* x, int32_t model_dim,
                                   const void* a_k, const void* a_v, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    LayerInfo li;
    starkv_status s = check_layer(layer, &li);
    if (s != STARKV_OK) return s;
    if ((s = check_cache(cache, li)) != STARKV_OK) return s;
    if (pos < 0 || n_new < 0 || model_dim < 1) return STARKV_ERR_SHAPE;
    if (model_dim % 64) return STARKV_ERR_UNSUPPORTED;
    if (pos + n_new > cache->capacity) return STARKV_ERR_CAPACITY;
    if (n_new > INT32_MAX) return STARKV_ERR_UNSUPPORTED;
    if (n_new == 0 || cache->batch == 0) return STARKV_OK;
    if (!x || !a_k || !a_v || !workspace) return STARKV_ERR_NULL;
    if (!aligned16(x) || !aligned16(a_k) || !aligned16(a_v) || !aligned16(workspace))
        return STARKV_ERR_MISALIGNED;
    const int B = cache->batch;
    if (workspace_bytes < starkv_append_tokens_workspace_bytes(layer, B, n_new, model_dim))
        return STARKV_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    LinearRun r;
    r.x = x;
    r.x_tokens = n_new;
    r.w0 = a_k;
    r.w1 = a_v;
    r.N0 = li.dense ? li.H * li.D : li.Rk_src;
    r.N = li.dense ? 2 * li.H * li.D : li.Rk_src + li.rv_src;
    r.padded = li.padded;
    if (li.padded) r.map = pad_map(li);
    r.pages = pages_of(cache);
    r.Kd = model_dim;
    r.elem = elem_kind(li.dense ? li.cache_dt : li.factor_dt);
    r.part = static_cast<float*>(workspace);
    r.pos = pos;
    if (!li.q43) {
        r.kind = li.dense ? 2 : 1;
        r.store_elem = elem_kind(li.cache_dt);
        r.dst0 = cache->zk;
        r.dst1 = cache->zv;
        r.cap = li.dense ? cache->capacity : cache->capacity / kTile;
        return run_linear(r, B, 0, n_new, st);
    }
    // mixed 4/3-bit cache: the binary16 rows go to the tail one 64-token group at a time; a group
    // that this call completes is then quantised from the tail
    r.kind = 3;
    r.dst0 = cache->zk_tail;
    r.dst1 = cache->zv_tail;
    Q43Layout K, V;
    q43_layouts(li, &K, &V);
    for (int64_t t0 = 0; t0 < n_new;) {
        const int64_t g_end = ((pos + t0) / kTile + 1) * kTile;
        const int64_t t1 = std::min(n_new, g_end - pos);
        if ((s = run_linear(r, B, t0, t1 - t0, st)) != STARKV_OK) return s;
        if (pos + t1 == g_end) {
            for (int which = 0; which < 2; ++which) {
                Q43QuantParams q;
                q.pages = pages_of(cache);
                q.L = which ? V : K;
                q.src = which ? cache->zv_tail : cache->zk_tail;   // every row comes from the tail
                q.tail = q.src;
                q.codes = which ? cache->zv : cache->zk;
                q.meta = which ? cache->zv_meta : cache->zk_meta;
                q.B = B;
                q.nblk_cap = cache->capacity / kTile;
                q.g_first = static_cast<int>(g_end / kTile) - 1;
                q.pos = g_end;
                q.n = 0;
                if ((s = dev(launch_q43_quantize(q, 1, st))) != STARKV_OK) return s;
            }
        }
        t0 = t1;
    }
    return STARKV_OK;
}

}  // extern "C"
