// routing.h - top-k selection, weight renormalisation and the routing
// metadata (active experts, their token lists, column units of <= 8 tokens).
//
// Selection follows the layer definition: each token keeps the k experts with
// the largest key s_e + bias_e (equal keys: the lower id first) and weights
// them by s_e / sum of the selected s (page "快是可以生成的，可信只能证明（vLLM
// 重写 Kimi K3 解码路径…）", section "为什么一条请求会慢": 16 of 896 experts are
// active per token; sigmoid scores, the bias on the key only and the
// renormalisation are readings of the layer definition).
//
// The work runs inside the kernel that produces the router scores: every
// router tile ends with an arrival on one agent-scope counter, and the
// workgroup whose arrival completes the router runs the whole routing with
// all of its waves (tokens split by wave), hands the selections over in LDS
// and builds the metadata; no other workgroup waits or polls.  Wave-wide
// reductions and scans use DPP row operations and scalar lane reads, and the
// selection rounds touch no memory.
#pragma once

#include "device_common.h"
#include "step_args.h"

namespace moe {

constexpr int kKeysPerLane = kMaxExperts / kWave;  // 16

// DPP controls (GFX9 encoding).
enum : int {
    kQuadSwap1 = 0xB1,   // quad_perm [1,0,3,2]
    kQuadSwap2 = 0x4E,   // quad_perm [2,3,0,1]
    kRowShr1 = 0x111,
    kRowShr2 = 0x112,
    kRowShr4 = 0x114,
    kRowShr8 = 0x118,
    kRowMirror = 0x140,
    kRowHalfMirror = 0x141,
    kRowBcast15 = 0x142,
    kRowBcast31 = 0x143,
};

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}

__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Wave-wide maximum / minimum of a u32, as a scalar.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp<kQuadSwap1>(v));
    v = max(v, dpp<kQuadSwap2>(v));
    v = max(v, dpp<kRowHalfMirror>(v));
    v = max(v, dpp<kRowMirror>(v));
    return max(max(readlane(v, 0), readlane(v, 16)), max(readlane(v, 32), readlane(v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

// Inclusive prefix sum over the wave (lane order).
__device__ __forceinline__ int wave_incl_scan(int v) {
    uint32_t u = (uint32_t)v;
    u += dpp<kRowShr1>(u);
    u += dpp<kRowShr2>(u);
    u += dpp<kRowShr4>(u);
    u += dpp<kRowShr8>(u);
    u += dpp<kRowBcast15, 0xA>(u);
    u += dpp<kRowBcast31, 0xC>(u);
    return (int)u;
}

// Orders f32 keys as u32 (larger key -> larger u32; 0 never occurs for a
// finite key, so 0 marks "no candidate").
__device__ __forceinline__ uint32_t orderable(float key) {
    const uint32_t u = __float_as_uint(key);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kMaxRouteWaves = 8;

// What the routing reads and writes.
struct RouteArgs {
    int32_t B, k, E;
    const float *score, *key;
    int32_t *idx;
    float *wsel;
    int32_t *user_idx;
    float *user_w;
    int32_t *meta, *act_expert, *act_off, *cu_rec, *pair_slot, *pair_of_slot;
};

__device__ __forceinline__ RouteArgs route_args(const StepArgs &a) {
    RouteArgs r;
    r.B = a.B;
    r.k = a.k;
    r.E = a.E;
    r.score = a.score;
    r.key = a.key;
    r.idx = a.idx;
    r.wsel = a.wsel;
    r.user_idx = a.user_idx;
    r.user_w = a.user_w;
    r.meta = a.meta;
    r.act_expert = a.act_expert;
    r.act_off = a.act_off;
    r.cu_rec = a.cu_rec;
    r.pair_slot = a.pair_slot;
    r.pair_of_slot = a.pair_of_slot;
    return r;
}

// LDS of the routing: the selections of every token (MaxPairs = B k at
// most), the token masks of the experts, per-expert offsets and per-wave scan
// totals, the candidate lists of the threshold selection, and (MaxCols > 1)
// the unit records when they are kept in LDS.
template <int MaxPairs, int MaxCols, int CandRows>
struct RouteLdsT {
    int16_t idx[MaxPairs];
    float w[MaxPairs];
    unsigned long long mask[kMaxExperts];
    int off[kMaxExperts];
    int unit[kMaxExperts];
    int wsum[kMaxRouteWaves][4];
    // Per wave: the candidates of the threshold selection (key, expert,
    // score), then the selection in key order (expert, score).
    uint32_t cand_key[CandRows][kWave];
    int cand_id[CandRows][kWave];
    float cand_s[CandRows][kWave];
    int rec[MaxCols][kRecWords];
    int ncols, n_active;
    // Selection of one token by the whole workgroup: per-wave lane maxima,
    // the threshold, per-wave candidate counts.
    uint32_t wmax[kMaxRouteWaves][kWave];
    uint32_t thr;
    int wcnt[kMaxRouteWaves];
};
// The routing of the dense-in launch (any batch up to kMaxBatch): records go
// to global memory.
typedef RouteLdsT<kMaxBatch * kMaxTopK, 1, 2> RouteLds;
// The routing at the start of the gate/up launch: at most kLatePairs (token,
// expert) pairs, every unit record kept in LDS.
constexpr int kLatePairs = 128;
typedef RouteLdsT<kLatePairs, kLatePairs + kLatePairs / 8, kMaxRouteWaves> LateRouteLds;

// Best remaining experts of one lane, best first: orderable keys (0: none),
// slots (expert = lane + 64 * slot) and scores.
constexpr int kList = 4;
struct LaneList {
    uint32_t k[kList];
    int i[kList];
    float s[kList];
};

// The lane's kList best experts among those that come after (after_k,
// after_i) in selection order: larger key first, equal keys by lower slot
// (= lower expert id).  Branch-free insertion over the lane's slots.
__device__ __forceinline__ void fill_list(LaneList &L, const uint32_t (&ok)[kKeysPerLane],
                                          const float (&sc)[kKeysPerLane], uint32_t after_k,
                                          int after_i) {
#pragma unroll
    for (int j = 0; j < kList; ++j) {
        L.k[j] = 0u;
        L.i[j] = 0;
        L.s[j] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
        const uint32_t v = ok[i];
        const bool elig = v != 0u && (v < after_k || (v == after_k && i > after_i));
        const uint32_t w = elig ? v : 0u;
        bool gt[kList];
#pragma unroll
        for (int j = 0; j < kList; ++j) gt[j] = w > L.k[j];  // strict: a later slot goes after
#pragma unroll
        for (int j = kList - 1; j >= 1; --j) {
            L.k[j] = gt[j - 1] ? L.k[j - 1] : (gt[j] ? w : L.k[j]);
            L.i[j] = gt[j - 1] ? L.i[j - 1] : (gt[j] ? i : L.i[j]);
            L.s[j] = gt[j - 1] ? L.s[j - 1] : (gt[j] ? sc[i] : L.s[j]);
        }
        L.k[0] = gt[0] ? w : L.k[0];
        L.i[0] = gt[0] ? i : L.i[0];
        L.s[0] = gt[0] ? sc[i] : L.s[0];
    }
}

// Number of set bits of m below the calling lane.
__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Selection by threshold, one wave, without the k serial rounds:
//  1. T = the k-th largest of the 64 lane maxima (a radix select over its 32
//     bits, each bit one wave-wide count), so that at least k keys are >= T
//     and every expert of the top k has a key >= T;
//  2. the keys >= T are compacted into LDS in slot-major, lane-minor order,
//     which is ascending expert id;
//  3. each candidate's rank in selection order (larger key first, equal keys
//     by lower id) is its count of candidates that come before it;
//  4. the candidates of rank < k are selected: sel on their lanes (mine and
//     s_mine: expert and score), pos = their place among the selected ids
//     (the selected lanes below, the candidates being in ascending id), and
//     total = the sum of the selected scores in selection order (the scores
//     written to LDS by rank, then added in rank order).
// Returns false, having changed nothing the caller uses, when more than 64
// keys are >= T (the caller then runs the rounds).
__device__ __forceinline__ bool select_by_threshold(const uint32_t (&ok)[kKeysPerLane],
                                                    const float (&sc)[kKeysPerLane], int k,
                                                    uint32_t *cand_key, int *cand_id,
                                                    float *cand_s, int &mine, float &s_mine,
                                                    bool &sel, int &pos, float &total) {
    const int lane = lane_id();
    uint32_t lm = 0u;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) lm = max(lm, ok[i]);
    uint32_t T = 0u;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t t = T | (1u << bit);
        T = __popcll(__ballot(lm >= t)) >= k ? t : T;
    }
    int n = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
        const bool c = ok[i] != 0u && ok[i] >= T;
        const unsigned long long m = __ballot(c);
        const int pos = n + lanes_below(m);
        if (c && pos < kWave) {
            cand_key[pos] = ok[i];
            cand_id[pos] = lane + kWave * i;
            cand_s[pos] = sc[i];
        }
        n += __popcll(m);
    }
    if (n > kWave) return false;
    wave_sync();
    const bool have = lane < n;
    const uint32_t ck = have ? cand_key[lane] : 0u;
    const int cid = have ? cand_id[lane] : 0;
    const float cs = have ? cand_s[lane] : 0.f;
    int rank = 0;
    for (int j = 0; j < n; ++j) {
        const uint32_t kj = readlane(ck, j);
        rank += (kj > ck || (kj == ck && j < lane)) ? 1 : 0;
    }
    // The candidates are in ascending id, so a selection's place among the
    // selected ids is its count of selected lanes below; the scores go to
    // LDS in selection order for the sum.
    sel = have && rank < k;
    pos = lanes_below(__ballot(sel));
    wave_sync();
    if (sel) cand_s[rank] = cs;
    wave_sync();
    total = 0.f;
    for (int r = 0; r < k; ++r) total += cand_s[r];
    mine = cid;
    s_mine = cs;
    wave_sync();
    return true;
}

// Selection by k rounds (any key distribution): lane l keeps a short list of
// its best remaining experts; each round takes the wave-wide largest list
// head (equal keys: the lowest expert id); lane r keeps the id and score of
// round r's winner, and the winning lane drops its head (and rebuilds its list
// after kList drops).
__device__ __forceinline__ void select_by_rounds(const uint32_t (&ok)[kKeysPerLane],
                                                 const float (&sc)[kKeysPerLane], int k,
                                                 int &mine, float &s_mine) {
    const int lane = lane_id();
    LaneList L;
    fill_list(L, ok, sc, 0xFFFFFFFFu, -1);
    int npop = 0;
    for (int r = 0; r < k; ++r) {
        const uint32_t ck = L.k[0];
        const int cid = lane + kWave * L.i[0];
        const uint32_t m = wave_max_u32(ck);
        const unsigned long long tied = __ballot(ck == m);
        int wl = (int)__ffsll((long long)tied) - 1;
        if (__popcll(tied) > 1) {  // equal keys in several lanes: lowest expert id wins
            const uint32_t id = (ck == m) ? (uint32_t)cid : 0xFFFFFFFFu;
            wl = (int)(wave_min_u32(id) & (kWave - 1));
        }
        const int e = (int)readlane((uint32_t)cid, wl);
        const float se = __uint_as_float(readlane(__float_as_uint(L.s[0]), wl));
        mine = lane == r ? e : mine;
        s_mine = lane == r ? se : s_mine;
        // The winning lane drops its head; every lane runs the same
        // selects, so the round has no branch.
        const bool pop = lane == wl;
        const uint32_t pk = L.k[0];
        const int pi = L.i[0];
#pragma unroll
        for (int j = 0; j + 1 < kList; ++j) {
            L.k[j] = pop ? L.k[j + 1] : L.k[j];
            L.i[j] = pop ? L.i[j + 1] : L.i[j];
            L.s[j] = pop ? L.s[j + 1] : L.s[j];
        }
        L.k[kList - 1] = pop ? 0u : L.k[kList - 1];
        npop += pop ? 1 : 0;
        if (__ballot(npop == kList)) {  // rare: some lane used its whole list
            if (npop == kList) {
                fill_list(L, ok, sc, pk, pi);
                npop = 0;
            }
        }
    }
}

// Top-k of one token, by one wave.  Lane l owns experts l, l+64, ... and
// keeps their keys and scores in registers.  The selection (by threshold, or
// by rounds when more than 64 keys pass the threshold) leaves lane r with the
// id and score of the r-th expert in selection order; ranks among the
// selected ids and the sum of the selected scores (in selection order) follow,
// and the ids are written in ascending order with weights s_e / sum(s).
// Scores and keys are read with agent-scope loads, all in one batch: they
// were published by other workgroups.
// Agent: the keys and scores come from other workgroups of the same launch
// (agent-scope loads) and the selections go to them (agent-scope stores);
// otherwise the keys come from an earlier launch and the selections are
// written to global memory only when `global` (LDS always).
// FromLds: the keys and scores are read from kr and sr (LDS rows of
// kMaxExperts entries written before a workgroup barrier), and the threshold
// selection takes wave w's candidate row w of lds.
template <bool Agent, bool FromLds = false, typename Lds>
__device__ __forceinline__ void topk_token(const RouteArgs &a, int b, Lds &lds, bool global = true,
                                           const float *kr = nullptr, const float *sr = nullptr) {
    const int lane = lane_id();
    const int E = a.E, k = a.k;
    const float *keyrow = FromLds ? kr : a.key + (size_t)b * kMaxExperts;  // rows padded to kMaxExperts
    const float *srow = FromLds ? sr : a.score + (size_t)b * kMaxExperts;
    const int nk = (E + kWave - 1) / kWave;
    // All loads first, then their uses: the compiler keeps atomic loads in
    // program order, so a use between two of them would serialise the round
    // trips.
    uint32_t ok[kKeysPerLane];
    float sc[kKeysPerLane];
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i)
        ok[i] = __float_as_uint(Agent && !FromLds ? load_agent(keyrow + lane + kWave * i)
                                                  : keyrow[lane + kWave * i]);
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i)
        sc[i] = Agent && !FromLds ? load_agent(srow + lane + kWave * i) : srow[lane + kWave * i];
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
        const bool in = i < nk && lane + kWave * i < E;
        ok[i] = in ? orderable(__uint_as_float(ok[i])) : 0u;
    }
    int mine = 0;
    float s_mine = 0.f;
    // The routing inside the dense-in launch takes the rounds when it loads
    // the keys from memory: the threshold selection's registers would spill
    // there, in a kernel whose other code needs them all.
    // Each lane's selection (sel), its place among the selected ids (pos)
    // and the sum of the selected scores in selection order (total).
    bool done = false, sel = false;
    int pos = 0;
    float total = 0.f;
    if constexpr (!Agent || FromLds) {
        const int wv = wave_index();
        done = select_by_threshold(ok, sc, k, lds.cand_key[wv], lds.cand_id[wv], lds.cand_s[wv],
                                   mine, s_mine, sel, pos, total);
    }
    if (!done) {
        // Lane r holds the r-th selection.
        select_by_rounds(ok, sc, k, mine, s_mine);
        for (int r = 0; r < k; ++r) {
            const int other = (int)readlane((uint32_t)mine, r);
            pos += other < mine ? 1 : 0;
            total += __uint_as_float(readlane(__float_as_uint(s_mine), r));
        }
        sel = lane < k;
    }
    if (sel) {
        const float w = s_mine / total;
        const int o = b * k + pos;
        lds.idx[o] = (int16_t)mine;
        lds.w[o] = w;
        if (Agent) {
            // With routing units, another workgroup of the launch builds the
            // metadata from these.
            store_agent(a.idx + o, mine);
            store_agent(a.wsel + o, w);
        } else if (global) {
            a.idx[o] = mine;
            a.wsel[o] = w;
        }
        if (global && a.user_idx) a.user_idx[o] = mine;
        if (global && a.user_w) a.user_w[o] = w;
    }
}

// Top-k of one token by all kWG waves of a workgroup (every wave calls it;
// workgroup barriers inside).  Wave w holds the keys and scores of the
// experts lane + 64 (2w) and lane + 64 (2w + 1), so that the loads and the
// scans are spread over the waves:
//  1. every wave publishes its lanes' maxima; wave 0 takes per lane the
//     maximum over the waves (the lane's maximum over all its experts) and
//     finds T, the k-th largest of those 64 (a radix select over the bits
//     below the lanes' common prefix), so that at least k keys are >= T and
//     every expert of the top k has a key >= T;
//  2. every wave counts its keys >= T; the candidates are compacted into LDS
//     in (slot, lane) order, which is ascending expert id;
//  3. wave 0 ranks the candidates in selection order (larger key first, equal
//     keys by lower id), keeps those of rank < k, writes them in ascending id
//     (the candidate order) with weights s / sum(s), the sum taken in
//     selection order.
// More than 64 candidates (ties over many experts): wave 0 loads every key of
// the token and takes the rounds.  Agent: the keys come from other workgroups
// of the same launch and the selections go to them; `global`: write the
// selections to global memory (LDS always).
template <bool Agent, typename Lds>
__device__ void topk_token_wg(const RouteArgs &a, int b, Lds &lds, bool global = true) {
    const int lane = lane_id(), wave = wave_index();
    const int E = a.E, k = a.k;
    const float *keyrow = a.key + (size_t)b * kMaxExperts;
    const float *srow = a.score + (size_t)b * kMaxExperts;
    uint32_t ok[2];
    float sc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = lane + kWave * (2 * wave + j);
        const int ec = e < E ? e : 0;
        ok[j] = __float_as_uint(Agent ? load_agent(keyrow + ec) : keyrow[ec]);
        sc[j] = Agent ? load_agent(srow + ec) : srow[ec];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = lane + kWave * (2 * wave + j);
        ok[j] = e < E ? orderable(__uint_as_float(ok[j])) : 0u;
    }
    lds.wmax[wave][lane] = max(ok[0], ok[1]);
    __syncthreads();
    if (wave == 0) {
        uint32_t lm = 0u;
#pragma unroll
        for (int w = 0; w < kWG; ++w) lm = max(lm, lds.wmax[w][lane]);
        // Radix select of the k-th largest lane maximum, over the bits below
        // the common prefix of the lanes' maxima (absent lanes, 0, excluded).
        const uint32_t hi = wave_max_u32(lm);
        const uint32_t lo = wave_min_u32(lm != 0u ? lm : hi);
        const int top = 31 - __builtin_clz((hi ^ lo) | 1u);
        uint32_t T = hi & ~((2u << top) - 1u);
        for (int bit = top; bit >= 0; --bit) {
            const uint32_t t = T | (1u << bit);
            T = __popcll(__ballot(lm >= t)) >= k ? t : T;
        }
        if (lane == 0) lds.thr = T;
    }
    __syncthreads();
    const uint32_t T = lds.thr;
    const bool c0 = ok[0] != 0u && ok[0] >= T, c1 = ok[1] != 0u && ok[1] >= T;
    const unsigned long long m0 = __ballot(c0), m1 = __ballot(c1);
    if (lane == 0) lds.wcnt[wave] = __popcll(m0) + __popcll(m1);
    __syncthreads();
    int base = 0, n = 0;
#pragma unroll
    for (int w = 0; w < kWG; ++w) {
        const int cw = lds.wcnt[w];
        base += w < wave ? cw : 0;
        n += cw;
    }
    if (n <= kWave) {
        const int p0 = base + lanes_below(m0), p1 = base + __popcll(m0) + lanes_below(m1);
        if (c0) {
            lds.cand_key[0][p0] = ok[0];
            lds.cand_id[0][p0] = lane + kWave * (2 * wave);
            lds.cand_s[0][p0] = sc[0];
        }
        if (c1) {
            lds.cand_key[0][p1] = ok[1];
            lds.cand_id[0][p1] = lane + kWave * (2 * wave + 1);
            lds.cand_s[0][p1] = sc[1];
        }
    }
    if (n > kWave) {
        // More than 64 keys >= T (ties over many experts): the keys and
        // scores go to LDS (the token-mask area, free until the metadata)
        // and wave 0 takes the exact k-th largest key Tk, then the experts
        // with larger keys and the lowest-id ones equal to Tk, as the k
        // candidates.
        unsigned long long *kv = lds.mask;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = lane + kWave * (2 * wave + j);
            if (e < E) kv[e] = (unsigned long long)ok[j] | ((unsigned long long)__float_as_uint(sc[j]) << 32);
        }
        __syncthreads();
        if (wave == 0) {
            const int nk = (E + kWave - 1) / kWave;
            uint32_t Tk = 0u;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t t = Tk | (1u << bit);
                int cnt = 0;
                for (int i = 0; i < nk; ++i) {
                    const int e = lane + kWave * i;
                    cnt += __popcll(__ballot(e < E && (uint32_t)kv[e] >= t));
                }
                Tk = cnt >= k ? t : Tk;
            }
            int gt = 0;
            for (int i = 0; i < nk; ++i) {
                const int e = lane + kWave * i;
                gt += __popcll(__ballot(e < E && (uint32_t)kv[e] > Tk));
            }
            int eq_before = 0, sel_before = 0;
            for (int i = 0; i < nk; ++i) {
                const int e = lane + kWave * i;
                const uint32_t key = e < E ? (uint32_t)kv[e] : 0u;
                const bool eq = e < E && key == Tk;
                const unsigned long long me = __ballot(eq);
                const bool sel = (e < E && key > Tk) || (eq && eq_before + lanes_below(me) < k - gt);
                const unsigned long long ms = __ballot(sel);
                if (sel) {
                    const int pos = sel_before + lanes_below(ms);
                    lds.cand_key[0][pos] = key;
                    lds.cand_id[0][pos] = e;
                    lds.cand_s[0][pos] = __uint_as_float((uint32_t)(kv[e] >> 32));
                }
                eq_before += __popcll(me);
                sel_before += __popcll(ms);
            }
        }
        n = k;
    }
    __syncthreads();
    if (wave != 0) return;
    // Wave 0: lanes < n hold the candidates in ascending id; their ranks in
    // selection order pick the k.
    const bool have = lane < n;
    const uint32_t ck = have ? lds.cand_key[0][lane] : 0u;
    const int mine = have ? lds.cand_id[0][lane] : 0;
    const float s_mine = have ? lds.cand_s[0][lane] : 0.f;
    int rank = 0;
    for (int j = 0; j < n; ++j) {
        const uint32_t kj = readlane(ck, j);
        rank += (kj > ck || (kj == ck && j < lane)) ? 1 : 0;
    }
    const bool selected = have && rank < k;
    const int sel_pos = lanes_below(__ballot(selected));  // ascending id among the selected
    wave_sync();
    if (selected) lds.cand_s[1][rank] = s_mine;  // scores in selection order
    wave_sync();
    float total = 0.f;
    for (int r = 0; r < k; ++r) total += lds.cand_s[1][r];
    if (selected) {
        const float w = s_mine / total;
        const int o = b * k + sel_pos;
        lds.idx[o] = (int16_t)mine;
        lds.w[o] = w;
        if (Agent) {
            store_agent(a.idx + o, mine);
            store_agent(a.wsel + o, w);
        } else if (global) {
            a.idx[o] = mine;
            a.wsel[o] = w;
        }
        if (global && a.user_idx) a.user_idx[o] = mine;
        if (global && a.user_w) a.user_w[o] = w;
    }
}

// Routing metadata from the selections in LDS, by all nw waves of the routing
// workgroup.  Active experts are listed in ascending id; the pairs of an
// expert in ascending token; each expert's pairs are cut into column units of
// at most 8 tokens (16 MFMA columns: hi and lo of each token).  A unit's
// record holds everything its workgroups need, so that they read it in one
// round trip: expert, pair count, first pair, and per pair the token and the
// routing weight.  A pair's place follows from the token mask of its expert
// (the token's rank among the expert's tokens), so pairs are placed in
// parallel; expert offsets come from a two-level scan (lanes, then waves).
// Everything is written with agent-scope stores: in the fused step the
// expert units of other workgroups read it within the same launch.
// ToLds: the records go to lds.rec (and the unit count to lds.ncols) for the
// workgroup's own use, and nothing is written to global memory.
// A store of the routing metadata: agent-scope (written through to the
// device's coherent level) when workgroups of the same launch read it, plain
// when only later launches do (the kernel boundary publishes it; a plain
// store stays in the writer's L2 until then and costs the routing workgroup
// far less under a full memory stream).
template <bool Agent, typename T>
__device__ __forceinline__ void meta_store(T *p, T v) {
    if constexpr (Agent)
        store_agent(p, v);
    else
        *p = v;
}

template <bool ToLds, bool Agent = true, typename Lds>
__device__ __forceinline__ void build_meta(const RouteArgs &a, Lds &lds, int nw) {
    const int lane = lane_id(), wave = wave_index();
    const int tid = threadIdx.x, nt = nw * kWave;
    const int B = a.B, k = a.k, E = a.E, P = B * k;
    for (int e = tid; e < E; e += nt) lds.mask[e] = 0ull;
    __syncthreads();
    for (int p = tid; p < P; p += nt) atomicOr(&lds.mask[lds.idx[p]], 1ull << (p / k));
    __syncthreads();
    const int C = (E + nt - 1) / nt;
    const int e0 = min(E, tid * C), e1 = min(E, e0 + C);
    int na = 0, np = 0, nc = 0;
    for (int e = e0; e < e1; ++e) {
        const int n = __popcll(lds.mask[e]);
        na += n ? 1 : 0;
        np += n;
        nc += (n + 7) >> 3;
    }
    const int ia = wave_incl_scan(na), ip = wave_incl_scan(np), ic = wave_incl_scan(nc);
    if (lane == kWave - 1) {
        lds.wsum[wave][0] = ia;
        lds.wsum[wave][1] = ip;
        lds.wsum[wave][2] = ic;
    }
    __syncthreads();
    int ba = 0, bp = 0, bc = 0, D = 0, PT = 0, NC = 0;
    for (int w = 0; w < nw; ++w) {
        const int xa = lds.wsum[w][0], xp = lds.wsum[w][1], xc = lds.wsum[w][2];
        if (w < wave) {
            ba += xa;
            bp += xp;
            bc += xc;
        }
        D += xa;
        PT += xp;
        NC += xc;
    }
    int ai = ba + ia - na, pi = bp + ip - np, ci = bc + ic - nc;
    for (int e = e0; e < e1; ++e) {
        const int n = __popcll(lds.mask[e]);
        lds.off[e] = pi;
        lds.unit[e] = ci;
        if (!n) continue;
        if (!ToLds) {
            meta_store<Agent>(a.act_expert + ai, e);
            meta_store<Agent>(a.act_off + ai, pi);
        }
        for (int r = 0; r < n; r += 8, ++ci) {
            if (ToLds) {
                lds.rec[ci][R_EXPERT] = e;
                lds.rec[ci][R_COUNT] = min(8, n - r);
                lds.rec[ci][R_PAIR0] = pi + r;
            } else {
                int32_t *rec = a.cu_rec + (size_t)ci * kRecWords;
                meta_store<Agent>(rec + R_EXPERT, e);
                meta_store<Agent>(rec + R_COUNT, min(8, n - r));
                meta_store<Agent>(rec + R_PAIR0, pi + r);
            }
        }
        ++ai;
        pi += n;
    }
    __syncthreads();
    for (int p = tid; p < P; p += nt) {
        const int e = lds.idx[p], b = p / k;
        const int r = __popcll(lds.mask[e] & ((1ull << b) - 1ull));
        const int pos = lds.off[e] + r;
        if (ToLds) {
            int *rec = lds.rec[lds.unit[e] + (r >> 3)];
            rec[R_TOKEN + (r & 7)] = b;
            rec[R_WEIGHT + (r & 7)] = __float_as_int(lds.w[p]);
        } else {
            meta_store<Agent>(a.pair_slot + pos, p);
            meta_store<Agent>(a.pair_of_slot + p, pos);
            int32_t *rec = a.cu_rec + (size_t)(lds.unit[e] + (r >> 3)) * kRecWords;
            meta_store<Agent>(rec + R_TOKEN + (r & 7), b);
            meta_store<Agent>(rec + R_WEIGHT + (r & 7), __float_as_int(lds.w[p]));
        }
    }
    if (tid == 0) {
        if (ToLds) {
            lds.ncols = NC;
            lds.n_active = D;
        } else {
            meta_store<Agent>(a.meta + M_N_ACTIVE, D);
            meta_store<Agent>(a.meta + M_N_COLS, NC);
            meta_store<Agent>(a.act_off + D, PT);
        }
    }
}

// The whole routing of the step, by every wave of the workgroup whose router
// arrival completed the router (all waves call it, after a workgroup
// barrier).  Tokens are split across the waves; the selections meet in LDS.
// Agent: workgroups of the same launch read the metadata (the persistent
// step); otherwise only later launches do.
template <bool Agent>
__device__ __forceinline__ void route_step(const RouteArgs &a, RouteLds *lds, int nwaves) {
    if (a.B == 1 && nwaves == kWG)
        topk_token_wg<true>(a, 0, *lds);
    else
        for (int b = wave_index(); b < a.B; b += nwaves) topk_token<true>(a, b, *lds);
    __syncthreads();
    build_meta<false, Agent>(a, *lds, nwaves);
}

// The routing at the start of the gate/up launch (B k <= kLatePairs; the keys
// and scores come from the dense-in launch before it): every workgroup
// selects the experts of every token (a wave per token) and builds the unit
// records in its own LDS.  The workgroup `lead` also writes the selections and
// the per-pair lists to global memory for the later launches (the unit
// records and the metadata header are written by the caller).  Ends with a
// workgroup barrier.
__device__ __forceinline__ void route_late(const RouteArgs &a, LateRouteLds &lds, bool lead) {
    if (a.B == 1)
        topk_token_wg<false>(a, 0, lds, lead);
    else
        for (int b = wave_index(); b < a.B; b += kWG) topk_token<false>(a, b, lds, lead);
    __syncthreads();
    if (a.B == 1) {
        // One token: every selected expert is one unit of one pair, in
        // ascending id (the order of the selection in LDS).
        const int tid = threadIdx.x, k = a.k;
        for (int i = tid; i < k * kRecWords; i += kWGThreads) {
            const int c = i / kRecWords, wd = i % kRecWords;
            int v = 0;
            if (wd == R_EXPERT) v = lds.idx[c];
            else if (wd == R_COUNT) v = 1;
            else if (wd == R_PAIR0) v = c;
            else if (wd == R_WEIGHT) v = __float_as_int(lds.w[c]);
            lds.rec[c][wd] = v;  // R_TOKEN: token 0
        }
        if (lead)
            for (int c = tid; c <= k; c += kWGThreads) {
                if (c < k) {
                    a.act_expert[c] = lds.idx[c];
                    a.pair_slot[c] = c;
                    a.pair_of_slot[c] = c;
                }
                a.act_off[c] = c;
            }
        if (tid == 0) {
            lds.ncols = k;
            lds.n_active = k;
        }
        __syncthreads();
        return;
    }
    build_meta<true>(a, lds, kWG);
    __syncthreads();
    if (lead) {
        // The active experts in ascending id (those with a non-empty token
        // mask) with the pair offsets that build_meta gave them, then the
        // pair maps.
        const int tid = threadIdx.x, P = a.B * a.k;
        if (wave_index() == 0) {
            int ai = 0;
            for (int e0 = 0; e0 < a.E; e0 += kWave) {
                const int e = e0 + lane_id();
                const bool act = e < a.E && lds.mask[e] != 0ull;
                const unsigned long long m = __ballot(act);
                if (act) {
                    const int i = ai + lanes_below(m);
                    a.act_expert[i] = e;
                    a.act_off[i] = lds.off[e];
                }
                ai += __popcll(m);
            }
            if (lane_id() == 0) a.act_off[ai] = P;
        }
        for (int p = tid; p < P; p += kWGThreads) {
            const int e = lds.idx[p], b = p / a.k;
            const int r = __popcll(lds.mask[e] & ((1ull << b) - 1ull));
            const int pos = lds.off[e] + r;
            a.pair_slot[pos] = p;
            a.pair_of_slot[p] = pos;
        }
        __syncthreads();
    }
}

}  // namespace moe
