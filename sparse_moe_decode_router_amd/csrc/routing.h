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

// LDS of the routing workgroup: the selections of every token, the token
// masks of the experts, per-expert offsets and per-wave scan totals.
struct RouteLds {
    int16_t idx[kMaxBatch * kMaxTopK];
    float w[kMaxBatch * kMaxTopK];
    unsigned long long mask[kMaxExperts];
    int off[kMaxExperts];
    int unit[kMaxExperts];
    int wsum[kMaxRouteWaves][4];
};

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

// Top-k of one token, by one wave.  Lane l owns experts l, l+64, ... and
// keeps their keys and scores in registers and a short list of its best
// remaining ones.  Each round takes the wave-wide largest list head (equal
// keys: the lowest expert id); lane r keeps the id and score of round r's
// winner, and the winning lane drops its head (and rebuilds its list after
// kList drops).  The round does nothing else: ranks among the selected ids
// and the sum of the selected scores (in selection order) follow the last
// round, and the ids are written in ascending order with weights
// s_e / sum(s).  Scores and keys are read with agent-scope loads, all in one
// batch: they were published by other workgroups.
__device__ __forceinline__ void topk_token(const RouteArgs &a, int b, RouteLds &lds) {
    const int lane = lane_id();
    const int E = a.E, k = a.k;
    const float *keyrow = a.key + (size_t)b * kMaxExperts;  // rows padded to kMaxExperts
    const float *srow = a.score + (size_t)b * kMaxExperts;
    const int nk = (E + kWave - 1) / kWave;
    // All loads first, then their uses: the compiler keeps atomic loads in
    // program order, so a use between two of them would serialise the round
    // trips.
    uint32_t ok[kKeysPerLane];
    float sc[kKeysPerLane];
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) ok[i] = __float_as_uint(load_agent(keyrow + lane + kWave * i));
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) sc[i] = load_agent(srow + lane + kWave * i);
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
        const bool in = i < nk && lane + kWave * i < E;
        ok[i] = in ? orderable(__uint_as_float(ok[i])) : 0u;
    }
    LaneList L;
    fill_list(L, ok, sc, 0xFFFFFFFFu, -1);
    int npop = 0;
    int mine = 0;
    float s_mine = 0.f;
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
    // Rank of each selection among the selected ids; sum of the selected
    // scores in selection order.
    int rank = 0;
    float total = 0.f;
    for (int r = 0; r < k; ++r) {
        const int other = (int)readlane((uint32_t)mine, r);
        rank += other < mine ? 1 : 0;
        total += __uint_as_float(readlane(__float_as_uint(s_mine), r));
    }
    if (lane < k) {
        const float w = s_mine / total;
        const int o = b * k + rank;
        lds.idx[o] = (int16_t)mine;
        lds.w[o] = w;
        // Agent-scope: with routing units, another workgroup of the launch
        // builds the metadata from these.
        store_agent(a.idx + o, mine);
        store_agent(a.wsel + o, w);
        if (a.user_idx) a.user_idx[o] = mine;
        if (a.user_w) a.user_w[o] = w;
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
__device__ __forceinline__ void build_meta(const RouteArgs &a, RouteLds &lds, int nw) {
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
        store_agent(a.act_expert + ai, e);
        store_agent(a.act_off + ai, pi);
        for (int r = 0; r < n; r += 8, ++ci) {
            int32_t *rec = a.cu_rec + (size_t)ci * kRecWords;
            store_agent(rec + R_EXPERT, e);
            store_agent(rec + R_COUNT, min(8, n - r));
            store_agent(rec + R_PAIR0, pi + r);
        }
        ++ai;
        pi += n;
    }
    __syncthreads();
    for (int p = tid; p < P; p += nt) {
        const int e = lds.idx[p], b = p / k;
        const int r = __popcll(lds.mask[e] & ((1ull << b) - 1ull));
        const int pos = lds.off[e] + r;
        store_agent(a.pair_slot + pos, p);
        store_agent(a.pair_of_slot + p, pos);
        int32_t *rec = a.cu_rec + (size_t)(lds.unit[e] + (r >> 3)) * kRecWords;
        store_agent(rec + R_TOKEN + (r & 7), b);
        store_agent(rec + R_WEIGHT + (r & 7), __float_as_int(lds.w[p]));
    }
    if (tid == 0) {
        store_agent(a.meta + M_N_ACTIVE, D);
        store_agent(a.meta + M_N_COLS, NC);
        store_agent(a.act_off + D, PT);
    }
}

// The whole routing of the step, by every wave of the workgroup whose router
// arrival completed the router (all waves call it, after a workgroup
// barrier).  Tokens are split across the waves; the selections meet in LDS.
__device__ __forceinline__ void route_step(const RouteArgs &a, RouteLds *lds, int nwaves) {
    for (int b = wave_index(); b < a.B; b += nwaves) topk_token(a, b, *lds);
    __syncthreads();
    build_meta(a, *lds, nwaves);
}

}  // namespace moe
