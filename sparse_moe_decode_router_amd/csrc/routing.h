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
// The work runs inside the kernel that produces the router scores: the wave
// whose arrival completes the router starts claiming tokens, and any wave that
// finishes a tile afterwards joins it; the wave that completes the last token
// builds the metadata.  No wave ever waits on another.  Wave-wide reductions
// and scans use DPP row operations and scalar lane reads, so one top-16 of
// 896 costs a few thousand cycles of one wave.
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

// Top-k of one token, by one wave.  Lane l owns experts l, l+64, ... and
// keeps its best remaining (key, lowest id) as a candidate.  Each round takes
// the wave-wide largest candidate key (equal keys: the lowest expert id), the
// winning lane advances its candidate, and the selection is recorded in lane
// r (round r) together with its rank among the selected ids.  Selected ids
// are written in ascending order with weights s_e / sum(s); the sum is taken
// in selection order.
__device__ __forceinline__ void topk_token(const StepArgs &a, int b) {
    const int lane = lane_id();
    const int E = a.E, k = a.k;
    const float *keyrow = a.key + (size_t)b * E;
    const float *srow = a.score + (size_t)b * E;
    const int nk = (E + kWave - 1) / kWave;
    uint32_t ok[kKeysPerLane];
    uint32_t avail = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
        const int e = lane + kWave * i;
        const bool in = i < nk && e < E;
        ok[i] = in ? orderable(keyrow[in ? e : 0]) : 0u;
        avail |= in ? (1u << i) : 0u;
    }
    auto candidate = [&](uint32_t &ck, int &ci) {
        ck = 0;
        ci = 0;
#pragma unroll
        for (int i = 0; i < kKeysPerLane; ++i) {
            const bool take = ((avail >> i) & 1u) && ok[i] > ck;  // strict: lowest i on ties
            ck = take ? ok[i] : ck;
            ci = take ? i : ci;
        }
    };
    uint32_t ck;
    int ci;
    candidate(ck, ci);
    int mine = 0, rank = 0;
    float s_mine = 0.f, total = 0.f;
    for (int r = 0; r < k; ++r) {
        const uint32_t m = wave_max_u32(ck);
        const unsigned long long tied = __ballot(ck == m);
        int wl = (int)__ffsll((long long)tied) - 1;
        if (__popcll(tied) > 1) {  // equal keys in several lanes: lowest expert id wins
            const uint32_t id = (ck == m) ? (uint32_t)(lane + kWave * ci) : 0xFFFFFFFFu;
            wl = (int)(wave_min_u32(id) & (kWave - 1));
        }
        const int e = (int)readlane((uint32_t)(wl + kWave * ci), wl);
        const float s = srow[e];  // same address in every lane: one load
        total += s;
        // Ranks: earlier selections above e move up; the new one counts the
        // earlier selections below it.
        const bool earlier = lane < r;
        rank += (earlier && mine > e) ? 1 : 0;
        const unsigned long long below = __ballot(earlier && mine < e);
        if (lane == r) {
            mine = e;
            s_mine = s;
            rank = __popcll(below);
        }
        if (lane == wl) {
            avail &= ~(1u << ci);
            candidate(ck, ci);
        }
    }
    if (lane < k) {
        const float w = s_mine / total;
        const int o = b * k + rank;
        a.idx[o] = mine;
        a.wsel[o] = w;
        if (a.user_idx) a.user_idx[o] = mine;
        if (a.user_w) a.user_w[o] = w;
    }
}

// Routing metadata from idx [B][k], by one wave, with an LDS bit mask of the
// tokens of each expert.  Active experts are listed in ascending id; the pairs
// of an expert in ascending token; each expert's pairs are cut into column
// units of at most 8 tokens (16 MFMA columns: hi and lo of each token).  A
// unit's record holds everything its workgroups need, so that they read it in
// one round trip: expert, pair count, first pair, and per pair the token and
// the routing weight.
__device__ __forceinline__ void build_meta(const StepArgs &a, unsigned long long *s_mask) {
    const int lane = lane_id();
    const int B = a.B, k = a.k, E = a.E;
    for (int e = lane; e < E; e += kWave) s_mask[e] = 0ull;
    wave_sync();
    for (int p = lane; p < B * k; p += kWave) atomicOr(&s_mask[a.idx[p]], 1ull << (p / k));
    wave_sync();
    const int C = (E + kWave - 1) / kWave;
    const int e0 = lane * C, e1 = min(E, e0 + C);
    int na = 0, np = 0, nc = 0;
    for (int e = e0; e < e1; ++e) {
        const int n = __popcll(s_mask[e]);
        na += n ? 1 : 0;
        np += n;
        nc += (n + 7) >> 3;
    }
    const int ia = wave_incl_scan(na), ip = wave_incl_scan(np), ic = wave_incl_scan(nc);
    const int D = (int)readlane((uint32_t)ia, kWave - 1);
    const int P = (int)readlane((uint32_t)ip, kWave - 1);
    const int NC = (int)readlane((uint32_t)ic, kWave - 1);
    int ai = ia - na, pi = ip - np, ci = ic - nc;
    for (int e = e0; e < e1; ++e) {
        unsigned long long m = s_mask[e];
        const int n = __popcll(m);
        if (!n) continue;
        a.act_expert[ai] = e;
        a.act_off[ai] = pi;
        for (int r = 0; m; ++r) {
            const int b = __ffsll((long long)m) - 1;
            m &= m - 1;
            const int *row = a.idx + b * k;  // ascending ids
            int lo = 0, hi = k - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (row[mid] < e) lo = mid + 1; else hi = mid;
            }
            const int slot = b * k + lo;
            a.pair_slot[pi + r] = slot;
            a.pair_of_slot[slot] = pi + r;
            int32_t *rec = a.cu_rec + (size_t)(ci + (r >> 3)) * kRecWords;
            if ((r & 7) == 0) {
                rec[R_EXPERT] = e;
                rec[R_COUNT] = min(8, n - r);
                rec[R_PAIR0] = pi + r;
            }
            rec[R_TOKEN + (r & 7)] = b;
            rec[R_WEIGHT + (r & 7)] = __float_as_int(a.wsel[slot]);
        }
        ci += (n + 7) >> 3;
        ++ai;
        pi += n;
    }
    if (lane == 0) {
        a.meta[M_N_ACTIVE] = D;
        a.meta[M_N_COLS] = NC;
        a.act_off[D] = P;
    }
}

// Claims tokens until none is left; the wave that finishes the last token
// builds the metadata.  Called only once the router is complete.
__device__ __forceinline__ void topk_loop(const StepArgs &a, unsigned long long *s_mask) {
    acquire_agent();
    // Claims are unique, so one wave can never claim more than B tokens.
    for (int it = 0; it < a.B; ++it) {
        const uint32_t t = wave_fetch_add(&a.gctr[G_NEXT_TOKEN], 1u);
        if (t >= (uint32_t)a.B) break;
        topk_token(a, (int)t);
        if (wave_arrive(&a.gctr[G_TOKENS_DONE]) == (uint32_t)a.B - 1u) {
            acquire_agent();
            build_meta(a, s_mask);
        }
    }
}

// A wave that finished a tile helps with the top-k when the router is
// complete and tokens are still unclaimed.
__device__ __forceinline__ void maybe_join_topk(const StepArgs &a, unsigned long long *s_mask) {
    if (wave_load_counter(&a.gctr[G_ROUTER_DONE]) != (uint32_t)a.router_target) return;
    if (wave_load_counter(&a.gctr[G_NEXT_TOKEN]) >= (uint32_t)a.B) return;
    topk_loop(a, s_mask);
}

}  // namespace moe
