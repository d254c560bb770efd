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

// LDS of the routing workgroup: the selections of every token, the token
// masks of the experts and per-expert offsets.
struct RouteLds {
    int16_t idx[kMaxBatch * kMaxTopK];
    float w[kMaxBatch * kMaxTopK];
    unsigned long long mask[kMaxExperts];
    int off[kMaxExperts];
    int unit[kMaxExperts];
};

// Top-k of one token, by one wave.  Lane l owns experts l, l+64, ... and
// keeps their keys and scores in registers, plus its best remaining (key,
// lowest id) as a candidate.  Each round takes the wave-wide largest
// candidate key (equal keys: the lowest expert id), the winning lane advances
// its candidate, and the selection is recorded in lane r (round r) together
// with its rank among the selected ids.  Selected ids are written in
// ascending order with weights s_e / sum(s); the sum is taken in selection
// order.  No memory access happens inside the rounds.
__device__ __forceinline__ void topk_token(const StepArgs &a, int b, RouteLds &lds) {
    const int lane = lane_id();
    const int E = a.E, k = a.k;
    const float *keyrow = a.key + (size_t)b * E;
    const float *srow = a.score + (size_t)b * E;
    const int nk = (E + kWave - 1) / kWave;
    uint32_t ok[kKeysPerLane];
    float os[kKeysPerLane];
    uint32_t avail = 0;
#pragma unroll
    for (int i = 0; i < kKeysPerLane; ++i) {
        const int e = lane + kWave * i;
        const bool in = i < nk && e < E;
        ok[i] = in ? orderable(keyrow[in ? e : 0]) : 0u;
        os[i] = in ? srow[in ? e : 0] : 0.f;
        avail |= in ? (1u << i) : 0u;
    }
    uint32_t ck;
    int ci;
    float cs;
    auto candidate = [&]() {
        ck = 0;
        ci = 0;
        cs = 0.f;
#pragma unroll
        for (int i = 0; i < kKeysPerLane; ++i) {
            const bool take = ((avail >> i) & 1u) && ok[i] > ck;  // strict: lowest i on ties
            ck = take ? ok[i] : ck;
            ci = take ? i : ci;
            cs = take ? os[i] : cs;
        }
    };
    candidate();
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
        const int e = (int)readlane((uint32_t)(lane + kWave * ci), wl);
        const float s = __uint_as_float(readlane(__float_as_uint(cs), wl));
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
            candidate();
        }
    }
    if (lane < k) {
        const float w = s_mine / total;
        const int o = b * k + rank;
        lds.idx[o] = (int16_t)mine;
        lds.w[o] = w;
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
// the routing weight.  A pair's place follows from the bit mask alone (its
// token's rank among the expert's tokens), so the pairs are placed in
// parallel.
__device__ __forceinline__ void build_meta(const StepArgs &a, RouteLds &lds) {
    const int lane = lane_id();
    const int B = a.B, k = a.k, E = a.E;
    for (int e = lane; e < E; e += kWave) lds.mask[e] = 0ull;
    wave_sync();
    for (int p = lane; p < B * k; p += kWave) atomicOr(&lds.mask[lds.idx[p]], 1ull << (p / k));
    wave_sync();
    const int C = (E + kWave - 1) / kWave;
    const int e0 = lane * C, e1 = min(E, e0 + C);
    int na = 0, np = 0, nc = 0;
    for (int e = e0; e < e1; ++e) {
        const int n = __popcll(lds.mask[e]);
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
        const int n = __popcll(lds.mask[e]);
        lds.off[e] = pi;
        lds.unit[e] = ci;
        if (!n) continue;
        a.act_expert[ai] = e;
        a.act_off[ai] = pi;
        for (int r = 0; r < n; r += 8, ++ci) {
            int32_t *rec = a.cu_rec + (size_t)ci * kRecWords;
            rec[R_EXPERT] = e;
            rec[R_COUNT] = min(8, n - r);
            rec[R_PAIR0] = pi + r;
        }
        ++ai;
        pi += n;
    }
    wave_sync();
    for (int p = lane; p < B * k; p += kWave) {
        const int e = lds.idx[p], b = p / k;
        const int r = __popcll(lds.mask[e] & ((1ull << b) - 1ull));
        const int pos = lds.off[e] + r;
        a.pair_slot[pos] = p;
        a.pair_of_slot[p] = pos;
        int32_t *rec = a.cu_rec + (size_t)(lds.unit[e] + (r >> 3)) * kRecWords;
        rec[R_TOKEN + (r & 7)] = b;
        rec[R_WEIGHT + (r & 7)] = __float_as_int(lds.w[p]);
    }
    if (lane == 0) {
        a.meta[M_N_ACTIVE] = D;
        a.meta[M_N_COLS] = NC;
        a.act_off[D] = P;
    }
}

// The whole routing of the step, by every wave of the workgroup whose router
// arrival completed the router (all waves call it, after a workgroup
// barrier).  Tokens are split across the waves; the selections meet in LDS.
__device__ __forceinline__ void route_step(const StepArgs &a, RouteLds &lds, int nwaves) {
    acquire_agent();  // every router tile's scores and keys
    for (int b = wave_index(); b < a.B; b += nwaves) topk_token(a, b, lds);
    __syncthreads();
    if (wave_index() == 0) build_meta(a, lds);
}

}  // namespace moe
