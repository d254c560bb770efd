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
// builds the metadata.  No wave ever waits on another.
#pragma once

#include "device_common.h"
#include "step_args.h"

namespace moe {

// Orders (key, id) pairs: larger key first, then lower id, as one u64 maximum.
__device__ __forceinline__ uint64_t pack_key(float key, int e) {
    const uint32_t u = __float_as_uint(key);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}

// Top-k of one token, by one wave.  The token's keys are staged in the
// wave's LDS buffer; lane l owns experts l, l+64, ...; k rounds of a
// wave-wide maximum pick the experts in key order; they are then written in
// ascending id with weights s_e / sum(s).
__device__ __forceinline__ void topk_token(const StepArgs &a, int b, float *s_keys) {
    const int lane = lane_id();
    const int E = a.E, k = a.k;
    const float *keyrow = a.key + (size_t)b * E;
    for (int e = lane; e < E; e += kWave) s_keys[e] = keyrow[e];
    wave_sync();
    const int nk = (E + kWave - 1) / kWave;
    uint32_t avail = 0;
    for (int i = 0; i < nk; ++i) avail |= (lane + kWave * i < E) ? (1u << i) : 0u;
    // First maximum of this lane's available keys in ascending id, packed.
    auto local_best = [&]() {
        float bk = 0.f;
        int bi = -1;
        for (int i = 0; i < nk; ++i) {
            const float v = s_keys[lane + kWave * i];
            const bool take = ((avail >> i) & 1u) && (bi < 0 || v > bk);
            bk = take ? v : bk;
            bi = take ? i : bi;
        }
        return bi < 0 ? (uint64_t)0 : pack_key(bk, lane + kWave * bi);
    };
    uint64_t best = local_best();
    int mine = 0x7FFFFFFF;
    for (int r = 0; r < k; ++r) {
        const uint64_t w = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)w);
        if (lane == r) mine = e;
        if ((e & (kWave - 1)) == lane) {
            avail &= ~(1u << (e >> 6));
            best = local_best();
        }
    }
    int rank = 0;
    for (int r = 0; r < k; ++r) rank += __shfl(mine, r) < mine ? 1 : 0;
    const float s = lane < k ? a.score[(size_t)b * E + mine] : 0.f;
    const float total = wave_sum(s);
    if (lane < k) {
        const float w = s / total;
        const int o = b * k + rank;
        a.idx[o] = mine;
        a.wsel[o] = w;
        if (a.user_idx) a.user_idx[o] = mine;
        if (a.user_w) a.user_w[o] = w;
    }
    wave_sync();
}

// Routing metadata from idx [B][k], by one wave, with an LDS bit mask of the
// tokens of each expert.  Active experts are listed in ascending id; the pairs
// of an expert in ascending token; each expert's pairs are cut into column
// units of at most 8 tokens (16 MFMA columns: hi and lo of each token).
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
    int D, P, NC;
    int ai = wave_excl_scan(na, &D);
    int pi = wave_excl_scan(np, &P);
    int ci = wave_excl_scan(nc, &NC);
    for (int e = e0; e < e1; ++e) {
        unsigned long long m = s_mask[e];
        const int n = __popcll(m);
        if (!n) continue;
        a.act_expert[ai] = e;
        a.act_off[ai] = pi;
        for (int q = 0; q < n; q += 8, ++ci) {
            a.cu_expert[ci] = e;
            a.cu_p0[ci] = pi + q;
            a.cu_n[ci] = min(8, n - q);
        }
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
        }
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
// builds the metadata.  Called only once the router is complete.  s_keys is
// the calling wave's own LDS buffer of kMaxExperts floats.
__device__ __forceinline__ void topk_loop(const StepArgs &a, unsigned long long *s_mask,
                                       float *s_keys) {
    acquire_agent();
    // Claims are unique, so one wave can never claim more than B tokens.
    for (int it = 0; it < a.B; ++it) {
        const uint32_t t = wave_fetch_add(&a.gctr[G_NEXT_TOKEN], 1u);
        if (t >= (uint32_t)a.B) break;
        topk_token(a, (int)t, s_keys);
        if (wave_arrive(&a.gctr[G_TOKENS_DONE]) == (uint32_t)a.B - 1u) {
            acquire_agent();
            build_meta(a, s_mask);
        }
    }
}

// A wave that finished a tile helps with the top-k when the router is
// complete and tokens are still unclaimed.
__device__ __forceinline__ void maybe_join_topk(const StepArgs &a, unsigned long long *s_mask,
                                                float *s_keys) {
    if (wave_load_counter(&a.gctr[G_ROUTER_DONE]) != (uint32_t)a.router_target) return;
    if (wave_load_counter(&a.gctr[G_NEXT_TOKEN]) >= (uint32_t)a.B) return;
    topk_loop(a, s_mask, s_keys);
}

}  // namespace moe
