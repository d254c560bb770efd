// moe_limits.h - sizes and slot numbers shared by the host planning code and the
// kernels: wave and workgroup shapes, the supported maxima, and the layout of
// the counter area at the head of the workspace.  Plain C++: no HIP headers,
// so that the host planning code also builds with an ordinary compiler.
#pragma once

namespace moe {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kWG = 8;               // waves per workgroup of the step kernels
constexpr int kWGThreads = kWG * kWave;
constexpr int kXcds = 8;             // XCDs of MI355X; workgroup i runs on XCD i % 8
constexpr int kKStep = 128;          // K elements one lane group covers per step (4 x 32)
constexpr int kMaxExperts = 1024;
constexpr int kMaxBatch = 64;
constexpr int kMaxTopK = 64;
constexpr int kMaxStepsPerChunk = 8;
// Longest dense reduction: kWG waves of kMaxStepsPerChunk steps.
constexpr int kMaxDenseK = kKStep * kWG * kMaxStepsPerChunk;  // 8192

// Counter slots (u32 word indices into the counter area).  G_ROUTER_DONE:
// router arrivals.  The fused step also uses: the unit queue (G_WORK),
// workgroups that left it (G_EXIT), the routing published (G_ROUTED),
// latent-down / shared gate/up / shared-down / down units done, and a sticky
// error flag (a bounded wait ran out).  Counters sit 256 bytes apart: atomics
// and polls on one line from many workgroups serialise at the memory side.
constexpr int kCtrStride = 64;
enum {
    G_ROUTER_DONE = 0,
    G_WORK = 1 * kCtrStride,
    G_EXIT = 2 * kCtrStride,
    G_ROUTED = 3 * kCtrStride,
    G_LATENT = 4 * kCtrStride,
    G_SHARED = 5 * kCtrStride,
    G_SHDOWN = 6 * kCtrStride,
    G_W2 = 7 * kCtrStride,
    G_ERROR = 8 * kCtrStride,
    G_COUNT = 9 * kCtrStride
};
// Routing metadata header (i32).
enum { M_N_ACTIVE = 0, M_N_COLS = 1, M_COUNT = 16 };
// Column-unit record (i32 words): expert, pair count (<= 8), first pair index,
// then the token and the routing weight (f32 bits) of each pair.
enum { R_EXPERT = 0, R_COUNT = 1, R_PAIR0 = 2, R_TOKEN = 8, R_WEIGHT = 16, kRecWords = 32 };

constexpr int kMaxSlices = 16;     // K slices of the large-batch dense-in kernel
constexpr int kMaxSlicesOut = 8;   // ... and of the large-batch output kernel

// Tokens per routing unit of the large-batch dense-in launch when that
// launch holds the bf16 router (the units add the router's K-slice partial
// sums themselves).
constexpr int kRouteTokensTp = 2;

// Ordered latent combine: one arrival counter per (token, tile group of the
// down kernel), tile groups of at least 64 latent rows, counters 64 bytes
// apart.
constexpr int kOrdGroups = kMaxDenseK / 64;
constexpr int kOrdStride = 16;

}  // namespace moe
