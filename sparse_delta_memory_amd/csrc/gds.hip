// The backward movers on gfx950 (GDS, GWR and PA below). GDS: the backward of the read gather q0[t] = sum_r q_w[t, r]
// M0[q_idx[t, r]] for the chunks of one step (page "sparse_delta_memory/cuda/mover_da2_cuda.py": the GDS part of the module
// docstring and the comment of its scatter role).
//
// Every kernel here works in teams of TEAM lanes (16, 32 or 64), one item per team: rows of up to
// 128 columns leave most of a 64-lane wave idle, so narrow teams put several items' memory round
// trips in flight per wave. A team sum is a butterfly of xor shuffles inside the team.
//
// gds_dots_kernel: d_q_w[t, r] = <gr[t], M0[q_idx[t, r]]>, token order, one team per 4 reads of a
// token (their rows in flight together), a team sum per dot (no atomics).
// gds_scatter_kernel: the gradient rows in sorted order, one team per position of the Q-only rows:
// at a valid group FIRST the team walks the group's members in sorted order (TEAM records and
// weights at a time, 4 or 8 gradient rows in flight), acc = fma(q_w, gr[t], acc) from +0, and at
// LAST adds acc to grad[slot] with one read-modify-write (the team is that row's only writer in the
// launch, so the result is deterministic). With a workspace, a group of more than 32 members is
// walked in 32-member segments by separate teams; the last to finish adds their partial rows in
// segment order and makes the read-modify-write (the same sums whichever finishes last).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdm.h"
#include "sdm_device.hpp"
#include "sdm_launch.hpp"

namespace sdm {
namespace {

struct GdsArgs {
    const void* bank;       // M0, float32 or bf16 rows
    const void* q_idx;      // int32 or int64 absolute ids
    const void* q_w;        // float32 or bf16
    const uint32_t* spay_q;
    const float* gr;
    float* d_q_w;
    void* grad;
    float* part;       // split groups (NULL: not split): two partial rows per block of kSplitSeg positions
    int* cnt;          // per block of kSplitSeg positions (a split group's FIRST): arrival counter, zero between calls
    int* meta;         // per block of kSplitSeg positions: the group's segment count
    int64_t rows, chunk0, row0;
    int P, C, R, hd, first_partial, valid_last, id64, vbf, bank_bf16, grad_bf16;
};

// Long groups (GDS read groups, PA write groups; with a workspace) are walked in segments of SEG =
// 32 members (16-member segments measured slower on skewed slots: twice the partial rows for the
// last segment to add). The last in-group distance that still marks a segment start: the distance
// field saturates at 4095.
constexpr int kSplitSeg = 32;
template <int SEG>
constexpr int split_seg_limit() { return (4095 / SEG) * SEG; }
// Workspace slots, by step-wide row position G (stream p's position j is p * (its row length) + j):
// a split group has more than SEG members, so at most one split group's FIRST falls in each
// aligned block of SEG positions (its counter and segment count), and at most two segment starts
// (the first segment of a group starting there, a later one of the group running through): two
// partial rows per block.
template <int SEG>
__device__ __forceinline__ int64_t split_group_slot(int64_t g_first) { return g_first / SEG; }
template <int SEG>
__device__ __forceinline__ int64_t split_part_row(int64_t g_start, bool first_segment) {
    return 2 * (g_start / SEG) + (first_segment ? 0 : 1);
}

// The combining team's sum of a split group's partial rows (columns col .. col + 3), in segment
// order from +0: device-scope atomic loads (the partials come from other XCDs), four segments'
// loads in flight together.
template <int SEG>
__device__ __forceinline__ float4 sum_partials(const float* part, int64_t g_first, int nseg, int hd, int col) {
    float4 tot = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int sg0 = 0; sg0 < nseg; sg0 += 4) {
        float4 pv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int sg = min(sg0 + b, nseg - 1);   // (past the count: the last segment again, not added)
            const float* pp = part + split_part_row<SEG>(g_first + static_cast<int64_t>(sg) * SEG, sg == 0) * hd + col;
            pv[b].x = __hip_atomic_load(pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pv[b].y = __hip_atomic_load(pp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pv[b].z = __hip_atomic_load(pp + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            pv[b].w = __hip_atomic_load(pp + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (sg0 + b < nseg) {
                tot.x = tot.x + pv[b].x;
                tot.y = tot.y + pv[b].y;
                tot.z = tot.z + pv[b].z;
                tot.w = tot.w + pv[b].w;
            }
        }
    }
    return tot;
}

constexpr int kGdsThreads = 256;
constexpr int kGdsWaves = kGdsThreads / kWave;

__device__ __forceinline__ int64_t gds_id(const GdsArgs& a, int64_t i) {
    return a.id64 ? static_cast<const int64_t*>(a.q_idx)[i] : static_cast<const int32_t*>(a.q_idx)[i];
}

// Four columns col .. col + 3 of a row as floats (float32 or bf16 storage; hd a multiple of 4).
__device__ __forceinline__ float4 load4(const void* base, int bf, int64_t row, int hd, int col) {
    if (bf) {
        const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + row * hd + col);
        return make_float4(bf16_bits_to_f32(w.x & 0xFFFFu), bf16_bits_to_f32(w.x >> 16), bf16_bits_to_f32(w.y & 0xFFFFu),
                           bf16_bits_to_f32(w.y >> 16));
    }
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + row * hd + col);
}

// load4 with the row dtype fixed at compile time: a run-time dtype branch around each load makes
// the compiler wait for every load before the next (the bf16 path widens its data at once), which
// serialises the rows a loop means to keep in flight together.
template <bool BF>
__device__ __forceinline__ float4 load4t(const void* base, int64_t row, int hd, int col) {
    if constexpr (BF) {
        const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + row * hd + col);
        return make_float4(bf16_bits_to_f32(w.x & 0xFFFFu), bf16_bits_to_f32(w.x >> 16), bf16_bits_to_f32(w.y & 0xFFFFu),
                           bf16_bits_to_f32(w.y >> 16));
    } else {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + row * hd + col);
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// Sum over a team of TEAM lanes (an aligned group of 16 or 32 lanes, or the whole wave).
template <int TEAM>
__device__ __forceinline__ float team_sum(float v) {
#pragma unroll
    for (int d = TEAM / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

// A ballot restricted to the lane's team, shifted so that bit i is team lane i.
template <int TEAM>
__device__ __forceinline__ uint64_t team_bits(uint64_t ballot, int lane) {
    return TEAM == kWave ? ballot : (ballot >> (lane / TEAM * TEAM)) & ((1ull << TEAM) - 1ull);
}

// A 64-bit value of another lane (src counted within segments of `width` lanes).
__device__ __forceinline__ int64_t shfl64(int64_t v, int src, int width = kWave) {
    const int lo = __shfl(static_cast<int>(static_cast<uint64_t>(v) & 0xFFFFFFFFull), src, width);
    const int hi = __shfl(static_cast<int>(static_cast<uint64_t>(v) >> 32), src, width);
    return static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32 | static_cast<uint32_t>(lo));
}

constexpr int kDotReads = 4;   // reads whose rows are in flight together
constexpr int kWalkRows = 8;   // member gradient rows in flight together

// TEAM: lanes per item (32 for rows of up to 128 columns: two items per wave). BBF: bf16 bank rows.
template <int TEAM, bool BBF>
__global__ void __launch_bounds__(kGdsThreads) gds_dots_kernel(GdsArgs a) {
    const int wv = static_cast<int>(threadIdx.x) / kWave;
    const int lane = static_cast<int>(lane_id());
    const int tl = lane % TEAM;
    const int groups = (a.R + kDotReads - 1) / kDotReads;   // read groups per token
    const int64_t item = (static_cast<int64_t>(blockIdx.x) * kGdsWaves + wv) * (kWave / TEAM) + lane / TEAM;   // (p, t, read group)
    if (item >= static_cast<int64_t>(a.P) * a.C * groups) return;
    const int64_t tok = item / groups;
    const int r0 = static_cast<int>(item % groups) * kDotReads;
    const int nr = min(kDotReads, a.R - r0);
    const int p = static_cast<int>(tok / a.C), t = static_cast<int>(tok % a.C);
    const int64_t c = a.chunk0 + p;
    const int tv = c >= a.first_partial ? a.valid_last : a.C;
    const int64_t eo = (c * a.C + t) * a.R + r0;   // the group's first Q entry
    if (t >= tv) {   // masked: no reads, dots 0
        if (tl < nr) a.d_q_w[eo + tl] = 0.0f;
        return;
    }
    const int64_t grow = a.row0 + static_cast<int64_t>(p) * a.C + t;
    const int64_t my_id = tl < nr ? gds_id(a, eo + tl) : -1;
    int64_t s[kDotReads];
    bool ok[kDotReads];
#pragma unroll
    for (int u = 0; u < kDotReads; ++u) {
        s[u] = shfl64(my_id, min(u, nr - 1), TEAM);
        ok[u] = u < nr && s[u] >= 0 && s[u] < a.rows;   // (a slot outside the bank contributes nothing)
    }
    float acc[kDotReads] = {};
    for (int col = 4 * tl; col < a.hd; col += 4 * TEAM) {
        const float4 g = load4(a.gr, 0, grow, a.hd, col);
        float4 m[kDotReads];
#pragma unroll
        for (int u = 0; u < kDotReads; ++u) m[u] = load4t<BBF>(a.bank, ok[u] ? s[u] : 0, a.hd, col);
#pragma unroll
        for (int u = 0; u < kDotReads; ++u) {
            if (ok[u]) acc[u] = fmaf(g.w, m[u].w, fmaf(g.z, m[u].z, fmaf(g.y, m[u].y, fmaf(g.x, m[u].x, acc[u]))));
        }
    }
#pragma unroll
    for (int u = 0; u < kDotReads; ++u) {
        const float d = team_sum<TEAM>(acc[u]);
        if (tl == 0 && u < nr) a.d_q_w[eo + u] = d;
    }
}

// TEAM lanes per Q-row position (two or four positions per wave for narrow rows). ONE: each lane's
// NCB 4-column blocks (cb * 4 TEAM + 4 lane) cover the row, else (NCB = 1) a column loop over the
// row, the members walked again per block of 4 TEAM columns.
template <bool ONE, int TEAM, int NCB>
__global__ void __launch_bounds__(kGdsThreads) gds_scatter_kernel(GdsArgs a) {
    constexpr int kRows = NCB == 1 ? kWalkRows : 4;   // member gradient rows in flight together
    constexpr int SEG = kSplitSeg;   // members per segment of a split group
    const int wv = static_cast<int>(threadIdx.x) / kWave;
    const int lane = static_cast<int>(lane_id());
    const int tl = lane % TEAM;
    const int n = a.C * a.R;
    const int64_t pos = (static_cast<int64_t>(blockIdx.x) * kGdsWaves + wv) * (kWave / TEAM) + lane / TEAM;   // p * C * R + j
    if (pos >= static_cast<int64_t>(a.P) * n) return;
    const int p = static_cast<int>(pos / n), j = static_cast<int>(pos % n);
    const int64_t c = a.chunk0 + p;
    const uint32_t* row = a.spay_q + c * n;
    const uint32_t e0 = row[j];
    if (e0 & kInvalid) return;
    // Work starts at a valid group's FIRST and, when long groups are split, at every SEG-th
    // member (distance counts the group's valid entries before this one).
    const bool split = a.part != nullptr;
    const int dist = static_cast<int>((e0 >> kDistShift) & kDistMax);
    const bool first = (e0 & kFirst) != 0u;
    if (!first && (!split || dist % SEG != 0 || dist > split_seg_limit<SEG>())) return;
    const bool unbounded = !split || dist == split_seg_limit<SEG>();   // the last segment start runs to LAST
    const int64_t qbase = c * n;   // entry-order Q index of (t, lane) is t * R + lane
    auto entry = [&](uint32_t el) { return static_cast<int64_t>((el >> kTokShift) & 0xFFu) * a.R + (el & 0xFFu); };
    const int64_t slot = gds_id(a, qbase + entry(e0));   // (every member, so every segment, reads it)
    if (slot < 0 || slot >= a.rows) return;
    const int64_t grow0 = a.row0 + static_cast<int64_t>(p) * a.C;
    // One read-modify-write of 4 columns of the slot's row (this team is the row's only writer).
    auto add_row = [&](int col, float4 v) {
        if (a.grad_bf16) {
            uint2* gp = reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.grad) + slot * a.hd + col);
            const uint2 o = *gp;
            const float x = bf16_bits_to_f32(o.x & 0xFFFFu) + v.x, y = bf16_bits_to_f32(o.x >> 16) + v.y;
            const float z = bf16_bits_to_f32(o.y & 0xFFFFu) + v.z, u = bf16_bits_to_f32(o.y >> 16) + v.w;
            *gp = make_uint2(f32_to_bf16_rne(x) | f32_to_bf16_rne(y) << 16, f32_to_bf16_rne(z) | f32_to_bf16_rne(u) << 16);
        } else {
            float4* gp = reinterpret_cast<float4*>(static_cast<float*>(a.grad) + slot * a.hd + col);
            const float4 o = *gp;
            *gp = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
        }
    };
    const int64_t prow = static_cast<int64_t>(p) * n;
    bool last_seen = false;
    for (int col0 = 0; col0 < (ONE ? 1 : a.hd); col0 += 4 * TEAM) {
        float4 acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        bool done = false;
        int taken = 0;
        // The members in sorted order, TEAM records at a time (team lane l: member m0 + l), their
        // gradient rows kRows at a time; the sum runs over the members in order from +0.
        for (int m0 = j; !done && m0 < n; m0 += TEAM) {
            const int budget = unbounded ? TEAM : min(TEAM, SEG - taken);   // members still in the segment
            const int m = m0 + tl;
            const uint32_t el = m < n ? row[m] : (kFirst | kLast | kInvalid);
            const int tk = static_cast<int>((el >> kTokShift) & 0xFFu);
            const bool in = m < n && !(el & kInvalid);
            const float w = in ? load_val(a.q_w, qbase + entry(el), a.vbf) : 0.0f;
            const uint64_t lastm = team_bits<TEAM>(__ballot(tl < budget && (el & kLast) != 0u), lane);
            const int cnt = lastm != 0ull ? __builtin_ctzll(lastm) + 1 : budget;   // (LAST included)
            last_seen = lastm != 0ull;
            taken += cnt;
            done = last_seen || (!unbounded && taken == SEG);
            for (int k0 = 0; k0 < cnt; k0 += kRows) {
                float wk[kRows];
                float4 g[kRows][NCB];
#pragma unroll
                for (int u = 0; u < kRows; ++u) {
                    const int kk = min(k0 + u, cnt - 1);
                    wk[u] = __shfl(w, kk, TEAM);
                    const int t = __shfl(tk, kk, TEAM);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const int col = col0 + cb * 4 * TEAM + 4 * tl;
                        // (rows past the group's end are not loaded: most groups have one member)
                        g[u][cb] = (col < a.hd && k0 + u < cnt) ? load4(a.gr, 0, grow0 + t, a.hd, col)
                                                                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    }
                }
#pragma unroll
                for (int u = 0; u < kRows; ++u) {
                    if (k0 + u < cnt) {
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) {
                            acc[cb].x = fmaf(wk[u], g[u][cb].x, acc[cb].x);
                            acc[cb].y = fmaf(wk[u], g[u][cb].y, acc[cb].y);
                            acc[cb].z = fmaf(wk[u], g[u][cb].z, acc[cb].z);
                            acc[cb].w = fmaf(wk[u], g[u][cb].w, acc[cb].w);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int col = col0 + cb * 4 * TEAM + 4 * tl;
            if (col >= a.hd) continue;
            if (first && last_seen) {   // the whole group in one segment
                add_row(col, acc[cb]);
            } else {   // a segment of a split group: its partial row (device-scope stores, see below)
                float* part = a.part + split_part_row<SEG>(prow + j, dist == 0) * a.hd + col;
                __hip_atomic_store(part, acc[cb].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(part + 1, acc[cb].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(part + 2, acc[cb].z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(part + 3, acc[cb].w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (first && last_seen) return;
    // Split group: the last segment to arrive adds the partial rows in segment order and updates
    // the row. Segments run in blocks on different XCDs, whose L2 caches are not coherent with each
    // other: partials and the segment count are device-scope atomic stores, the wave waits for
    // their completion before it adds to the arrival counter (a device-scope atomic), and the
    // combining wave reads them with device-scope atomic loads after seeing the last arrival.
    const int first_pos = j - dist;
    const int64_t gslot = split_group_slot<SEG>(prow + first_pos);
    const int seg = dist / SEG;
    if (last_seen && tl == 0) __hip_atomic_store(a.meta + gslot, seg + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the stores above have completed
    // The segment holding LAST adds 1 - (segments), every other adds 1: the counter returns to 0
    // exactly at the last arrival (and is left at 0 for the next call).
    const int delta = last_seen ? -seg : 1;
    int after = 0;
    if (tl == 0) after = atomicAdd(a.cnt + gslot, delta) + delta;
    after = __shfl(after, 0, TEAM);
    if (after != 0) return;
    // (clamped to the segment starts the row holds, so no read can leave the workspace)
    const int nseg = min(max(__hip_atomic_load(a.meta + gslot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), 0),
                         (n - first_pos + SEG - 1) / SEG);
    for (int col0 = 0; col0 < (ONE ? 1 : a.hd); col0 += 4 * TEAM) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int col = col0 + cb * 4 * TEAM + 4 * tl;
            if (col >= a.hd) continue;
            const float4 tot = sum_partials<SEG>(a.part, prow + first_pos, nseg, a.hd, col);
            add_row(col, tot);
        }
    }
}

// GWR (page "sparse_delta_memory/cuda/pa_dc_cuda.py", module docstring: the GWR gather of the
// deterministic backward) for the tokens of one step: d_dv[t] = sum_n w[t, n] grad[k_idx[t, n]]
// (entries in order, fma chain from +0) and d_k_pd[t, n] = <dv[t], grad[k_idx[t, n]]>. One team
// per token: each lane holds 4 columns of every 4 * TEAM (hd <= 1024) of dv[t] and of the d_dv sum;
// the token's ids and weights are loaded one per lane, then its gradient rows a few at a time.
struct GwrArgs {
    const void* grad;
    const void* k_idx;
    const float* w;
    const float* dv;
    float* d_dv;
    float* d_k_pd;
    int64_t rows, chunk0, row0;
    int P, C, W, hd, first_partial, valid_last, id64, grad_bf16;
};

// NCB: the blocks of 4 * TEAM columns a lane's registers hold (with 64-lane teams 1, 2 or 4: hd <=
// 256, 512, 1024), so that narrow rows keep few registers and many waves per SIMD.
template <int NCB, int GR, int TEAM, bool GBF>
__global__ void __launch_bounds__(kGdsThreads) gwr_kernel(GwrArgs a) {
    const int wv = static_cast<int>(threadIdx.x) / kWave;
    const int lane = static_cast<int>(lane_id());
    const int tl = lane % TEAM;   // lane in the token's team (TEAM lanes per token)
    const int64_t tok = (static_cast<int64_t>(blockIdx.x) * kGdsWaves + wv) * (kWave / TEAM) + lane / TEAM;
    if (tok >= static_cast<int64_t>(a.P) * a.C) return;
    const int p = static_cast<int>(tok / a.C), t = static_cast<int>(tok % a.C);
    const int64_t c = a.chunk0 + p;
    const int tv = c >= a.first_partial ? a.valid_last : a.C;
    const int64_t eo = (c * a.C + t) * a.W;
    const int64_t vrow = a.row0 + static_cast<int64_t>(p) * a.C + t;
    if (t >= tv) {   // masked: zeros, nothing read
        if (a.d_k_pd != nullptr) {
            for (int n = tl; n < a.W; n += TEAM) a.d_k_pd[eo + n] = 0.0f;
        }
        if (a.d_dv != nullptr) {
            for (int col = 4 * tl; col < a.hd; col += 4 * TEAM)
                *reinterpret_cast<float4*>(a.d_dv + vrow * a.hd + col) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        return;
    }
    float4 v[NCB], acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = cb * 4 * TEAM + 4 * tl;
        v[cb] = col < a.hd ? *reinterpret_cast<const float4*>(a.dv + vrow * a.hd + col) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        acc[cb] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    for (int nb = 0; nb < a.W; nb += TEAM) {
        const int nr = min(TEAM, a.W - nb);
        const int64_t my_id = tl < nr ? (a.id64 ? static_cast<const int64_t*>(a.k_idx)[eo + nb + tl]
                                                  : static_cast<const int32_t*>(a.k_idx)[eo + nb + tl])
                                        : -1;
        const float my_w = tl < nr ? a.w[eo + nb + tl] : 0.0f;
        for (int n0 = 0; n0 < nr; n0 += GR) {
            int64_t s[GR];
            bool ok[GR];
            float wu[GR], part[GR];
#pragma unroll
            for (int u = 0; u < GR; ++u) {
                const int src = min(n0 + u, nr - 1);
                s[u] = shfl64(my_id, src, TEAM);
                wu[u] = __shfl(my_w, src, TEAM);
                ok[u] = n0 + u < nr && s[u] >= 0 && s[u] < a.rows;   // (a slot outside the bank contributes nothing)
                part[u] = 0.0f;
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int col = cb * 4 * TEAM + 4 * tl;
                if (col >= a.hd) break;
                float4 g[GR];
#pragma unroll
                for (int u = 0; u < GR; ++u) g[u] = load4t<GBF>(a.grad, ok[u] ? s[u] : 0, a.hd, col);
#pragma unroll
                for (int u = 0; u < GR; ++u) {
                    if (ok[u]) {
                        acc[cb].x = fmaf(wu[u], g[u].x, acc[cb].x);
                        acc[cb].y = fmaf(wu[u], g[u].y, acc[cb].y);
                        acc[cb].z = fmaf(wu[u], g[u].z, acc[cb].z);
                        acc[cb].w = fmaf(wu[u], g[u].w, acc[cb].w);
                        part[u] = fmaf(v[cb].w, g[u].w, fmaf(v[cb].z, g[u].z, fmaf(v[cb].y, g[u].y, fmaf(v[cb].x, g[u].x, part[u]))));
                    }
                }
            }
            if (a.d_k_pd != nullptr) {
#pragma unroll
                for (int u = 0; u < GR; ++u) {
                    const float d = team_sum<TEAM>(part[u]);
                    if (tl == 0 && n0 + u < nr) a.d_k_pd[eo + nb + n0 + u] = d;
                }
            }
        }
    }
    if (a.d_dv != nullptr) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int col = cb * 4 * TEAM + 4 * tl;
            if (col < a.hd) *reinterpret_cast<float4*>(a.d_dv + vrow * a.hd + col) = acc[cb];
        }
    }
}

// PA (page "sparse_delta_memory/cuda/pa_dc_cuda.py", module docstring: Phase A of the deterministic
// backward, the backward of DW) for the chunks of one step. A padding entry writes its zeros; a valid
// group's gradient row gdw and snapshot row (hd <= 1024: 4 columns of every 4 * TEAM per lane) give
// <gdw, snap>; its members, in sorted order, give acc = fma(-beta k_eff, d_dva[t], acc) from +0,
// d_k_eff[e] = -beta <d_dva[t], snap> and grad_g_decay[e] = cpe <gdw, snap>; then grad[s] =
// fma(gdw, cpe, acc) and bank[s] = snap. A long group (more than 32 members, with a workspace) is
// walked in segments of 32 members whose partial sums are added in segment order: one writer per row
// and per entry, the same bits run to run.
struct PaArgs {
    void* grad;
    void* bank;
    const void* snap;
    const uint4* krec;
    const void* k_eff;
    const float* beta;
    const float* d_dva;
    float* g_decay;
    float* d_k_eff;
    float* part;       // split groups (NULL: not split): two partial rows per block of kSplitSeg positions
    int* cnt;          // per block of kSplitSeg positions (a split group's FIRST): arrival counter, zero between calls
    int* meta;         // per block of kSplitSeg positions: the group's segment count
    int64_t rows, chunk0, row0, snap_row0;
    int P, C, W, CW, hd, vbf, grad_bf16, bank_bf16;
};

constexpr int kPaMembers = 4;   // member token rows in flight together

__device__ __forceinline__ void store4(void* base, int bf, int64_t row, int hd, int col, float4 v) {
    if (bf) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + row * hd + col) =
            make_uint2(f32_to_bf16_rne(v.x) | f32_to_bf16_rne(v.y) << 16, f32_to_bf16_rne(v.z) | f32_to_bf16_rne(v.w) << 16);
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(base) + row * hd + col) = v;
    }
}

// One team per K-row position that starts work: a group's FIRST or, with a workspace, every SEG-th
// member of a longer group. The team walks its members in sorted order (TEAM records at a time,
// kPaMembers token rows in flight): per member d_k_eff and g_decay, and acc = fma(sc, d_dva[tok], acc)
// from +0. A group in one segment then writes grad = fma(gdw, cpe, acc) and restores the bank row;
// a split group's segments publish their partial rows, and the last to arrive adds them in segment
// order and writes the rows (the same sums whichever segment arrives last).
// GBF, BBF: bf16 gradient rows, bf16 bank (and snapshot) rows.
template <int NCB, int TEAM, bool GBF, bool BBF>
__global__ void __launch_bounds__(kGdsThreads) pa_kernel(PaArgs a) {
    constexpr int SEG = kSplitSeg;   // members per segment of a split group
    const int wv = static_cast<int>(threadIdx.x) / kWave;
    const int lane = static_cast<int>(lane_id());
    const int tl = lane % TEAM;   // lane in the team (TEAM lanes per K-row position)
    const int64_t pos = (static_cast<int64_t>(blockIdx.x) * kGdsWaves + wv) * (kWave / TEAM) + lane / TEAM;   // p * CW + j
    if (pos >= static_cast<int64_t>(a.P) * a.CW) return;
    const int p = static_cast<int>(pos / a.CW), j = static_cast<int>(pos % a.CW);
    const int64_t c = a.chunk0 + p;
    const uint4* kr = a.krec + c * a.CW;
    const uint4 r0 = kr[j];
    auto eidx = [&](uint32_t el) {   // entry-order index [N, C, W] of a K-row element
        return (c * a.C + static_cast<int64_t>((el >> kTokShift) & 0xFFu)) * a.W + (el & 0xFFu);
    };
    if (r0.x & kInvalid) {   // padding: its outputs are zero
        if (tl == 0) {
            if (a.g_decay != nullptr) a.g_decay[eidx(r0.x)] = 0.0f;
            if (a.d_k_eff != nullptr) a.d_k_eff[eidx(r0.x)] = 0.0f;
        }
        return;
    }
    const bool split = a.part != nullptr;
    const int dist = static_cast<int>((r0.x >> kDistShift) & kDistMax);   // valid K entries before, in the group
    const bool first = (r0.x & kFirst) != 0u;
    if (!first && (!split || dist % SEG != 0 || dist > split_seg_limit<SEG>())) return;   // a member another wave walks
    const bool unbounded = !split || dist == split_seg_limit<SEG>();   // the last segment start runs to LAST
    const int first_pos = j - dist;                          // the group's FIRST (its snapshot row)
    const int64_t slot = static_cast<int64_t>(r0.y);
    const bool in = slot < a.rows;   // (a slot outside the bank: zero rows, nothing written)
    const float cpe = __uint_as_float(r0.w);   // (every member's record holds the group's cpe)
    const int64_t srow = a.snap_row0 + static_cast<int64_t>(p) * a.CW + first_pos;
    float4 gdw[NCB], sn[NCB], acc[NCB];
    float part0 = 0.0f;
    // (every load issued, from row 0 / the row's last 4 columns where its value is not used, so
    // that the group's rows are in flight together)
    const int64_t slot_c = in ? slot : 0;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = cb * 4 * TEAM + 4 * tl;
        gdw[cb] = load4t<GBF>(a.grad, slot_c, a.hd, min(col, a.hd - 4));
        sn[cb] = load4t<BBF>(a.snap, srow, a.hd, min(col, a.hd - 4));
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = cb * 4 * TEAM + 4 * tl;
        const bool con = in && col < a.hd;
        if (!con) {
            gdw[cb] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            sn[cb] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        acc[cb] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        part0 = fmaf(gdw[cb].w, sn[cb].w, fmaf(gdw[cb].z, sn[cb].z, fmaf(gdw[cb].y, sn[cb].y, fmaf(gdw[cb].x, sn[cb].x, part0))));
    }
    const float dot0 = team_sum<TEAM>(part0);
    const int64_t grow0 = a.row0 + static_cast<int64_t>(p) * a.C;
    bool done = false, last_seen = false;
    int taken = 0;
    for (int m0 = j; !done && m0 < a.CW; m0 += TEAM) {   // members TEAM records at a time, in sorted order
        const int budget = unbounded ? TEAM : min(TEAM, SEG - taken);   // members this segment may still take
        const int m = m0 + tl;
        const uint32_t el = m < a.CW ? kr[m].x : (kFirst | kLast | kInvalid);
        const int tk = static_cast<int>((el >> kTokShift) & 0xFFu);
        const bool valid = m < a.CW && !(el & kInvalid);
        const float nb = valid ? -a.beta[c * a.C + tk] : 0.0f;
        const float w = valid ? nb * load_val(a.k_eff, eidx(el), a.vbf) : 0.0f;
        const int64_t ei = valid ? eidx(el) : 0;
        const uint64_t lastm = team_bits<TEAM>(__ballot(tl < budget && (el & kLast) != 0u), lane);
        const int cnt = lastm != 0ull ? __builtin_ctzll(lastm) + 1 : budget;   // (LAST included)
        last_seen = lastm != 0ull;
        taken += cnt;
        done = last_seen || (!unbounded && taken == SEG);
        for (int k0 = 0; k0 < cnt; k0 += kPaMembers) {
            float4 d[kPaMembers][NCB];
            float wk[kPaMembers], bk[kPaMembers];
            int64_t ek[kPaMembers];
#pragma unroll
            for (int u = 0; u < kPaMembers; ++u) {
                const int kk = min(k0 + u, cnt - 1);
                wk[u] = __shfl(w, kk, TEAM);
                bk[u] = __shfl(nb, kk, TEAM);
                ek[u] = shfl64(ei, kk, TEAM);
                const int t = __shfl(tk, kk, TEAM);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const int col = cb * 4 * TEAM + 4 * tl;
                    // (rows past the group's end are not loaded: most groups have one member)
                    d[u][cb] = (col < a.hd && k0 + u < cnt) ? load4(a.d_dva, 0, grow0 + t, a.hd, col)
                                                            : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                }
            }
#pragma unroll
            for (int u = 0; u < kPaMembers; ++u) {
                if (k0 + u >= cnt) break;
                float part = 0.0f;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    acc[cb].x = fmaf(wk[u], d[u][cb].x, acc[cb].x);
                    acc[cb].y = fmaf(wk[u], d[u][cb].y, acc[cb].y);
                    acc[cb].z = fmaf(wk[u], d[u][cb].z, acc[cb].z);
                    acc[cb].w = fmaf(wk[u], d[u][cb].w, acc[cb].w);
                    part = fmaf(d[u][cb].w, sn[cb].w, fmaf(d[u][cb].z, sn[cb].z, fmaf(d[u][cb].y, sn[cb].y, fmaf(d[u][cb].x, sn[cb].x, part))));
                }
                const float dot = team_sum<TEAM>(part);
                if (tl == 0) {
                    if (a.d_k_eff != nullptr) a.d_k_eff[ek[u]] = bk[u] * dot;
                    if (a.g_decay != nullptr) a.g_decay[ek[u]] = cpe * dot0;
                }
            }
        }
    }
    if (first && last_seen) {   // the whole group in one segment
        if (!in) return;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int col = cb * 4 * TEAM + 4 * tl;
            if (col >= a.hd) break;
            const float4 g = make_float4(fmaf(gdw[cb].x, cpe, acc[cb].x), fmaf(gdw[cb].y, cpe, acc[cb].y),
                                         fmaf(gdw[cb].z, cpe, acc[cb].z), fmaf(gdw[cb].w, cpe, acc[cb].w));
            store4(a.grad, a.grad_bf16, slot, a.hd, col, g);
            if (a.bank != nullptr) store4(a.bank, a.bank_bf16, slot, a.hd, col, sn[cb]);
        }
        return;
    }
    // Split group: publish this segment's partial; the last segment to arrive combines the partials
    // in segment order. The segments run in blocks on different XCDs, whose L2 caches are not
    // coherent with each other: the partial and the segment count are written with device-scope
    // atomic stores, the wave waits until they have completed, and only then adds to the arrival
    // counter (a device-scope atomic); the combining wave reads them with device-scope atomic loads
    // after seeing the last arrival.
    const int64_t prow = static_cast<int64_t>(p) * a.CW;
    const int64_t gslot = split_group_slot<SEG>(prow + first_pos);
    float* part = a.part + split_part_row<SEG>(prow + j, dist == 0) * a.hd;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = cb * 4 * TEAM + 4 * tl;
        if (col < a.hd) {
            __hip_atomic_store(part + col, acc[cb].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(part + col + 1, acc[cb].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(part + col + 2, acc[cb].z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(part + col + 3, acc[cb].w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    const int seg = dist / SEG;
    // The segment holding LAST publishes the segment count.
    if (last_seen && tl == 0) __hip_atomic_store(a.meta + gslot, seg + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the stores above have completed
    // The segment holding LAST adds 1 - (segments), every other adds 1: the counter returns to 0
    // exactly at the last arrival (and is left at 0 for the next call).
    const int delta = last_seen ? -seg : 1;
    int after = 0;
    if (tl == 0) after = atomicAdd(a.cnt + gslot, delta) + delta;
    after = __shfl(after, 0, TEAM);
    if (after != 0) return;
    // (clamped to the segment starts the row holds, so no read can leave the workspace)
    const int nseg = min(max(__hip_atomic_load(a.meta + gslot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), 0),
                         (a.CW - first_pos + SEG - 1) / SEG);
    float4 tot[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = cb * 4 * TEAM + 4 * tl;
        tot[cb] = col < a.hd ? sum_partials<SEG>(a.part, prow + first_pos, nseg, a.hd, col) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    if (!in) return;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = cb * 4 * TEAM + 4 * tl;
        if (col >= a.hd) break;
        const float4 g = make_float4(fmaf(gdw[cb].x, cpe, tot[cb].x), fmaf(gdw[cb].y, cpe, tot[cb].y),
                                     fmaf(gdw[cb].z, cpe, tot[cb].z), fmaf(gdw[cb].w, cpe, tot[cb].w));
        store4(a.grad, a.grad_bf16, slot, a.hd, col, g);
        if (a.bank != nullptr) store4(a.bank, a.bank_bf16, slot, a.hd, col, sn[cb]);
    }
}

}  // namespace

GdsWorkspace gds_workspace_layout(const sdm_gds_io* io) {
    const size_t pos = static_cast<size_t>(io->P) * static_cast<size_t>(io->C) * static_cast<size_t>(io->R);
    const size_t blocks = (pos + kSplitSeg - 1) / kSplitSeg;
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    GdsWorkspace w;
    w.cnt_off = 0;
    w.meta_off = up(blocks * sizeof(int));
    w.part_off = w.meta_off + up(blocks * sizeof(int));
    w.total = w.part_off + up(2 * blocks * static_cast<size_t>(io->hd) * sizeof(float));
    return w;
}

hipError_t gds_launch(const sdm_gds_io* io, int64_t ti, hipStream_t st) {
    GdsArgs a;
    a.bank = io->bank;
    a.q_idx = io->q_idx;
    a.q_w = io->q_w;
    a.spay_q = reinterpret_cast<const uint32_t*>(io->spay_q);
    a.gr = io->gr;
    a.d_q_w = io->d_q_w;
    a.grad = io->grad;
    a.rows = io->rows;
    a.chunk0 = ti * io->P;
    a.row0 = ti * io->step_rows;
    a.P = io->P;
    a.C = io->C;
    a.R = io->R;
    a.hd = io->hd;
    a.first_partial = io->first_partial;
    a.valid_last = io->valid_last;
    a.id64 = io->idx_bytes == 8;
    a.vbf = io->val_bytes == 2;
    a.bank_bf16 = io->bank_dtype == SDM_BF16;
    a.grad_bf16 = io->grad_dtype == SDM_BF16;
    a.part = nullptr;
    a.cnt = nullptr;
    a.meta = nullptr;
    if (io->workspace != nullptr) {
        const GdsWorkspace w = gds_workspace_layout(io);
        char* ws = static_cast<char*>(io->workspace);
        a.part = reinterpret_cast<float*>(ws + w.part_off);
        a.cnt = reinterpret_cast<int*>(ws + w.cnt_off);
        a.meta = reinterpret_cast<int*>(ws + w.meta_off);
    }
    const int64_t toks = static_cast<int64_t>(io->P) * io->C;
    const int64_t poss = toks * io->R;
    const int64_t items = toks * ((io->R + kDotReads - 1) / kDotReads);   // (token, read group) items
    // Rows of up to 128 columns: 32-lane teams, two items (positions) per wave.
    const bool half = io->hd <= 4 * 32;
    const int64_t per_block = static_cast<int64_t>(kGdsWaves) * (half ? 2 : 1);
    void* kargs[] = {&a};
    hipError_t e = hipSuccess;
    if (io->d_q_w != nullptr) {
        const bool bbf = io->bank_dtype == SDM_BF16;
        e = hipLaunchKernel(half ? (bbf ? reinterpret_cast<const void*>(&gds_dots_kernel<32, true>)
                                        : reinterpret_cast<const void*>(&gds_dots_kernel<32, false>))
                                 : (bbf ? reinterpret_cast<const void*>(&gds_dots_kernel<kWave, true>)
                                        : reinterpret_cast<const void*>(&gds_dots_kernel<kWave, false>)),
                            dim3(static_cast<unsigned>((items + per_block - 1) / per_block)), dim3(kGdsThreads), kargs, 0, st);
        if (e != hipSuccess) return e;
    }
    if (io->grad != nullptr) {
        // (the scatter: 16-lane teams of 8 columns per lane, four positions per wave)
        const int64_t per_block_s = static_cast<int64_t>(kGdsWaves) * (half ? 4 : 1);
        e = hipLaunchKernel(half ? reinterpret_cast<const void*>(&gds_scatter_kernel<true, 16, 2>)
                            : io->hd <= 4 * kWave ? reinterpret_cast<const void*>(&gds_scatter_kernel<true, kWave, 1>)
                                                  : reinterpret_cast<const void*>(&gds_scatter_kernel<false, kWave, 1>),
                            dim3(static_cast<unsigned>((poss + per_block_s - 1) / per_block_s)), dim3(kGdsThreads), kargs, 0, st);
    }
    return e;
}

namespace {

// The GWR and PA kernels for a head dim and the rows' dtypes: rows of up to 128 columns take
// 32-lane (GWR) or 16-lane (PA) teams, wider rows a wave per item with 1, 2 or 4 column blocks.
template <bool GBF>
const void* gwr_fn(int hd) {
    return hd <= 4 * 32 ? reinterpret_cast<const void*>(&gwr_kernel<1, 8, 32, GBF>)
         : hd <= 256    ? reinterpret_cast<const void*>(&gwr_kernel<1, 8, kWave, GBF>)
         : hd <= 512    ? reinterpret_cast<const void*>(&gwr_kernel<2, 4, kWave, GBF>)
                        : reinterpret_cast<const void*>(&gwr_kernel<4, 4, kWave, GBF>);
}

template <bool GBF, bool BBF>
const void* pa_fn(int hd) {
    return hd <= 4 * 32 ? reinterpret_cast<const void*>(&pa_kernel<2, 16, GBF, BBF>)
         : hd <= 256    ? reinterpret_cast<const void*>(&pa_kernel<1, kWave, GBF, BBF>)
         : hd <= 512    ? reinterpret_cast<const void*>(&pa_kernel<2, kWave, GBF, BBF>)
                        : reinterpret_cast<const void*>(&pa_kernel<4, kWave, GBF, BBF>);
}

}  // namespace

hipError_t gwr_launch(const sdm_gwr_io* io, int64_t ti, hipStream_t st) {
    GwrArgs a;
    a.grad = io->grad;
    a.k_idx = io->k_idx;
    a.w = io->w;
    a.dv = io->dv;
    a.d_dv = io->d_dv;
    a.d_k_pd = io->d_k_pd;
    a.rows = io->rows;
    a.chunk0 = ti * io->P;
    a.row0 = ti * io->step_rows;
    a.P = io->P;
    a.C = io->C;
    a.W = io->W;
    a.hd = io->hd;
    a.first_partial = io->first_partial;
    a.valid_last = io->valid_last;
    a.id64 = io->idx_bytes == 8;
    a.grad_bf16 = io->grad_dtype == SDM_BF16;
    const int64_t toks = static_cast<int64_t>(io->P) * io->C;
    void* kargs[] = {&a};
    // Rows of up to 128 columns: a 32-lane team per token, two per wave (16-lane teams measured slower).
    const bool half = io->hd <= 4 * 32;
    const void* fn = a.grad_bf16 ? gwr_fn<true>(io->hd) : gwr_fn<false>(io->hd);
    const int64_t per_block = static_cast<int64_t>(kGdsWaves) * (half ? 2 : 1);
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>((toks + per_block - 1) / per_block)), dim3(kGdsThreads), kargs, 0, st);
}

PaWorkspace pa_workspace_layout(const sdm_pa_io* io) {
    const size_t pos = static_cast<size_t>(io->P) * static_cast<size_t>(io->C) * static_cast<size_t>(io->W);
    const size_t blocks = (pos + kSplitSeg - 1) / kSplitSeg;
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    PaWorkspace w;
    w.cnt_off = 0;
    w.meta_off = up(blocks * sizeof(int));
    w.part_off = w.meta_off + up(blocks * sizeof(int));
    w.total = w.part_off + up(2 * blocks * static_cast<size_t>(io->hd) * sizeof(float));
    return w;
}

hipError_t pa_launch(const sdm_pa_io* io, int64_t ti, hipStream_t st) {
    PaArgs a;
    a.grad = io->grad;
    a.bank = io->bank;
    a.snap = io->snap;
    a.krec = reinterpret_cast<const uint4*>(io->krec);
    a.k_eff = io->k_eff;
    a.beta = io->beta;
    a.d_dva = io->d_dva;
    a.g_decay = io->g_decay;
    a.d_k_eff = io->d_k_eff;
    a.rows = io->rows;
    a.chunk0 = ti * io->P;
    a.row0 = ti * io->step_rows;
    a.snap_row0 = ti * io->snap_step_rows;
    a.P = io->P;
    a.C = io->C;
    a.W = io->W;
    a.CW = io->C * io->W;
    a.hd = io->hd;
    a.vbf = io->val_bytes == 2;
    a.grad_bf16 = io->grad_dtype == SDM_BF16;
    a.bank_bf16 = io->bank_dtype == SDM_BF16;
    a.part = nullptr;
    a.cnt = nullptr;
    a.meta = nullptr;
    if (io->workspace != nullptr) {
        const PaWorkspace w = pa_workspace_layout(io);
        char* ws = static_cast<char*>(io->workspace);
        a.part = reinterpret_cast<float*>(ws + w.part_off);
        a.cnt = reinterpret_cast<int*>(ws + w.cnt_off);
        a.meta = reinterpret_cast<int*>(ws + w.meta_off);
    }
    const int64_t poss = static_cast<int64_t>(io->P) * io->C * io->W;
    void* kargs[] = {&a};
    // Rows of up to 128 columns: a 16-lane team per K-row position (8 columns per lane), four per
    // wave (faster than 32-lane teams where groups are short; long groups walk more record rounds).
    const bool half = io->hd <= 4 * 32;
    const bool gbf = a.grad_bf16 != 0, bbf = a.bank_bf16 != 0;
    const void* fn = gbf ? (bbf ? pa_fn<true, true>(io->hd) : pa_fn<true, false>(io->hd))
                         : (bbf ? pa_fn<false, true>(io->hd) : pa_fn<false, false>(io->hd));
    const int64_t per_block = static_cast<int64_t>(kGdsWaves) * (half ? 4 : 1);
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>((poss + per_block - 1) / per_block)), dim3(kGdsThreads), kargs, 0, st);
}

}  // namespace sdm
