// DW decay-and-write step on gfx950.
//
// Definition (page "sparse_delta_memory/cuda/mover_da2_cuda.py", module docstring; bit contract
// on "sparse_delta_memory/cuda/mover_fx_cuda.py", module docstring): per valid slot group of a
// chunk's K-only row, acc = fma(sc_m, dv[token_m], acc) over the members in sorted order from +0,
// then bank[slot] = fma(base, cpe_last, acc), rounded to nearest-even bf16 for a bf16 bank.
//
// Mapping: a team of lanes per K-row position. The team whose position holds a valid FIRST owns
// that group: it reads the group's base row straight from the bank (every slot has one group per
// step, so no other team writes it), walks the members' records and token rows in sorted order
// and writes the new row. Each lane owns CPL consecutive columns and moves them with 16-byte
// vector accesses; row offsets are 64-bit. Teams on positions that are not a valid FIRST exit.
#include <hip/hip_ext.h>

#include "sdm_device.hpp"
#include "sdm_launch.hpp"

namespace sdm {
namespace {

constexpr int kDwThreads = 256;

struct DwArgs {
    void* bank;
    const void* dv;
    const uint4* krec;
    int64_t dv_row0;   // ti * dv_step_rows
    int64_t chunk0;    // ti * P
    int64_t rows;      // bank rows
    float* part;       // split groups: one partial row per K-row position (NULL: groups are not split)
    int* cnt;          // per group FIRST: arrival counter, zero between calls
    int2* meta;        // per group FIRST: {segments, LAST position}
    int P, C, CW, hd, ts_log2, teams_per_block;
};

template <int CPL, bool BF16>
__device__ __forceinline__ void load_cols(const void* row, int col0, float (&x)[CPL]) {
    if constexpr (BF16) {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + col0);
#pragma unroll
        for (int v = 0; v < CPL / 8; ++v) {
            const uint4 u = p[v];
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                x[v * 8 + 2 * h] = bf16_bits_to_f32(w4[h] & 0xFFFFu);
                x[v * 8 + 2 * h + 1] = bf16_bits_to_f32(w4[h] >> 16);
            }
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(row) + col0);
#pragma unroll
        for (int v = 0; v < CPL / 4; ++v) {
            const float4 f = p[v];
            x[v * 4 + 0] = f.x;
            x[v * 4 + 1] = f.y;
            x[v * 4 + 2] = f.z;
            x[v * 4 + 3] = f.w;
        }
    }
}

template <int CPL, bool BF16>
__device__ __forceinline__ void store_cols(void* row, int col0, const float (&x)[CPL]) {
    if constexpr (BF16) {
        uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(row) + col0);
#pragma unroll
        for (int v = 0; v < CPL / 8; ++v) {
            uint32_t w4[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                w4[h] = f32_to_bf16_rne(x[v * 8 + 2 * h]) | (f32_to_bf16_rne(x[v * 8 + 2 * h + 1]) << 16);
            }
            p[v] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
    } else {
        float4* p = reinterpret_cast<float4*>(static_cast<float*>(row) + col0);
#pragma unroll
        for (int v = 0; v < CPL / 4; ++v) p[v] = make_float4(x[v * 4], x[v * 4 + 1], x[v * 4 + 2], x[v * 4 + 3]);
    }
}

// Members of a group per segment when the group is split (a workspace is given), and the last
// in-group distance that still marks a segment start (the distance field saturates at 4095).
constexpr int kSeg = 32;
constexpr int kSegLimit = (4095 / kSeg) * kSeg;

template <int CPL, bool BANK_BF16, bool DV_BF16>
__global__ void __launch_bounds__(kDwThreads) dw_kernel(DwArgs a) {
    static_assert(CPL % (BANK_BF16 ? 8 : 4) == 0 && CPL % (DV_BF16 ? 8 : 4) == 0, "16-byte column groups");
    // Member records and token rows loaded together (fewer when the rows take more registers).
    constexpr int kBatch = (CPL == 8 && DV_BF16) ? 4 : 2;
    const int team = threadIdx.x >> a.ts_log2;
    const int tl = threadIdx.x & ((1 << a.ts_log2) - 1);
    const int64_t J = static_cast<int64_t>(blockIdx.x) * a.teams_per_block + team;
    if (J >= static_cast<int64_t>(a.P) * a.CW) return;
    const int p = static_cast<int>(J / a.CW);
    const int j = static_cast<int>(J - static_cast<int64_t>(p) * a.CW);
    const int col0 = tl * CPL;
    if (col0 >= a.hd) return;   // lanes past the row (the team's lane 0 always stays)
    const uint4* kr = a.krec + (a.chunk0 + p) * a.CW;
    const uint4 r0 = kr[j];
    if (r0.x & kInvalid) return;
    // A team starts work at a group's FIRST, and, when groups are split, at every kSeg-th member.
    const bool split = a.part != nullptr;
    const int dist = static_cast<int>((r0.x >> kDistShift) & kDistMax);   // valid K entries before, in the group
    const bool first = (r0.x & kFirst) != 0u;
    if (!first && (!split || dist % kSeg != 0 || dist > kSegLimit)) return;
    const bool unbounded = !split || dist == kSegLimit;   // the last segment start runs to LAST
    if (static_cast<int64_t>(r0.y) >= a.rows) return;     // a slot outside the bank: the group is skipped
    constexpr int kBankEs = BANK_BF16 ? 2 : 4;
    constexpr int kDvEs = DV_BF16 ? 2 : 4;
    unsigned char* bank_row = static_cast<unsigned char*>(a.bank) + static_cast<int64_t>(r0.y) * a.hd * kBankEs;
    float base[CPL];
    if (first) load_cols<CPL, BANK_BF16>(bank_row, col0, base);   // in flight during the walk
    const unsigned char* dv0 = static_cast<const unsigned char*>(a.dv) +
                               (a.dv_row0 + static_cast<int64_t>(p) * a.C) * a.hd * kDvEs;
    float acc[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) acc[q] = 0.0f;
    // Walk the members in sorted order: the first on its own (most groups have one member),
    // then kBatch records and token rows at a time.
    bool last_seen = false, done = false;
    int last_pos = j, taken = 1;
    float cpe = 1.0f;
    {
        float x0[CPL];
        const int tok = static_cast<int>((r0.x >> kTokShift) & 0xFFu);
        load_cols<CPL, DV_BF16>(dv0 + static_cast<int64_t>(tok) * a.hd * kDvEs, col0, x0);
        const float sc = __uint_as_float(r0.z);
#pragma unroll
        for (int q = 0; q < CPL; ++q) acc[q] = fmaf(sc, x0[q], acc[q]);
        if (r0.x & kLast) {
            last_seen = true;
            cpe = __uint_as_float(r0.w);
            done = true;
        } else if (!unbounded && taken == kSeg) {
            done = true;
        }
    }
    for (int m = j + 1; !done && m < a.CW; m += kBatch) {
        uint4 rb[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) rb[b] = kr[min(m + b, a.CW - 1)];
        float xv[kBatch][CPL];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int tok = static_cast<int>((rb[b].x >> kTokShift) & 0xFFu);
            load_cols<CPL, DV_BF16>(dv0 + static_cast<int64_t>(tok) * a.hd * kDvEs, col0, xv[b]);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (done || m + b >= a.CW) {
                done = true;
                break;
            }
            const float sc = __uint_as_float(rb[b].z);
#pragma unroll
            for (int q = 0; q < CPL; ++q) acc[q] = fmaf(sc, xv[b][q], acc[q]);
            ++taken;
            if (rb[b].x & kLast) {
                last_seen = true;
                last_pos = m + b;
                cpe = __uint_as_float(rb[b].w);
                done = true;
            } else if (!unbounded && taken == kSeg) {
                done = true;
            }
        }
    }
    if (first && last_seen) {   // the whole group in one segment
        float o[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) o[q] = fmaf(base[q], cpe, acc[q]);
        store_cols<CPL, BANK_BF16>(bank_row, col0, o);
        return;
    }
    // Split group: publish this segment's partial; the last segment team to arrive combines the
    // partials in segment order (the same sums whichever team arrives last).
    const int64_t prow = static_cast<int64_t>(p) * a.CW;
    const int first_pos = j - dist;
    const int64_t gslot = prow + first_pos;
    float* part = a.part + (prow + j) * a.hd;
#pragma unroll
    for (int q = 0; q < CPL; ++q) part[col0 + q] = acc[q];
    const int seg = dist / kSeg;
    if (last_seen && tl == 0) a.meta[gslot] = make_int2(seg + 1, last_pos);
    __threadfence();
    // The segment holding LAST adds 1 - (segments), every other adds 1: the counter returns to 0
    // exactly at the last arrival (and is left at 0 for the next call).
    const int delta = last_seen ? -seg : 1;
    int after = 0;
    if (tl == 0) after = atomicAdd(a.cnt + gslot, delta) + delta;
    after = __shfl(after, static_cast<int>(lane_id()) & ~((1 << a.ts_log2) - 1), kWave);
    if (after != 0) return;
    __threadfence();
    const int2 meta = a.meta[gslot];
    const int nseg = meta.x;
    float tot[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) tot[q] = 0.0f;
    for (int sgi = 0; sgi < nseg; ++sgi) {
        const float* pp = a.part + (prow + first_pos + sgi * kSeg) * a.hd + col0;
#pragma unroll
        for (int q = 0; q < CPL; ++q) tot[q] = tot[q] + __builtin_nontemporal_load(pp + q);
    }
    const uint4 rf = kr[first_pos];
    const uint4 rl = kr[meta.y];
    unsigned char* brow = static_cast<unsigned char*>(a.bank) + static_cast<int64_t>(rf.y) * a.hd * kBankEs;
    float b2[CPL];
    load_cols<CPL, BANK_BF16>(brow, col0, b2);
    const float cpe_l = __uint_as_float(rl.w);
    float o[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) o[q] = fmaf(b2[q], cpe_l, tot[q]);
    store_cols<CPL, BANK_BF16>(brow, col0, o);
}

template <int CPL, bool BB, bool DB>
hipError_t launch_dw(DwArgs a, hipStream_t st, const hipEvent_t* ev) {
    const int64_t teams = static_cast<int64_t>(a.P) * a.CW;
    const int64_t blocks = (teams + a.teams_per_block - 1) / a.teams_per_block;
    void* kargs[] = {&a};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(&dw_kernel<CPL, BB, DB>), dim3(static_cast<unsigned>(blocks)),
                              dim3(kDwThreads), kargs, 0, st, ev[0], ev[1], 0);
}

template <int CPL>
hipError_t launch_dw_types(const DwArgs& a, bool bank_bf16, bool dv_bf16, hipStream_t st, const hipEvent_t* ev) {
    if (bank_bf16) return dv_bf16 ? launch_dw<CPL, true, true>(a, st, ev) : launch_dw<CPL, true, false>(a, st, ev);
    return dv_bf16 ? launch_dw<CPL, false, true>(a, st, ev) : launch_dw<CPL, false, false>(a, st, ev);
}

}  // namespace

DwWorkspace dw_workspace_layout(const sdm_dw_io* io) {
    const size_t pos = static_cast<size_t>(io->P) * static_cast<size_t>(io->C) * static_cast<size_t>(io->W);
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    DwWorkspace w;
    w.cnt_off = 0;
    w.meta_off = up(pos * sizeof(int));
    w.part_off = w.meta_off + up(pos * sizeof(int2));
    w.total = w.part_off + up(pos * static_cast<size_t>(io->hd) * sizeof(float));
    return w;
}

int dw_cols_per_lane(int hd) {
    if (hd % 8 == 0 && hd <= 8 * kWave) return 8;
    if (hd % 16 == 0 && hd <= 16 * kWave) return 16;
    return 0;
}

hipError_t dw_launch(const DwLaunch& Lc, hipStream_t st) {
    const sdm_dw_io* io = Lc.io;
    DwArgs a;
    a.bank = io->bank;
    a.dv = io->dv;
    a.krec = reinterpret_cast<const uint4*>(io->krec);
    a.dv_row0 = Lc.ti * io->dv_step_rows;
    a.chunk0 = Lc.ti * io->P;
    a.rows = io->rows;
    a.part = nullptr;
    a.cnt = nullptr;
    a.meta = nullptr;
    if (io->workspace != nullptr) {
        const DwWorkspace w = dw_workspace_layout(io);
        a.part = reinterpret_cast<float*>(static_cast<char*>(io->workspace) + w.part_off);
        a.cnt = reinterpret_cast<int*>(static_cast<char*>(io->workspace) + w.cnt_off);
        a.meta = reinterpret_cast<int2*>(static_cast<char*>(io->workspace) + w.meta_off);
    }
    a.P = io->P;
    a.C = io->C;
    a.CW = io->C * io->W;
    a.hd = io->hd;
    const int cpl = dw_cols_per_lane(io->hd);
    const int lanes = (io->hd + cpl - 1) / cpl;
    int ts = 1;
    while (ts < lanes) ts <<= 1;
    a.ts_log2 = __builtin_ctz(static_cast<unsigned>(ts));
    a.teams_per_block = kDwThreads / ts;
    if (static_cast<int64_t>(a.P) * a.CW == 0) return hipSuccess;
    const bool bb = io->bank_dtype == SDM_BF16, db = io->dv_dtype == SDM_BF16;
    const hipEvent_t ev[2] = {io->events != nullptr ? io->events[0] : nullptr,
                              io->events != nullptr ? io->events[1] : nullptr};
    if (cpl == 8) return launch_dw_types<8>(a, bb, db, st, ev);
    return launch_dw_types<16>(a, bb, db, st, ev);
}

}  // namespace sdm
