// DW decay-and-write step on gfx950.
//
// Definition (page "sparse_delta_memory/cuda/mover_da2_cuda.py", module docstring; bit contract
// on "sparse_delta_memory/cuda/mover_fx_cuda.py", module docstring): per valid slot group of a
// chunk's K-only row, acc = fma(sc_m, dv[token_m], acc) over the members in sorted order from +0,
// then bank[slot] = fma(base, cpe_last, acc), rounded to nearest-even bf16 for a bf16 bank.
//
// Mapping: a team of lanes per U consecutive K-row positions. The team whose position holds a
// valid FIRST owns that group: it reads the group's base row straight from the bank (every slot
// has one group per step, so no other team writes it), walks the members' records and token rows
// in sorted order and writes the new row. Each lane owns CPL consecutive columns and moves them
// with 16-byte vector accesses; row offsets are 64-bit. One-member groups take a short path with
// every load issued before the first use; positions that start no work exit.
#include <hip/hip_ext.h>

#include <mutex>

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
    float* part;       // split groups: partial rows, two per block of 32 K-row positions (NULL: groups are not split)
    int* cnt;          // per block of 32 positions (a split group's FIRST): arrival counter, zero between calls
    int2* meta;        // per block of 32 positions (a split group's FIRST): {segments, cpe bits of LAST}
    void* snap;        // compact snapshot (NULL: none): row snap_row0 + p * CW + j_FIRST <- the group's pre-write row
    int64_t snap_row0; // ti * snap_step_rows
    int P, C, CW, hd, ts_log2, teams_per_block;
    int stream_bank;   // host side only: the launch takes the STREAM kernel (a bank far larger than the caches)
    const int32_t* snap_ord;   // dense snapshot layout (NULL: rows at FIRST positions): gord_k of the records
};

// CPL consecutive columns of a row as raw 16-byte vectors: loads are issued apart from their
// unpacking, so that several rows can be in flight before the first is used.
template <int CPL, bool BF16>
struct RawCols {
    static constexpr int kVec = CPL * (BF16 ? 2 : 4) / 16;
    uint4 v[kVec];
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// A 16-byte load marked non-temporal: the line is not kept in the caches for reuse. Rows of a large
// bank are touched once per step (their one group's team reads and writes them) and rarely in the
// next steps, so they stream past the token rows and records, which are reused.
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
    const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// TAIL (a head dim the 16-byte vectors do not divide, as in the mover pages' scalar variant): rows
// are only element-aligned, so a lane moves its first nv (1..CPL) columns element by element, with
// zeros in the rest of the raw vector; the values and roundings are those of the vector path.
// STREAM: vector loads marked non-temporal (bank rows).
template <int CPL, bool BF16, bool TAIL, bool STREAM = false>
__device__ __forceinline__ RawCols<CPL, BF16> load_raw(const void* row, int col0, int nv) {
    RawCols<CPL, BF16> r;
    if constexpr (TAIL) {
        uint32_t w[RawCols<CPL, BF16>::kVec * 4];
        if constexpr (BF16) {
            const uint16_t* p = reinterpret_cast<const uint16_t*>(static_cast<const unsigned char*>(row) + col0 * 2);
#pragma unroll
            for (int e = 0; e < CPL; e += 2) {
                const uint32_t lo = e < nv ? p[e] : 0u;
                const uint32_t hi = e + 1 < nv ? p[e + 1] : 0u;
                w[e / 2] = lo | hi << 16;
            }
        } else {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const unsigned char*>(row) + col0 * 4);
#pragma unroll
            for (int e = 0; e < CPL; ++e) w[e] = e < nv ? p[e] : 0u;
        }
#pragma unroll
        for (int v = 0; v < RawCols<CPL, BF16>::kVec; ++v) r.v[v] = make_uint4(w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]);
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(row) + col0 * (BF16 ? 2 : 4));
#pragma unroll
        for (int v = 0; v < RawCols<CPL, BF16>::kVec; ++v) r.v[v] = STREAM ? load_stream16(p + v) : p[v];
    }
    return r;
}

template <int CPL, bool BF16>
__device__ __forceinline__ void unpack_cols(const RawCols<CPL, BF16>& r, float (&x)[CPL]) {
#pragma unroll
    for (int v = 0; v < RawCols<CPL, BF16>::kVec; ++v) {
        const uint32_t w4[4] = {r.v[v].x, r.v[v].y, r.v[v].z, r.v[v].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            if constexpr (BF16) {
                x[v * 8 + 2 * h] = bf16_bits_to_f32(w4[h] & 0xFFFFu);
                x[v * 8 + 2 * h + 1] = bf16_bits_to_f32(w4[h] >> 16);
            } else {
                x[v * 4 + h] = __uint_as_float(w4[h]);
            }
        }
    }
}

template <int CPL, bool BF16, bool TAIL>
__device__ __forceinline__ void load_cols(const void* row, int col0, int nv, float (&x)[CPL]) {
    unpack_cols<CPL, BF16>(load_raw<CPL, BF16, TAIL>(row, col0, nv), x);
}

template <int CPL, bool BF16>
__device__ __forceinline__ RawCols<CPL, BF16> pack_cols(const float (&x)[CPL]) {
    RawCols<CPL, BF16> r;
#pragma unroll
    for (int v = 0; v < RawCols<CPL, BF16>::kVec; ++v) {
        uint32_t w4[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            w4[h] = BF16 ? (f32_to_bf16_rne(x[v * 8 + 2 * h]) | (f32_to_bf16_rne(x[v * 8 + 2 * h + 1]) << 16))
                         : __float_as_uint(x[v * 4 + h]);
        }
        r.v[v] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    return r;
}

template <int CPL, bool BF16, bool TAIL>
__device__ __forceinline__ void store_raw(void* row, int col0, int nv, const RawCols<CPL, BF16>& r) {
    if constexpr (TAIL) {
        uint32_t w[RawCols<CPL, BF16>::kVec * 4];
#pragma unroll
        for (int v = 0; v < RawCols<CPL, BF16>::kVec; ++v) {
            w[4 * v] = r.v[v].x;
            w[4 * v + 1] = r.v[v].y;
            w[4 * v + 2] = r.v[v].z;
            w[4 * v + 3] = r.v[v].w;
        }
        if constexpr (BF16) {
            uint16_t* p = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(row) + col0 * 2);
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                if (e < nv) p[e] = static_cast<uint16_t>(w[e / 2] >> (16 * (e % 2)));
            }
        } else {
            uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(row) + col0 * 4);
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                if (e < nv) p[e] = w[e];
            }
        }
    } else {
        uint4* p = reinterpret_cast<uint4*>(static_cast<unsigned char*>(row) + col0 * (BF16 ? 2 : 4));
#pragma unroll
        for (int v = 0; v < RawCols<CPL, BF16>::kVec; ++v) p[v] = r.v[v];
    }
}

// Pins computed values in registers at this point of the program (no code is emitted): later
// memory operations cannot move above it, nor the computation below it.
template <int CPL, bool BF16>
__device__ __forceinline__ void pin_raw(const RawCols<CPL, BF16>& r) {
#pragma unroll
    for (int v = 0; v < RawCols<CPL, BF16>::kVec; ++v) {
        asm volatile("" ::"v"(r.v[v].x), "v"(r.v[v].y), "v"(r.v[v].z), "v"(r.v[v].w) : "memory");
    }
}

template <int CPL, bool BF16, bool TAIL>
__device__ __forceinline__ void store_cols(void* row, int col0, int nv, const float (&x)[CPL]) {
    store_raw<CPL, BF16, TAIL>(row, col0, nv, pack_cols<CPL, BF16>(x));
}

// The snapshot row of the group whose FIRST is at K-row position j of stream p: j itself, or its
// dense ordinal among the chunk's groups (snap_ord).
__device__ __forceinline__ int64_t snap_row(const DwArgs& a, int p, int j) {
    const int64_t pos = static_cast<int64_t>(p) * a.CW;
    return a.snap_row0 + pos + (a.snap_ord != nullptr ? a.snap_ord[a.chunk0 * a.CW + pos + j] : j);
}

// One snapshot row's columns: SNAP 1 the raw bank bits; SNAP 2 (float32 bank, bf16 snapshot rows)
// the row rounded to bf16, nearest even (mover_fx_cuda page: the bf16 compact rows of a float32
// bank, each group's pre-write row rounded once).
template <int CPL, bool BANK_BF16, int SNAP, bool TAIL>
__device__ __forceinline__ void snap_store(const DwArgs& a, int64_t row, int col0, int nv, const RawCols<CPL, BANK_BF16>& raw) {
    if constexpr (SNAP == 2) {
        float f[CPL];
        unpack_cols<CPL, BANK_BF16>(raw, f);
        store_raw<CPL, true, TAIL>(static_cast<unsigned char*>(a.snap) + row * a.hd * 2, col0, nv, pack_cols<CPL, true>(f));
    } else {
        store_raw<CPL, BANK_BF16, TAIL>(static_cast<unsigned char*>(a.snap) + row * a.hd * (BANK_BF16 ? 2 : 4), col0, nv, raw);
    }
}

// Members of a group per segment when the group is split (a workspace is given), and the last
// in-group distance that still marks a segment start (the distance field saturates at 4095).
constexpr int kSeg = 32;
constexpr int kSegLimit = (4095 / kSeg) * kSeg;

// Workspace slots of split groups, by step-wide K-row position G (stream p's position j is
// p * CW + j). A split group has more than kSeg members, so two split groups' FIRSTs are more than
// kSeg apart: at most one falls in each aligned block of kSeg positions, which indexes the group's
// counter and metadata. Its segments start at FIRST + kSeg k; in one block there is at most one
// later segment start (k >= 1, of the group running through the block) and at most one first
// segment (k = 0, of a group starting there): two partial rows per block.
__device__ __forceinline__ int64_t seg_group_slot(int64_t g_first) { return g_first / kSeg; }
__device__ __forceinline__ int64_t seg_part_row(int64_t g_start, bool first_segment) {
    return 2 * (g_start / kSeg) + (first_segment ? 0 : 1);
}

// The general walk of the team at K-row position j of stream p (record r0, valid): a group's FIRST
// or, when groups are split, a segment start; other positions return at once. The members after
// the first are read a team-wide batch at a time and summed per run of one token (the token row is
// loaded once per run); the sum's order is fixed by the records, so results are reproducible.
template <int CPL, bool BANK_BF16, bool DV_BF16, int SNAP, bool TAIL>
__device__ __forceinline__ void dw_walk(const DwArgs& a, int p, int j, uint4 r0, int col0, int nv, int tl) {
    // Member records and token rows loaded together (fewer when the rows take more registers).
    constexpr int kBatch = (CPL == 8 && DV_BF16) ? 4 : 2;
    const uint4* kr = a.krec + (a.chunk0 + p) * a.CW;
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
    // The base row (a group's FIRST only) stays in flight during the walk.
    RawCols<CPL, BANK_BF16> base_raw = load_raw<CPL, BANK_BF16, TAIL>(first ? bank_row : static_cast<unsigned char*>(a.bank), col0, nv);
    const unsigned char* dv0 = static_cast<const unsigned char*>(a.dv) +
                               (a.dv_row0 + static_cast<int64_t>(p) * a.C) * a.hd * kDvEs;
    float acc[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) acc[q] = 0.0f;
    // Walk the members in sorted order: the first on its own (most groups have one member),
    // then kBatch records and token rows at a time.
    bool last_seen = false, done = false;
    int taken = 1;
    float cpe = 1.0f;
    {
        float x0[CPL];
        const int tok = static_cast<int>((r0.x >> kTokShift) & 0xFFu);
        load_cols<CPL, DV_BF16, TAIL>(dv0 + static_cast<int64_t>(tok) * a.hd * kDvEs, col0, nv, x0);
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
    // The next kBatch members (records and token rows together): small groups end here.
    int m = j + 1;
    if (!done && m < a.CW) {
        uint4 rb[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) rb[b] = kr[min(m + b, a.CW - 1)];
        RawCols<CPL, DV_BF16> xr[kBatch];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int tok = static_cast<int>((rb[b].x >> kTokShift) & 0xFFu);
            xr[b] = load_raw<CPL, DV_BF16, TAIL>(dv0 + static_cast<int64_t>(tok) * a.hd * kDvEs, col0, nv);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (done || m + b >= a.CW) {
                done = true;
                break;
            }
            const float sc = __uint_as_float(rb[b].z);
            float xv[CPL];
            unpack_cols<CPL, DV_BF16>(xr[b], xv);
#pragma unroll
            for (int q = 0; q < CPL; ++q) acc[q] = fmaf(sc, xv[q], acc[q]);
            ++taken;
            if (rb[b].x & kLast) {
                last_seen = true;
                cpe = __uint_as_float(rb[b].w);
                done = true;
            } else if (!unbounded && taken == kSeg) {
                done = true;
            }
        }
        m += kBatch;
    }
    // Longer groups: the other members, a batch of `la` records at a time (one per active lane of
    // the team, all in flight together). Inside a batch, consecutive members of one token form a run: the run's
    // scales are summed first (a segmented scan across the team's lanes), so the token row is
    // loaded and fused once per run, kBatch runs' rows at a time.
    const int la = (a.hd + CPL - 1) / CPL;                        // active lanes of the team
    const int tbase = static_cast<int>(lane_id()) & ~((1 << a.ts_log2) - 1);
    for (; !done && m < a.CW; m += la) {
        const int pos = m + tl;
        const uint4 rb = kr[min(pos, a.CW - 1)];
        // Members taken from this batch: up to LAST, within the segment's budget and the row.
        int cnt = min(la, a.CW - m);
        if (!unbounded) cnt = min(cnt, kSeg - taken);
        const uint64_t team_lanes = la < 64 ? (1ull << la) - 1ull : ~0ull;   // this team's lanes, after the shift
        const uint64_t lastm = (__ballot(tl < cnt && (rb.x & kLast)) >> tbase) & team_lanes;
        const int last_lane = lastm != 0ull ? __builtin_ctzll(lastm) : -1;
        if (last_lane >= 0) cnt = last_lane + 1;
        const bool member = tl < cnt;
        const int tok = static_cast<int>((rb.x >> kTokShift) & 0xFFu);
        const int ptok = __shfl(tok, tbase + max(tl - 1, 0), kWave);
        const bool start = member && (tl == 0 || tok != ptok);
        // Run sums: inclusive segmented scan of the scales over the team's lanes (fixed tree).
        float v = member ? __uint_as_float(rb.z) : 0.0f;
        bool f = start;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            if (d >= la) break;
            const float ov = __shfl(v, tbase + max(tl - d, 0), kWave);
            const bool of = __shfl(static_cast<int>(f), tbase + max(tl - d, 0), kWave) != 0;
            if (tl >= d && !f) v = ov + v;
            if (tl >= d) f = f || of;
        }
        const int ntok = __shfl(tok, tbase + min(tl + 1, la - 1), kWave);
        const bool end = member && (tl == cnt - 1 || ntok != tok);
        uint64_t ends = (__ballot(end) >> tbase) & team_lanes;
        // The runs in order, kBatch token rows in flight at a time.
        while (ends != 0ull) {
            float cb[kBatch];
            RawCols<CPL, DV_BF16> xr[kBatch];
            int nb = 0;
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int L = ends != 0ull ? __builtin_ctzll(ends) : 0;
                const bool ok = ends != 0ull;
                const int tk = __shfl(tok, tbase + L, kWave);
                cb[b] = ok ? __shfl(v, tbase + L, kWave) : 0.0f;
                xr[b] = load_raw<CPL, DV_BF16, TAIL>(dv0 + static_cast<int64_t>(tk) * a.hd * kDvEs, col0, nv);
                nb += ok ? 1 : 0;
                ends &= ends - 1ull;
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                if (b >= nb) break;
                float xv[CPL];
                unpack_cols<CPL, DV_BF16>(xr[b], xv);
#pragma unroll
                for (int q = 0; q < CPL; ++q) acc[q] = fmaf(cb[b], xv[q], acc[q]);
            }
        }
        taken += cnt;
        if (last_lane >= 0) {
            last_seen = true;
            cpe = __uint_as_float(__shfl(rb.w, tbase + last_lane, kWave));
            done = true;
        } else if (!unbounded && taken == kSeg) {
            done = true;
        }
    }
    if (SNAP && first) {   // the pre-write row, before this team's arrival or store
        snap_store<CPL, BANK_BF16, SNAP, TAIL>(a, snap_row(a, p, j), col0, nv, base_raw);
    }
    if (first && last_seen) {   // the whole group in one segment
        float base[CPL];
        unpack_cols<CPL, BANK_BF16>(base_raw, base);
        float o[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) o[q] = fmaf(base[q], cpe, acc[q]);
        store_cols<CPL, BANK_BF16, TAIL>(bank_row, col0, nv, o);
        return;
    }
    // Split group: publish this segment's partial; the last segment team to arrive combines the
    // partials in segment order (the same sums whichever team arrives last). The segments of a group
    // run in blocks on different XCDs, whose L2 caches are not coherent with each other: the partial
    // and the group's metadata are written as device-scope atomic stores (coherent at the device
    // level without a write-back of the whole L2), the wave waits until they have completed, and
    // only then adds to the arrival counter; the combining team reads them with device-scope atomic
    // loads after seeing the last arrival.
    const int64_t prow = static_cast<int64_t>(p) * a.CW;
    const int first_pos = j - dist;
    const int64_t gslot = seg_group_slot(prow + first_pos);
    float* part = a.part + seg_part_row(prow + j, dist == 0) * a.hd;
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
        if (!TAIL || q < nv) __hip_atomic_store(part + col0 + q, acc[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int seg = dist / kSeg;
    // The segment holding LAST publishes the segment count and the group's cpe (that of LAST).
    if (last_seen && tl == 0) {
        const unsigned long long m = static_cast<uint32_t>(seg + 1) |
                                     static_cast<unsigned long long>(__float_as_uint(cpe)) << 32;
        __hip_atomic_store(reinterpret_cast<unsigned long long*>(a.meta + gslot), m, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the stores above have completed
    // The segment holding LAST adds 1 - (segments), every other adds 1: the counter returns to 0
    // exactly at the last arrival (and is left at 0 for the next call).
    const int delta = last_seen ? -seg : 1;
    int after = 0;
    if (tl == 0) after = atomicAdd(a.cnt + gslot, delta) + delta;
    after = __shfl(after, static_cast<int>(lane_id()) & ~((1 << a.ts_log2) - 1), kWave);
    if (after != 0) return;
    // The segment count, the base row (every segment's record names the group's slot) and the first
    // batch of partials in one round trip; partials past the count are read from in-row positions
    // and dropped.
    constexpr int kPartBatch = CPL == 8 ? 4 : 2;
    const unsigned long long mw = __hip_atomic_load(reinterpret_cast<const unsigned long long*>(a.meta + gslot),
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int2 meta = make_int2(static_cast<int>(mw & 0xFFFFFFFFull), static_cast<int>(mw >> 32));
    const RawCols<CPL, BANK_BF16> b2raw = load_raw<CPL, BANK_BF16, TAIL>(bank_row, col0, nv);
    float tot[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) tot[q] = 0.0f;
    int nseg = kPartBatch;   // the true count once meta has arrived
    for (int sg0 = 0; sg0 < nseg; sg0 += kPartBatch) {
        float pv[kPartBatch][CPL];
#pragma unroll
        for (int b = 0; b < kPartBatch; ++b) {
            // (before the count has arrived, a segment past it reads a row of this block range,
            // clamped to the stream's row, and is dropped)
            const int sgb = sg0 + b;
            const float* pp = a.part + seg_part_row(prow + min(first_pos + sgb * kSeg, a.CW - 1), sgb == 0) * a.hd + col0;
#pragma unroll
            for (int q = 0; q < CPL; ++q) {
                pv[b][q] = (!TAIL || q < nv) ? __hip_atomic_load(pp + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.0f;
            }
        }
#pragma unroll
        for (int b = 0; b < kPartBatch; ++b) {
#pragma unroll
            for (int q = 0; q < CPL; ++q) asm volatile("" ::"v"(pv[b][q]));   // the batch in flight together
        }
        nseg = meta.x;
#pragma unroll
        for (int b = 0; b < kPartBatch; ++b) {
            if (sg0 + b < nseg) {
#pragma unroll
                for (int q = 0; q < CPL; ++q) tot[q] = tot[q] + pv[b][q];
            }
        }
    }
    float b2[CPL];
    unpack_cols<CPL, BANK_BF16>(b2raw, b2);
    const float cpe_l = __uint_as_float(static_cast<uint32_t>(meta.y));
    float o[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) o[q] = fmaf(b2[q], cpe_l, tot[q]);
    store_cols<CPL, BANK_BF16, TAIL>(bank_row, col0, nv, o);
}

// Teams take U consecutive K-row positions. Groups of one member (the common case) are done
// together: their records, base rows and token rows are all in flight at once. Every other valid
// position goes through the general walk, one after the other.
// SNAP: also write the compact snapshot (the raw pre-write row of every valid group at its FIRST).
// STREAM: one-member groups load their bank rows non-temporally.
template <int CPL, bool BANK_BF16, bool DV_BF16, int U, int SNAP, bool TAIL, bool STREAM>
__global__ void __launch_bounds__(kDwThreads) dw_kernel(DwArgs a) {
    static_assert(CPL % (BANK_BF16 ? 8 : 4) == 0 && CPL % (DV_BF16 ? 8 : 4) == 0, "16-byte column groups");
    constexpr int kBankEs = BANK_BF16 ? 2 : 4;
    constexpr int kDvEs = DV_BF16 ? 2 : 4;
    const int team = threadIdx.x >> a.ts_log2;
    const int tl = threadIdx.x & ((1 << a.ts_log2) - 1);
    const int total = a.P * a.CW;   // < 2^31 (host checked)
    // Positions by logical block: a stream's K row runs on one XCD, whose L2 then holds its token rows.
    const int J0 = (xcd_block(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x)) * a.teams_per_block + team) * U;
    if (J0 >= total) return;
    const int col0 = tl * CPL;
    if (col0 >= a.hd) return;   // lanes past the row (the team's lane 0 always stays)
    const int nv = TAIL ? min(CPL, a.hd - col0) : CPL;   // the lane's columns
    const uint4* kr_step = a.krec + a.chunk0 * a.CW;
    if constexpr (U == 1) {   // one position: straight into the walk (its first member is the short path)
        const uint4 r0 = kr_step[J0];
        const int p = J0 / a.CW;
        if (!(r0.x & kInvalid)) dw_walk<CPL, BANK_BF16, DV_BF16, SNAP, TAIL>(a, p, J0 - p * a.CW, r0, col0, nv, tl);
        return;
    }
    // The records of positions J0 .. J0+U-1 (the steps' chunks are contiguous in krec), then the
    // base and token rows of the one-member groups among them, all in flight before any is used.
    uint4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        r[u] = kr_step[min(J0 + u, total - 1)];
        if (J0 + u >= total) r[u].x = kInvalid;
    }
    // Which positions hold one-member groups, decided for all of them (one wait for every record)
    // before any row load is issued.
    uint32_t ones = 0u;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool one = (r[u].x & (kInvalid | kFirst | kLast)) == (kFirst | kLast) && static_cast<int64_t>(r[u].y) < a.rows;
        ones |= one ? 1u << u : 0u;
    }
    // Keeps the compiler from sinking the record waits between the row loads (where the wait for a
    // later record would also wait for the rows already in flight).
    asm volatile("" ::"v"(ones) : "memory");
    RawCols<CPL, BANK_BF16> braw[U] = {};
    RawCols<CPL, DV_BF16> xraw[U] = {};
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (ones & (1u << u)) {
            const int pu = (J0 + u) / a.CW;
            const int64_t tok_row = static_cast<int64_t>(pu) * a.C + ((r[u].x >> kTokShift) & 0xFFu);
            const unsigned char* brow = static_cast<const unsigned char*>(a.bank) + static_cast<int64_t>(r[u].y) * a.hd * kBankEs;
            braw[u] = load_raw<CPL, BANK_BF16, TAIL, STREAM>(brow, col0, nv);
            xraw[u] = load_raw<CPL, DV_BF16, TAIL>(
                static_cast<const unsigned char*>(a.dv) + (a.dv_row0 + tok_row) * a.hd * kDvEs, col0, nv);
        }
    }
    // Every new row first (rows of other positions are computed on zeros and dropped), then the
    // stores: gfx9 counts stores in vmcnt, so a wait placed between stores would hold them up.
    RawCols<CPL, BANK_BF16> oraw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float sc = __uint_as_float(r[u].z), cpe = __uint_as_float(r[u].w);
        float b[CPL], x[CPL], o[CPL];
        if (SNAP && (ones & (1u << u))) {   // the pre-write row of a one-member group
            const int pu = (J0 + u) / a.CW;
            snap_store<CPL, BANK_BF16, SNAP, TAIL>(a, snap_row(a, pu, J0 + u - pu * a.CW), col0, nv, braw[u]);
        }
        unpack_cols<CPL, BANK_BF16>(braw[u], b);
        unpack_cols<CPL, DV_BF16>(xraw[u], x);
#pragma unroll
        for (int q = 0; q < CPL; ++q) o[q] = fmaf(b[q], cpe, fmaf(sc, x[q], 0.0f));
        oraw[u] = pack_cols<CPL, BANK_BF16>(o);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) pin_raw<CPL, BANK_BF16>(oraw[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (ones & (1u << u)) {
            store_raw<CPL, BANK_BF16, TAIL>(static_cast<unsigned char*>(a.bank) + static_cast<int64_t>(r[u].y) * a.hd * kBankEs,
                                            col0, nv, oraw[u]);
        }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!(ones & (1u << u)) && !(r[u].x & kInvalid)) {
            const int pu = (J0 + u) / a.CW;
            dw_walk<CPL, BANK_BF16, DV_BF16, SNAP, TAIL>(a, pu, J0 + u - pu * a.CW, r[u], col0, nv, tl);
        }
    }
}

// Positions per team: 2 once the launch has at least 32 waves per compute unit (two rows in flight
// per team then outweigh the shorter grid), else 1.
constexpr int64_t kDwWavesForPairs = 32 * 256;

template <int CPL, bool BB, bool DB, int U, bool TAIL, bool STREAM>
hipError_t launch_dw_u(DwArgs a, bool snap_bf16, hipStream_t st, const hipEvent_t* ev) {
    const void* fn = reinterpret_cast<const void*>(&dw_kernel<CPL, BB, DB, U, 0, TAIL, STREAM>);
    if (a.snap != nullptr) fn = reinterpret_cast<const void*>(&dw_kernel<CPL, BB, DB, U, 1, TAIL, STREAM>);
    if constexpr (!BB) {   // (a bf16 bank's rows are bf16 already: its bf16 snapshot is the raw one)
        if (a.snap != nullptr && snap_bf16) fn = reinterpret_cast<const void*>(&dw_kernel<CPL, BB, DB, U, 2, TAIL, STREAM>);
    }
    const int64_t teams = (static_cast<int64_t>(a.P) * a.CW + U - 1) / U;
    const int64_t blocks = (teams + a.teams_per_block - 1) / a.teams_per_block;
    void* kargs[] = {&a};
    return hipExtLaunchKernel(fn, dim3(static_cast<unsigned>(blocks)), dim3(kDwThreads), kargs, 0, st, ev[0], ev[1], 0);
}

template <int CPL, bool BB, bool DB>
hipError_t launch_dw(const DwArgs& a, bool tail, bool sbf, hipStream_t st, const hipEvent_t* ev) {
    if (tail) return launch_dw_u<CPL, BB, DB, 1, true, false>(a, sbf, st, ev);   // (element accesses: one position per team)
    const int64_t waves = static_cast<int64_t>(a.P) * a.CW * (int64_t(1) << a.ts_log2) / kWave;
    if (waves < kDwWavesForPairs) return launch_dw_u<CPL, BB, DB, 1, false, false>(a, sbf, st, ev);
    return a.stream_bank ? launch_dw_u<CPL, BB, DB, 2, false, true>(a, sbf, st, ev)
                         : launch_dw_u<CPL, BB, DB, 2, false, false>(a, sbf, st, ev);
}

template <int CPL>
hipError_t launch_dw_types(const DwArgs& a, bool bank_bf16, bool dv_bf16, bool tail, bool sbf, hipStream_t st,
                           const hipEvent_t* ev) {
    if (bank_bf16) {
        return dv_bf16 ? launch_dw<CPL, true, true>(a, tail, sbf, st, ev) : launch_dw<CPL, true, false>(a, tail, sbf, st, ev);
    }
    return dv_bf16 ? launch_dw<CPL, false, true>(a, tail, sbf, st, ev) : launch_dw<CPL, false, false>(a, tail, sbf, st, ev);
}

}  // namespace

DwWorkspace dw_workspace_layout(const sdm_dw_io* io) {
    const size_t pos = static_cast<size_t>(io->P) * static_cast<size_t>(io->C) * static_cast<size_t>(io->W);
    const size_t blocks = (pos + kSeg - 1) / kSeg;
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    DwWorkspace w;
    w.cnt_off = 0;
    w.cnt_bytes = blocks * sizeof(int);
    w.meta_off = up(w.cnt_bytes);
    w.part_off = w.meta_off + up(blocks * sizeof(int2));
    w.total = w.part_off + up(2 * blocks * static_cast<size_t>(io->hd) * sizeof(float));
    return w;
}

int dw_cols_per_lane(int hd) {
    if (hd % 8 == 0 && hd <= 8 * kWave) return 8;
    if (hd % 16 == 0 && hd <= 16 * kWave) return 16;
    if (hd >= 1 && hd <= 8 * kWave) return 8;      // tail variant (element accesses)
    if (hd >= 1 && hd <= 16 * kWave) return 16;
    return 0;
}

bool dw_tail(int hd) { return !(hd % 8 == 0 && hd <= 8 * kWave) && !(hd % 16 == 0 && hd <= 16 * kWave); }

namespace {

hipError_t dw_launch_ws(const DwLaunch& Lc, hipStream_t st, int* cnt, int2* meta, float* part) {
    const sdm_dw_io* io = Lc.io;
    DwArgs a;
    a.bank = io->bank;
    a.dv = io->dv;
    a.krec = reinterpret_cast<const uint4*>(io->krec);
    a.dv_row0 = Lc.ti * io->dv_step_rows;
    a.chunk0 = Lc.ti * io->P;
    a.rows = io->rows;
    a.part = part;
    a.cnt = cnt;
    a.meta = meta;
    a.snap = io->snap;
    a.snap_row0 = Lc.ti * io->snap_step_rows;
    a.snap_ord = io->snap_ord;
    a.P = io->P;
    a.C = io->C;
    a.CW = io->C * io->W;
    a.hd = io->hd;
    // Rows of a bank of a GiB or more (four times the last-level cache and more) are not kept in the
    // caches: they are not touched again before they would be evicted. Smaller banks keep theirs
    // (measured: non-temporal loads cost 2-3 % per step on a 0.13-0.25 GiB bank and gain 3-7 % on
    // 7.5-16 GiB banks).
    const int es = io->bank_dtype == SDM_BF16 ? 2 : 4;
    a.stream_bank = static_cast<double>(io->rows) * io->hd * es >= double(1 << 30) ? 1 : 0;
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
    const bool tail = dw_tail(io->hd);
    const bool sbf = io->snap_dtype == SDM_BF16;
    if (cpl == 8) return launch_dw_types<8>(a, bb, db, tail, sbf, st, ev);
    return launch_dw_types<16>(a, bb, db, tail, sbf, st, ev);
}

// ---- Allocation-free variant: the split-group workspace in a fixed device array of the library.
// Fixed layout (independent of the call's shape, so one call's partial rows never fall where a
// later call's counters are): counters for up to kScratchPositions K-row positions per step at
// offset 0, then their metadata pairs, then the partial rows.
constexpr int64_t kScratchPositions = int64_t(1) << 22;
constexpr size_t kScratchBlocks = static_cast<size_t>(kScratchPositions / kSeg);
constexpr size_t kScratchCntBytes = kScratchBlocks * sizeof(int);
constexpr size_t kScratchMetaBytes = kScratchBlocks * sizeof(int2);
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr size_t kScratchPartBytes = kScratchBytes - kScratchCntBytes - kScratchMetaBytes;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Per device: the array's device address (hipGetSymbolAddress with that device current), found once.
constexpr int kScratchDevices = 64;
struct ScratchDev {
    std::once_flag once;
    hipError_t err = hipSuccess;
    unsigned char* ptr = nullptr;
};
ScratchDev g_scratch[kScratchDevices];

__global__ void __launch_bounds__(256) dw_clear_counters(int* cnt, int n) {
    const int i = static_cast<int>(blockIdx.x) * 256 + static_cast<int>(threadIdx.x);
    if (i < n) cnt[i] = 0;
}

}  // namespace

hipError_t dw_launch(const DwLaunch& Lc, hipStream_t st) {
    const sdm_dw_io* io = Lc.io;
    if (io->workspace == nullptr) return dw_launch_ws(Lc, st, nullptr, nullptr, nullptr);
    const DwWorkspace w = dw_workspace_layout(io);
    char* ws = static_cast<char*>(io->workspace);
    return dw_launch_ws(Lc, st, reinterpret_cast<int*>(ws + w.cnt_off), reinterpret_cast<int2*>(ws + w.meta_off),
                        reinterpret_cast<float*>(ws + w.part_off));
}

bool dw_static_fits(const sdm_dw_io* io, size_t* need, size_t* cap) {
    const int64_t pos = static_cast<int64_t>(io->P) * io->C * io->W;
    const size_t blocks = static_cast<size_t>((pos + kSeg - 1) / kSeg);
    *need = 2 * blocks * static_cast<size_t>(io->hd) * sizeof(float);
    *cap = kScratchPartBytes;
    return pos <= kScratchPositions && *need <= kScratchPartBytes;
}

hipError_t dw_static_setup() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    ScratchDev& d = g_scratch[dev];
    std::call_once(d.once, [&d]() {
        void* ptr = nullptr;
        d.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (d.err == hipSuccess) d.ptr = static_cast<unsigned char*>(ptr);
        else (void)hipGetLastError();
    });
    return d.err;
}

hipError_t dw_launch_static(const DwLaunch& Lc, hipStream_t st) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    unsigned char* base = g_scratch[dev].ptr;   // (dw_static_setup succeeded on this device)
    int* cnt = reinterpret_cast<int*>(base);
    int2* meta = reinterpret_cast<int2*>(base + kScratchCntBytes);
    float* part = reinterpret_cast<float*>(base + kScratchCntBytes + kScratchMetaBytes);
    const sdm_dw_io* io = Lc.io;
    const int64_t pos = static_cast<int64_t>(io->P) * io->C * io->W;
    if (pos == 0) return hipSuccess;
    // The counters this call uses start at zero: a fill kernel (not a memset node, so the pair
    // replays correctly from a captured graph), then the step.
    const int nblk = static_cast<int>((pos + kSeg - 1) / kSeg);
    int n_clear = nblk;
    void* cargs[] = {&cnt, &n_clear};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&dw_clear_counters), dim3((nblk + 255) / 256), dim3(256), cargs, 0, st);
    if (e != hipSuccess) return e;
    return dw_launch_ws(Lc, st, cnt, meta, part);
}

}  // namespace sdm
