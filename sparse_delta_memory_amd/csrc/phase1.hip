// Phase 1 of the chunked SDM recurrence on gfx950.
//
// One 1024-thread workgroup per chunk:
//   1. sort: the chunk's entries, keyed by local slot, are sorted stably in LDS by an LSD radix
//      sort whose ranks come from ballot-built peer masks (no atomics, stable by construction);
//   2. reverse scan: in tiles of 4096 sorted positions (4 per thread), last tile first, a
//      segmented scan of gate contributions and peer counts; each thread keeps its exclusive
//      prefix per tile in registers, plus its entries' values;
//   3. forward scan: the same tiles in order; each thread keeps its forward prefix and kind-row
//      base per tile. After these two passes every per-entry quantity can be recomputed by a
//      thread from its own registers and the sorted row, with no further block-wide work;
//   4. output rounds: entry-order fields are scattered into LDS at their entry index and copied
//      out with 16-byte stores; sorted-order records (for the pair kernel), the sorted kind rows
//      and the mover records are staged tile by tile (their indices are contiguous per tile).
// A second kernel sums the A / QK triangles.
//
// Definitions: page "sparse_delta_memory/cuda/phase1_cuda.py" (module docstring; keys and payloads
// of p1_keys_zw_kernel; the scan semantics of p1_scan_kernel; the pair terms of p1_pairs_kernel).
// Scans combine TwoSum-compensated float sums in a fixed tree; every output element has one
// writer; no floating-point atomics are used, so results are bitwise reproducible.
#include <hip/hip_ext.h>

#include "sdm_device.hpp"
#include "sdm_launch.hpp"

namespace sdm {
namespace {

constexpr int kNT = kP1Threads;   // 1024 threads = 16 waves per chunk
constexpr int kNW = kNT / kWave;
constexpr int kTileItems = 4;     // scan items per thread per tile
constexpr int kTile = kNT * kTileItems;
constexpr uint32_t kFlagHead = 1u << 14;   // group head, kept beside r (< 2^14) in the sorted row
constexpr uint32_t kFlagRep = 1u << 15;    // repeated K entry (its gate is not applied again)
constexpr uint32_t kRMask = kFlagHead - 1u;

// Entry-order fields assembled in LDS and copied out with wide stores: the outputs, then two
// workspace arrays for the pair kernel (sorted position of every entry; "starts a run with
// earlier K entries in its group").
enum Field : int {
    kFLogK, kFRex, kFCpe, kFKEff, kFIsLast, kFIsOnly, kFPosK,
    kFLogQ, kFQW, kFPosQ, kFQLast, kFQOnly, kFInv, kFWalk, kNumFields
};
constexpr int kMaxRounds = 8;

struct Rounds {
    int count;
    uint32_t mask[kMaxRounds];
    uint32_t flat;            // rounds copied out by one loop over all their 16-byte vectors
    int offset[kNumFields];   // byte offset of a field inside the staging area of its round
    int vtotal[kMaxRounds];   // 16-byte vectors staged in a round
    // Per round, the first vector of each of its fields (offset / 16); a large value for the other
    // fields, so the field of vector v is the last one whose start is <= v.
    int vstart[kMaxRounds][kNumFields];
};

struct P1Args {
    const int32_t* k_idx;
    const int32_t* q_idx;
    const float* k_val;
    const float* q_val;
    const float* g;
    void* field[kNumFields];   // entry-order destinations (NULL: skipped); kFInv, kFWalk: workspace
    int32_t* spay_k;
    int32_t* spay_q;
    int4* krec;
    int32_t* tiles_k;
    int32_t* repeats;
    uint4* rec;
    uint2* hot;          // per chunk: {count, 0}, then {head position, size} of each hot group (NULL: none)
    int C, W, R, P, key_bits, first_partial, valid_last, tile_len, digit_bits;
    int stage_bytes;
    int hot_min;         // valid K entries that make a group hot for the pair kernel
    int hot_cap;         // hot groups one chunk can have (list entries after the count)
    uint32_t wr_magic;   // ceil(2^32 / (W + R)): r / (W + R) == umulhi(r, wr_magic) for r < 2^17
    int64_t stream_offset;
    Rounds rounds;
};

__host__ __device__ constexpr int field_bytes(int f) {
    return (f == kFIsLast || f == kFIsOnly || f == kFQLast || f == kFQOnly || f == kFWalk) ? 1 : f == kFInv ? 2 : 4;
}
__host__ __device__ constexpr bool field_is_q(int f) { return f >= kFLogQ && f <= kFQOnly; }
__host__ __device__ constexpr bool field_is_all(int f) { return f == kFInv || f == kFWalk; }

// r / (W + R) for entry indices r < 2^17 and W + R <= 512 (multiply-high by a rounded-up
// reciprocal; the error term r / 2^32 stays below 1 / (W + R)).
__device__ __forceinline__ int token_of_entry(int r, uint32_t magic) {
    return static_cast<int>(__umulhi(static_cast<uint32_t>(r), magic));
}

// Segmented-scan element: a TwoSum-compensated float sum (s + c), the valid K count (bits 0-15),
// the valid Q count (bits 16-30) and a segment-start flag (bit 31).
struct Seg {
    float s;
    float c;
    uint32_t f;
};
constexpr uint32_t kSegHead = 0x80000000u;
constexpr uint32_t kSegQOne = 1u << 16;

__device__ __forceinline__ Seg seg_zero() { return Seg{0.0f, 0.0f, 0u}; }

// a precedes b in scan order. A segment start in b discards a.
__device__ __forceinline__ Seg seg_combine(Seg a, Seg b) {
    if (b.f & kSegHead) return b;
    const float s = a.s + b.s;
    const float bb = s - a.s;
    const float err = (a.s - (s - bb)) + (b.s - bb);
    return Seg{s, (a.c + b.c) + err, ((a.f & ~kSegHead) + (b.f & ~kSegHead)) | (a.f & kSegHead)};
}

template <bool REV>
__device__ __forceinline__ Seg seg_shfl(Seg v, int d) {
    Seg o;
    if (REV) {
        o.s = __shfl_down(v.s, d, kWave);
        o.c = __shfl_down(v.c, d, kWave);
        o.f = __shfl_down(v.f, d, kWave);
    } else {
        o.s = __shfl_up(v.s, d, kWave);
        o.c = __shfl_up(v.c, d, kWave);
        o.f = __shfl_up(v.f, d, kWave);
    }
    return o;
}

// Barrier for LDS hazards only: LDS operations complete, global stores may stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Exclusive segmented scan of one element per thread over the block, in thread order
// (REV: descending). Fixed tree: lane doubling, then the wave totals in scan order. `total`
// receives the block's combined element. wtot: kNW elements of LDS.
template <bool REV>
__device__ __forceinline__ Seg block_exclusive_seg(Seg agg, Seg* wtot, Seg& total) {
    const int lane = static_cast<int>(lane_id());
    const int w = threadIdx.x / kWave;
    Seg incl = agg;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const Seg o = seg_shfl<REV>(incl, d);
        if (REV ? (lane + d < kWave) : (lane >= d)) incl = seg_combine(o, incl);
    }
    Seg ex = seg_shfl<REV>(incl, 1);
    if (REV ? (lane == kWave - 1) : (lane == 0)) ex = seg_zero();
    if (REV ? (lane == 0) : (lane == kWave - 1)) wtot[w] = incl;
    lds_barrier();
    Seg pre = seg_zero(), tot = seg_zero();
    for (int i = 0; i < kNW; ++i) {
        const int ww = REV ? kNW - 1 - i : i;
        if (ww == w) pre = tot;
        tot = seg_combine(tot, wtot[ww]);
    }
    lds_barrier();
    total = tot;
    return seg_combine(pre, ex);
}

// Exclusive integer sum over the block in thread order; `total` receives the block sum.
__device__ __forceinline__ uint32_t block_exclusive_add(uint32_t v, uint32_t* wsum, uint32_t& total) {
    const int lane = static_cast<int>(lane_id());
    const int w = threadIdx.x / kWave;
    uint32_t incl = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) wsum[w] = incl;
    lds_barrier();
    uint32_t pre = 0, tot = 0;
    for (int ww = 0; ww < kNW; ++ww) {
        const uint32_t x = wsum[ww];
        pre += ww < w ? x : 0u;
        tot += x;
    }
    lds_barrier();
    total = tot;
    return pre + incl - v;
}

// Stable LSD radix sort of the block's kNT * IPT (key, value) pairs over key bits [0, bits), in
// digits of up to `dmax` bits. Items live in registers in striped order (item k of lane l of wave
// w is element w * 64 * IPT + k * 64 + l). Per digit: ranks inside the wave from ballot-built
// peer masks, slice by slice (equal digits keep element order); per-wave digit counts in LDS
// (rows of 2^dmax); one block scan over (digit, wave) gives every (wave, digit) its start; a
// scatter into skey / sval. On return skey / sval hold the sorted sequence.
template <int IPT>
__device__ void block_radix_sort(uint32_t (&key)[IPT], uint32_t (&val)[IPT], int bits, int dmax, uint32_t* skey,
                                 uint16_t* sval, uint32_t* hist, uint32_t* wsum) {
    const int lane = static_cast<int>(lane_id());
    const int w = threadIdx.x / kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int stride = 1 << dmax;
    uint32_t* my_hist = hist + w * stride;
    const int passes = (bits + dmax - 1) / dmax;
    for (int pass = 0; pass < passes; ++pass) {
        const int sh = pass * dmax;
        const int db = min(dmax, bits - sh);
        const int nd = 1 << db;
        const uint32_t dmask = static_cast<uint32_t>(nd - 1);
        for (int d = lane; d < nd; d += kWave) my_hist[d] = 0u;
        lds_barrier();
        // The rank inside the wave (< 2^16) rides in the upper half of val (values are < 2^16).
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const uint32_t d = (key[k] >> sh) & dmask;
            uint64_t peers = ~0ull;
            for (int b = 0; b < db; ++b) {
                const bool bit = (d >> b) & 1u;
                const uint64_t m = __ballot(bit);
                peers &= bit ? m : ~m;
            }
            const uint32_t below = static_cast<uint32_t>(__popcll(peers & lt_mask));
            const uint32_t cnt = static_cast<uint32_t>(__popcll(peers));
            const uint32_t base = my_hist[d];
            val[k] = (val[k] & 0xFFFFu) | (base + below) << 16;
            if (below == 0) my_hist[d] = base + cnt;   // the slice's lowest lane of this digit
        }
        lds_barrier();
        // Exclusive scan over the counts in (digit, wave) order: thread x owns the `per`
        // consecutive elements e = x * per + u, element e being (digit e / kNW, wave e % kNW).
        const int per = (nd * kNW + kNT - 1) / kNT;
        uint32_t local = 0;
        for (int u = 0; u < per; ++u) {
            const int e = threadIdx.x * per + u;
            if (e < nd * kNW) local += hist[(e % kNW) * stride + e / kNW];
        }
        uint32_t tot;
        uint32_t run = block_exclusive_add(local, wsum, tot);
        for (int u = 0; u < per; ++u) {
            const int e = threadIdx.x * per + u;
            if (e < nd * kNW) {
                uint32_t* h = hist + (e % kNW) * stride + e / kNW;
                const uint32_t cnt = *h;
                *h = run;
                run += cnt;
            }
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const uint32_t d = (key[k] >> sh) & dmask;
            const uint32_t pos = my_hist[d] + (val[k] >> 16);
            skey[pos] = key[k];
            sval[pos] = static_cast<uint16_t>(val[k] & 0xFFFFu);
        }
        lds_barrier();
        if (pass + 1 < passes) {
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int i = w * kWave * IPT + k * kWave + lane;
                key[k] = skey[i];
                val[k] = sval[i];
            }
            lds_barrier();
        }
    }
}

// Copies `count` elements of `es` bytes from LDS (16-byte aligned) to global memory with the
// whole block: 16-byte accesses when the destination is 16-byte aligned, element-sized ones
// otherwise.
__device__ __forceinline__ void block_copy_out(void* dst, const unsigned char* src, int count, int es) {
    const int bytes = count * es;
    int done = 0;
    if ((reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
        const int vecs = bytes >> 4;
        for (int i = threadIdx.x; i < vecs; i += kNT) {
            reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
        }
        done = vecs << 4;
    }
    if (es == 4 && (reinterpret_cast<uintptr_t>(dst) & 3u) == 0) {
        for (int i = (done >> 2) + threadIdx.x; i < count; i += kNT) {
            reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src)[i];
        }
        return;
    }
    for (int i = done + threadIdx.x; i < bytes; i += kNT) static_cast<unsigned char*>(dst)[i] = src[i];
}

// Copies the round's staged fields out. A flat round (every field's rows 16-byte aligned and a
// multiple of 16 bytes long, so its vectors are contiguous in the staging area) is one loop over
// all its vectors, two per thread in flight: the field of a vector is found by comparisons with
// the round's field starts, its destination from a per-field table (`dtab[f]`: the chunk's row of
// field f, minus the field's staging start). Otherwise each field is copied on its own.
__device__ __forceinline__ void copy_round(const P1Args& a, int rd, uint32_t mask, const unsigned char* stage,
                                           const uint2* dtab, int64_t crow, int64_t cr, int64_t cw, int C) {
    if ((a.rounds.flat >> rd) & 1u) {   // block-uniform
        const int total = a.rounds.vtotal[rd];
        int vs[kNumFields];
#pragma unroll
        for (int k = 0; k < kNumFields; ++k) vs[k] = a.rounds.vstart[rd][k];
        // Destination of vector v: the table holds plain integers, so the store names the global
        // address space itself (a generic pointer would make it a flat store).
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(1))) u32x4 global_u32x4;
        auto dst_of = [&](int v) {
            int f = 0;
#pragma unroll
            for (int k = 0; k < kNumFields; ++k) f = v >= vs[k] ? k : f;
            const uint2 d = dtab[f];
            return reinterpret_cast<global_u32x4*>(static_cast<uintptr_t>(d.x) | static_cast<uintptr_t>(d.y) << 32) + v;
        };
        const u32x4* src = reinterpret_cast<const u32x4*>(stage);
        for (int v0 = static_cast<int>(threadIdx.x); v0 < total; v0 += 2 * kNT) {
            const int v1 = min(v0 + kNT, total - 1);   // a second vector in flight (a repeat at the end)
            const u32x4 x0 = src[v0];
            const u32x4 x1 = src[v1];
            global_u32x4* d0 = dst_of(v0);
            global_u32x4* d1 = dst_of(v1);
            *d0 = x0;
            if (v0 + kNT < total) *d1 = x1;
        }
        return;
    }
    for (int f = 0; f < kNumFields; ++f) {
        if (!(mask & (1u << f))) continue;
        const int cnt = field_is_all(f) ? a.C * (a.W + a.R) : field_is_q(f) ? C * a.R : C * a.W;
        const int64_t base = field_is_all(f) ? crow : field_is_q(f) ? cr : cw;
        unsigned char* d = static_cast<unsigned char*>(a.field[f]) + base * field_bytes(f);
        block_copy_out(d, stage + a.rounds.offset[f], cnt, field_bytes(f));
    }
}

// Everything one sorted position yields, recomputed by its owner thread from its tile prefixes.
struct Entry {
    bool live;       // position < n
    bool valid;      // token inside the chunk's valid count
    bool q;          // read entry
    bool head;       // first of its group
    bool walk;       // starts its token's run of its kind and has earlier valid K entries in the group
    bool keep;       // its pair record is read: its group spans two or more positions, or it is the
                     // head right after such a group (the run sums of the walks stop there)
    int t, ln, r;
    uint32_t pay;    // entry bits of the payload
    float s, c;      // inclusive log-cumsum (compensated)
    float rex;       // sum after (K: rex)
    uint32_t bcnt;   // own-kind valid peers before
    uint32_t acnt;   // own-kind valid peers after
    uint32_t jkind;  // index in its kind's sorted row
    uint32_t kg;     // valid K entries of its group
    uint32_t gsize;  // valid entries of its group
    float v;
};

template <int IPT>
__global__ void __launch_bounds__(kNT) p1_main_kernel(P1Args a) {
    constexpr int NP = kNT * IPT;
    constexpr int NTILE = (NP + kTile - 1) / kTile;
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* stage = smem;                                   // staging, after the scans
    uint32_t* skey = reinterpret_cast<uint32_t*>(smem);           // sort keys (inside staging)
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + NP * 4);  // digit counts (inside staging)
    uint16_t* sval = reinterpret_cast<uint16_t*>(smem + a.stage_bytes);
    float* gates = reinterpret_cast<float*>(smem + a.stage_bytes + NP * 2);
    __shared__ Seg wtot[kNW];
    __shared__ uint32_t wsum[kNW];
    __shared__ uint32_t tile_kind[NTILE + 1];   // kind counts (K | Q << 16) before each tile
    __shared__ uint32_t hot_n;                   // hot groups found so far
    __shared__ uint2 dtab[kNumFields];           // flat copy-out: per-field destination bases
    uint2* hot_buf = reinterpret_cast<uint2*>(smem + a.stage_bytes + NP * 2 + 256 * sizeof(float));

    const int c = blockIdx.x;
    const int C = a.C, W = a.W, R = a.R;
    const int wr = W + R;
    const int n = C * wr;
    const int tv = c >= a.first_partial ? a.valid_last : C;
    const int kb = a.key_bits;
    const uint32_t key_lim = 1u << kb;       // valid keys are below; invalid = key_lim
    const uint32_t pad_key = 0xFFFFFFFFu;    // padding past the row sorts last
    const int64_t id_base = static_cast<int64_t>(c % a.P) * a.stream_offset;
    const int64_t cw = static_cast<int64_t>(c) * C * W;
    const int64_t cr = static_cast<int64_t>(c) * C * R;
    const int64_t crow = static_cast<int64_t>(c) * n;
    const int lane = static_cast<int>(lane_id());
    const int w = threadIdx.x / kWave;
    const int ntiles = (n + kTile - 1) / kTile;

    for (int t = threadIdx.x; t < C; t += kNT) gates[t] = t < tv ? a.g[static_cast<int64_t>(c) * C + t] : 0.0f;
    if (threadIdx.x == 0) hot_n = 0u;
#pragma unroll
    for (int f = 0; f < kNumFields; ++f) {
        if (threadIdx.x == f) {
            // The chunk's row of field f, less the field's start in its round's staging area (the
            // flat copy adds the staged byte offset). Unused for skipped fields.
            const int64_t base = field_is_all(f) ? crow : field_is_q(f) ? cr : cw;
            const uintptr_t d = reinterpret_cast<uintptr_t>(a.field[f]) + base * field_bytes(f) -
                                static_cast<uintptr_t>(a.rounds.offset[f]);
            dtab[f] = make_uint2(static_cast<uint32_t>(d), static_cast<uint32_t>(d >> 32));
        }
    }

    // ---- 1. keys (element i of the striped layout is entry r = i) and the sort.
    {
        uint32_t key[IPT], val[IPT];
        if constexpr (IPT <= 8) {
            int32_t ids[IPT];
            // Every item loads (padding items re-read entry 0) before any id is used: the asm
            // below keeps the compiler from sinking a load into the select that uses it, where
            // each load would get a wait of its own. (With 16 items per thread the registers are
            // better spent otherwise: measured slower there.)
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int i = w * kWave * IPT + k * kWave + lane;
                val[k] = static_cast<uint32_t>(i);
                const int ic = i < n ? i : 0;
                const int t = token_of_entry(ic, a.wr_magic);
                const int j = ic - t * wr;
                ids[k] = *(j < W ? a.k_idx + cw + t * W + j : a.q_idx + cr + t * R + (j - W));
            }
#pragma unroll
            for (int k = 0; k < IPT; ++k) asm volatile("" ::"v"(ids[k]));
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int i = w * kWave * IPT + k * kWave + lane;
                const int t = token_of_entry(i < n ? i : 0, a.wr_magic);
                const uint32_t kv =
                    t < tv ? static_cast<uint32_t>(static_cast<int64_t>(ids[k]) - id_base) & (key_lim - 1u) : key_lim;
                key[k] = i < n ? kv : pad_key;
            }
        } else {
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int i = w * kWave * IPT + k * kWave + lane;
                val[k] = static_cast<uint32_t>(i);
                const int ic = i < n ? i : 0;
                const int t = token_of_entry(ic, a.wr_magic);
                const int j = ic - t * wr;
                const int32_t* src = j < W ? a.k_idx + cw + t * W + j : a.q_idx + cr + t * R + (j - W);
                const int64_t id = static_cast<int64_t>(*src);
                const uint32_t kv = t < tv ? static_cast<uint32_t>(id - id_base) & (key_lim - 1u) : key_lim;
                key[k] = i < n ? kv : pad_key;
            }
        }
        // Invalid entries need one more key bit only in a ragged chunk.
        block_radix_sort<IPT>(key, val, tv < C ? kb + 1 : kb, a.digit_bits, skey, sval, hist, wsum);
    }

    // Per-thread state carried from the scans to the output rounds (registers, tile-indexed).
    Seg rpre[NTILE], fpre[NTILE];
    uint32_t kpre[NTILE];
    float vv[NTILE][kTileItems];
    uint32_t repeat_count = 0;

    // ---- 2. reverse scan: sums and peer counts after each entry in its group.
    {
        Seg rcarry = seg_zero();
#pragma unroll
        for (int Ti = 0; Ti < NTILE; ++Ti) {
            const int T = NTILE - 1 - Ti;
            rpre[T] = seg_zero();
            if (T >= ntiles) continue;   // block-uniform
            const int p0 = T * kTile + threadIdx.x * kTileItems;
            uint32_t kk[kTileItems], rr[kTileItems];
#pragma unroll
            for (int k = 0; k < kTileItems; ++k) {
                const int p = p0 + k;
                kk[k] = p < n ? skey[p] : pad_key;
                rr[k] = p < n ? (sval[p] & kRMask) : 0u;
            }
            const bool has_prev = p0 > 0 && p0 <= n;
            const uint32_t prev_key = has_prev ? skey[p0 - 1] : pad_key;
            const uint32_t prev_r = has_prev ? (sval[p0 - 1] & kRMask) : 0u;
            const uint32_t next_key = p0 + kTileItems < n ? skey[p0 + kTileItems] : pad_key;
            uint32_t heads = 0, ends = 0, reps = 0;
            float x[kTileItems];
#pragma unroll
            for (int k = 0; k < kTileItems; ++k) {
                const uint32_t pk = k ? kk[k - 1] : prev_key;
                const uint32_t pr = k ? rr[k - 1] : prev_r;
                const bool valid = kk[k] < key_lim;
                const bool pvalid = pk < key_lim && (p0 + k) > 0;
                const bool head = !valid || !pvalid || kk[k] != pk;
                const int t = token_of_entry(static_cast<int>(rr[k]), a.wr_magic);
                const int j = static_cast<int>(rr[k]) - t * wr;
                const bool is_k = valid && j < W;
                const int pt = token_of_entry(static_cast<int>(pr), a.wr_magic);
                const int pj = static_cast<int>(pr) - pt * wr;
                const bool rep = !head && is_k && pj < W && pt == t;
                heads |= (head ? 1u : 0u) << k;
                reps |= (rep ? 1u : 0u) << k;
                x[k] = (is_k && !rep) ? gates[t] : 0.0f;
                // Keep the slot and the value for the outputs (one branch-free load per entry).
                const bool q = j >= W;
                const int ln = q ? j - W : j;
                const float* vsrc = q ? a.q_val + cr + t * R + ln : a.k_val + cw + t * W + ln;
                const float vl = *(p0 + k < n ? vsrc : a.k_val + cw);
                vv[T][k] = valid ? vl : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < kTileItems; ++k) {
                const bool end = k + 1 < kTileItems
                                     ? ((heads >> (k + 1)) & 1u)
                                     : (!(kk[k] < key_lim) || !(next_key < key_lim) || next_key != kk[k]);
                ends |= (end ? 1u : 0u) << k;
            }
            Seg agg = seg_zero();
#pragma unroll
            for (int k = kTileItems - 1; k >= 0; --k) {
                const bool valid = kk[k] < key_lim;
                const int t = token_of_entry(static_cast<int>(rr[k]), a.wr_magic);
                const bool q = static_cast<int>(rr[k]) - t * wr >= W;
                agg = seg_combine(agg, Seg{x[k], 0.0f, (valid ? (q ? kSegQOne : 1u) : 0u) |
                                                           (((ends >> k) & 1u) ? kSegHead : 0u)});
            }
            Seg total;
            rpre[T] = seg_combine(rcarry, block_exclusive_seg<true>(agg, wtot, total));
            rcarry = seg_combine(rcarry, total);
#pragma unroll
            for (int k = 0; k < kTileItems; ++k) {
                const int p = p0 + k;
                if (p < n) {
                    sval[p] = static_cast<uint16_t>(rr[k] | (((heads >> k) & 1u) ? kFlagHead : 0u) |
                                                    (((reps >> k) & 1u) ? kFlagRep : 0u));
                    repeat_count += (reps >> k) & 1u;
                }
            }
        }
    }
    __syncthreads();   // every flag of the sorted row is set; the keys are no longer needed

    // The tile's entries as the scans see them, from the flagged sorted row.
    auto load_tile = [&](int T, uint32_t (&rr)[kTileItems], float (&x)[kTileItems], uint32_t& heads,
                         uint32_t& ends) {
        const int p0 = T * kTile + threadIdx.x * kTileItems;
        heads = 0;
        ends = 0;
#pragma unroll
        for (int k = 0; k < kTileItems; ++k) {
            const int p = p0 + k;
            rr[k] = p < n ? sval[p] : kFlagHead;   // padding: a group of its own
            const int r = static_cast<int>(rr[k] & kRMask);
            const int t = token_of_entry(r, a.wr_magic);
            const bool q = r - t * wr >= W;
            const bool valid = p < n && t < tv;
            x[k] = (valid && !q && !(rr[k] & kFlagRep)) ? gates[t] : 0.0f;
            heads |= ((rr[k] & kFlagHead) ? 1u : 0u) << k;
        }
        const int pn = p0 + kTileItems;
        const bool next_head = pn >= n || (sval[pn] & kFlagHead);
#pragma unroll
        for (int k = 0; k < kTileItems; ++k) {
            const bool end = k + 1 < kTileItems ? ((heads >> (k + 1)) & 1u) : next_head;
            ends |= (end ? 1u : 0u) << k;
        }
    };
    auto tile_item = [&](int T, int k, const uint32_t (&rr)[kTileItems], const float (&x)[kTileItems],
                         bool seg_start) {
        const int p = T * kTile + threadIdx.x * kTileItems + k;
        const int r = static_cast<int>(rr[k] & kRMask);
        const int t = token_of_entry(r, a.wr_magic);
        const bool q = r - t * wr >= W;
        const bool valid = p < n && t < tv;
        return Seg{x[k], 0.0f, (valid ? (q ? kSegQOne : 1u) : 0u) | (seg_start ? kSegHead : 0u)};
    };

    // ---- 3. forward scan: per-tile forward prefixes and kind-row bases.
    {
        Seg fcarry = seg_zero();
        uint32_t kind_carry = 0;
#pragma unroll
        for (int T = 0; T < NTILE; ++T) {
            fpre[T] = seg_zero();
            kpre[T] = 0;
            if (T >= ntiles) continue;   // block-uniform
            const int p0 = T * kTile + threadIdx.x * kTileItems;
            uint32_t rr[kTileItems], heads, ends;
            float x[kTileItems];
            load_tile(T, rr, x, heads, ends);
            uint32_t kind_cnt = 0;
            Seg agg = seg_zero();
#pragma unroll
            for (int k = 0; k < kTileItems; ++k) {
                agg = seg_combine(agg, tile_item(T, k, rr, x, (heads >> k) & 1u));
                const int r = static_cast<int>(rr[k] & kRMask);
                const int t = token_of_entry(r, a.wr_magic);
                if (p0 + k < n) kind_cnt += (r - t * wr >= W) ? kSegQOne : 1u;
            }
            Seg total;
            fpre[T] = seg_combine(fcarry, block_exclusive_seg<false>(agg, wtot, total));
            fcarry = seg_combine(fcarry, total);
            uint32_t kind_total;
            kpre[T] = kind_carry + block_exclusive_add(kind_cnt, wsum, kind_total);
            if (threadIdx.x == 0) tile_kind[T] = kind_carry;
            kind_carry += kind_total;
        }
        if (threadIdx.x == 0) tile_kind[ntiles] = kind_carry;
        uint32_t rep_total;
        (void)block_exclusive_add(repeat_count, wsum, rep_total);
        if (threadIdx.x == 0 && a.repeats != nullptr) a.repeats[c] = static_cast<int32_t>(rep_total);
    }
    __syncthreads();

    // Recomputes the four entries of tile T owned by this thread and calls f(k, entry).
    auto for_tile = [&](int T, const Seg& rp, const Seg& fp, uint32_t kp, const float (&vl)[kTileItems], auto&& f) {
        const int p0 = T * kTile + threadIdx.x * kTileItems;
        uint32_t rr[kTileItems], heads, ends;
        float x[kTileItems];
        load_tile(T, rr, x, heads, ends);
        float rexs[kTileItems];
        uint32_t afts[kTileItems];
        Seg run = rp;
#pragma unroll
        for (int k = kTileItems - 1; k >= 0; --k) {
            const bool end = (ends >> k) & 1u;
            const Seg after = end ? seg_zero() : run;
            rexs[k] = after.s + after.c;
            afts[k] = after.f & ~kSegHead;
            run = seg_combine(run, tile_item(T, k, rr, x, end));
        }
        const uint32_t prev_raw = p0 > 0 && p0 <= n ? sval[p0 - 1] : (0xFFFFu & ~kFlagHead);
        const uint32_t prev_r = prev_raw & kRMask;
        run = fp;
        uint32_t jk = kp & 0xFFFFu, jq = kp >> 16;
#pragma unroll
        for (int k = 0; k < kTileItems; ++k) {
            const bool head = (heads >> k) & 1u;
            const Seg before = head ? seg_zero() : run;
            run = seg_combine(run, tile_item(T, k, rr, x, head));
            Entry e;
            e.live = p0 + k < n;
            e.r = static_cast<int>(rr[k] & kRMask);
            e.t = token_of_entry(e.r, a.wr_magic);
            const int j = e.r - e.t * wr;
            e.q = j >= W;
            e.ln = e.q ? j - W : j;
            e.valid = e.live && e.t < tv;
            e.head = head;
            e.pay = static_cast<uint32_t>(e.ln) | (e.q ? kIsQ : 0u) | (static_cast<uint32_t>(e.t) << kTokShift) |
                    (e.valid ? 0u : kInvalid);
            e.s = run.s;
            e.c = run.c;
            e.rex = rexs[k];
            e.bcnt = e.q ? ((before.f >> 16) & 0x7FFFu) : (before.f & 0xFFFFu);
            e.acnt = e.q ? ((afts[k] >> 16) & 0x7FFFu) : (afts[k] & 0xFFFFu);
            e.jkind = e.q ? jq : jk;
            e.v = vl[k];
            // Same token and kind as the previous position (inside the group): not a run start.
            const uint32_t pr = k ? (rr[k - 1] & kRMask) : prev_r;
            const int pt = token_of_entry(static_cast<int>(pr), a.wr_magic);
            const bool pq = static_cast<int>(pr) - pt * wr >= W;
            const bool same_run = !head && pt == e.t && pq == e.q;
            e.walk = e.valid && !same_run && (before.f & 0xFFFFu) != 0u;
            const bool prev_head = k ? ((heads >> (k - 1)) & 1u) : ((prev_raw & kFlagHead) != 0u);
            e.keep = !head || !((ends >> k) & 1u) || (p0 + k > 0 && !prev_head);
            e.kg = (before.f & 0xFFFFu) + (afts[k] & 0xFFFFu) + ((e.valid && !e.q) ? 1u : 0u);
            e.gsize = e.kg + ((before.f >> 16) & 0x7FFFu) + ((afts[k] >> 16) & 0x7FFFu) + ((e.valid && e.q) ? 1u : 0u);
            if (e.live) {
                jq += e.q ? 1u : 0u;
                jk += e.q ? 0u : 1u;
            }
            f(k, p0 + k, e);
        }
    };
    // exp of the group total: the compensated log-cumsum plus the sum after (TwoSum).
    auto group_exp = [](const Entry& e) {
        const float gs = e.s + e.rex;
        const float gb = gs - e.s;
        const float ge = (e.s - (gs - gb)) + (e.rex - gb);
        return e.valid ? expf(gs + (e.c + ge)) : 1.0f;
    };

    // ---- 4. Outputs: one pass per round over the thread's tile entries. Entry-order fields are
    // staged in LDS by entry index and copied out with 16-byte stores. Sorted-order outputs (pair
    // records, kind rows, mover records, tile bounds, the hot-group list) are written straight
    // from registers in the first pass: a thread owns consecutive sorted positions and its K (Q)
    // entries have consecutive kind indices, so these stores stay close to contiguous. With 16
    // items per thread that pass would not fit the registers; there the sorted-order outputs get
    // a pass of their own, staged tile by tile (4b).
    constexpr bool kMerged = IPT <= 8;
    // Tile bounds of the K-only row (values computed where they are used, to keep scalar
    // registers free through the rounds).
    auto tile_bounds = [&](int& nk, int& L, int64_t& tb) {
        nk = C * W;
        L = a.tile_len;
        const int ntk = (nk + L - 1) / L;
        tb = static_cast<int64_t>(c) * (ntk + 1);
        if (threadIdx.x == 0) a.tiles_k[tb + ntk] = nk;
    };
    if constexpr (kMerged) {
        int nk, L;
        int64_t tb;
        tile_bounds(nk, L, tb);
        const int npass = a.rounds.count > 0 ? a.rounds.count : 1;
        for (int rd = 0; rd < npass; ++rd) {
            const uint32_t mask = a.rounds.count > 0 ? a.rounds.mask[rd] : 0u;
            const bool sorted_pass = rd == 0;   // block-uniform
            auto stage_at = [&](int f, int idx) { return stage + a.rounds.offset[f] + idx * field_bytes(f); };
    #pragma unroll
            for (int T = 0; T < NTILE; ++T) {
                if (T >= ntiles) continue;
                // The ids of this thread's K entries in the tile (for the mover-record slots), all loads
                // in flight before the first use.
                int32_t kid[kTileItems];
                if (sorted_pass) {
                    const int p0 = T * kTile + static_cast<int>(threadIdx.x) * kTileItems;
    #pragma unroll
                    for (int k = 0; k < kTileItems; ++k) {
                        const int p = p0 + k;
                        const int r = p < n ? static_cast<int>(sval[p] & kRMask) : 0;
                        const int t = token_of_entry(r, a.wr_magic);
                        const int j = r - t * wr;
                        kid[k] = a.k_idx[cw + ((j < W && t < tv) ? t * W + j : 0)];
                    }
    #pragma unroll
                    for (int k = 0; k < kTileItems; ++k) asm volatile("" ::"v"(kid[k]));
                }
                for_tile(T, rpre[T], fpre[T], kpre[T], vv[T], [&](int k, int p, const Entry& e) {
                    if (!e.live) return;
                    const float Lv = e.s + e.c;
                    if (mask != 0u) {
                        const uint32_t packed =
                            e.valid ? (static_cast<uint32_t>(p) | min(e.acnt, kPosCountMax) << kPosAfterShift |
                                       min(e.bcnt + 1u + e.acnt, kPosCountMax) << kPosSizeShift)
                                    : static_cast<uint32_t>(p);
                        if (e.q) {
                            const int o = e.t * R + e.ln;
                            if (mask & (1u << kFLogQ)) *reinterpret_cast<float*>(stage_at(kFLogQ, o)) = Lv;
                            if (mask & (1u << kFQW)) *reinterpret_cast<float*>(stage_at(kFQW, o)) = e.v * expf(Lv);
                            if (mask & (1u << kFPosQ)) *reinterpret_cast<uint32_t*>(stage_at(kFPosQ, o)) = packed;
                            const bool ql = e.valid && e.acnt == 0;
                            if (mask & (1u << kFQLast)) *stage_at(kFQLast, o) = ql ? 1 : 0;
                            if (mask & (1u << kFQOnly)) *stage_at(kFQOnly, o) = (ql && e.bcnt == 0) ? 1 : 0;
                        } else {
                            const int o = e.t * W + e.ln;
                            const bool last = e.valid && e.acnt == 0;
                            if (mask & (1u << kFLogK)) *reinterpret_cast<float*>(stage_at(kFLogK, o)) = Lv;
                            if (mask & (1u << kFRex)) *reinterpret_cast<float*>(stage_at(kFRex, o)) = e.rex;
                            if (mask & (1u << kFCpe)) *reinterpret_cast<float*>(stage_at(kFCpe, o)) = group_exp(e);
                            if (mask & (1u << kFKEff)) *reinterpret_cast<float*>(stage_at(kFKEff, o)) = e.v * expf(Lv);
                            if (mask & (1u << kFIsLast)) *stage_at(kFIsLast, o) = last ? 1 : 0;
                            if (mask & (1u << kFIsOnly)) *stage_at(kFIsOnly, o) = (last && e.bcnt == 0) ? 1 : 0;
                            if (mask & (1u << kFPosK)) *reinterpret_cast<uint32_t*>(stage_at(kFPosK, o)) = packed;
                        }
                        if (mask & (1u << kFInv)) *reinterpret_cast<uint16_t*>(stage_at(kFInv, e.r)) = static_cast<uint16_t>(p);
                        if (mask & (1u << kFWalk)) {   // 1: walked by the pair kernel, 2: summed by its hot-group pass
                            *stage_at(kFWalk, e.r) = e.walk ? (e.kg >= static_cast<uint32_t>(a.hot_min) ? 2 : 1) : 0;
                        }
                    }
                    if (!sorted_pass) return;
                    // Hot groups (the pair kernel sums them densely): appended in any order, sorted below.
                    if (a.hot != nullptr && e.valid && e.head && e.kg >= static_cast<uint32_t>(a.hot_min)) {
                        hot_buf[atomicAdd(&hot_n, 1u)] = make_uint2(static_cast<uint32_t>(p), e.gsize);
                    }
                    if (a.rec != nullptr && e.keep) {   // pair records {payload | head, log-cumsum s, c, value}
                        a.rec[crow + p] = make_uint4(e.pay | (e.head ? kHead : 0u), __float_as_uint(e.s),
                                                     __float_as_uint(e.c), __float_as_uint(e.v));
                    }
                    const uint32_t elem = e.valid ? (e.pay | min(e.bcnt, kDistMax) << kDistShift |
                                                     (e.bcnt == 0 ? kFirst : 0u) | (e.acnt == 0 ? kLast : 0u))
                                                  : (e.pay | kFirst | kLast);
                    if (e.q) {
                        if (a.spay_q != nullptr) a.spay_q[cr + e.jkind] = static_cast<int32_t>(elem);
                    } else {
                        a.spay_k[cw + e.jkind] = static_cast<int32_t>(elem);
                        const float sc = e.valid ? e.v * expf(e.rex) : 0.0f;
                        const int64_t id = static_cast<int64_t>(kid[k]);
                        const uint32_t slot =
                            e.valid ? static_cast<uint32_t>((static_cast<uint32_t>(id - id_base) & (key_lim - 1u)) + id_base)
                                    : 0u;
                        a.krec[cw + e.jkind] = make_int4(static_cast<int32_t>(elem), static_cast<int32_t>(slot),
                                                         __float_as_int(sc), __float_as_int(group_exp(e)));
                        if (static_cast<int>(e.jkind) % L == 0) {
                            a.tiles_k[tb + static_cast<int>(e.jkind) / L] =
                                (elem & kFirst) ? static_cast<int>(e.jkind) : min(static_cast<int>(e.jkind + e.acnt + 1u), nk);
                        }
                    }
                });
            }
            if (mask != 0u) {   // block-uniform
                lds_barrier();
                copy_round(a, rd, mask, stage, dtab, crow, cr, cw, C);
                lds_barrier();
            }
        }
    } else {
        // Entry-order rounds only (4a).
        for (int rd = 0; rd < a.rounds.count; ++rd) {
            const uint32_t mask = a.rounds.mask[rd];
            auto stage_at = [&](int f, int idx) { return stage + a.rounds.offset[f] + idx * field_bytes(f); };
    #pragma unroll
            for (int T = 0; T < NTILE; ++T) {
                if (T >= ntiles) continue;
                for_tile(T, rpre[T], fpre[T], kpre[T], vv[T], [&](int k, int p, const Entry& e) {
                    if (!e.live) return;
                    const float Lv = e.s + e.c;
                    const uint32_t packed =
                        e.valid ? (static_cast<uint32_t>(p) | min(e.acnt, kPosCountMax) << kPosAfterShift |
                                   min(e.bcnt + 1u + e.acnt, kPosCountMax) << kPosSizeShift)
                                : static_cast<uint32_t>(p);
                    if (e.q) {
                        const int o = e.t * R + e.ln;
                        if (mask & (1u << kFLogQ)) *reinterpret_cast<float*>(stage_at(kFLogQ, o)) = Lv;
                        if (mask & (1u << kFQW)) *reinterpret_cast<float*>(stage_at(kFQW, o)) = e.v * expf(Lv);
                        if (mask & (1u << kFPosQ)) *reinterpret_cast<uint32_t*>(stage_at(kFPosQ, o)) = packed;
                        const bool ql = e.valid && e.acnt == 0;
                        if (mask & (1u << kFQLast)) *stage_at(kFQLast, o) = ql ? 1 : 0;
                        if (mask & (1u << kFQOnly)) *stage_at(kFQOnly, o) = (ql && e.bcnt == 0) ? 1 : 0;
                    } else {
                        const int o = e.t * W + e.ln;
                        const bool last = e.valid && e.acnt == 0;
                        if (mask & (1u << kFLogK)) *reinterpret_cast<float*>(stage_at(kFLogK, o)) = Lv;
                        if (mask & (1u << kFRex)) *reinterpret_cast<float*>(stage_at(kFRex, o)) = e.rex;
                        if (mask & (1u << kFCpe)) *reinterpret_cast<float*>(stage_at(kFCpe, o)) = group_exp(e);
                        if (mask & (1u << kFKEff)) *reinterpret_cast<float*>(stage_at(kFKEff, o)) = e.v * expf(Lv);
                        if (mask & (1u << kFIsLast)) *stage_at(kFIsLast, o) = last ? 1 : 0;
                        if (mask & (1u << kFIsOnly)) *stage_at(kFIsOnly, o) = (last && e.bcnt == 0) ? 1 : 0;
                        if (mask & (1u << kFPosK)) *reinterpret_cast<uint32_t*>(stage_at(kFPosK, o)) = packed;
                    }
                    if (mask & (1u << kFInv)) *reinterpret_cast<uint16_t*>(stage_at(kFInv, e.r)) = static_cast<uint16_t>(p);
                    if (mask & (1u << kFWalk)) {   // 1: walked by the pair kernel, 2: summed by its hot-group pass
                        *stage_at(kFWalk, e.r) = e.walk ? (e.kg >= static_cast<uint32_t>(a.hot_min) ? 2 : 1) : 0;
                    }
                });
            }
            lds_barrier();
            copy_round(a, rd, mask, stage, dtab, crow, cr, cw, C);
            lds_barrier();
        }
    }
    if constexpr (!kMerged) {
        // ---- 4b. sorted-order outputs: kind rows and krec staged per tile, pair records straight
        // from registers.
        int nk, L;
        int64_t tb;
        tile_bounds(nk, L, tb);
#pragma unroll
        for (int T = 0; T < NTILE; ++T) {
            if (T >= ntiles) continue;
            const int pbase = T * kTile;
            const int pcount = min(kTile, n - pbase);
            // Kind rows and mover records: the tile's K (Q) entries have consecutive kind indices.
            const uint32_t k0 = tile_kind[T] & 0xFFFFu, q0 = tile_kind[T] >> 16;
            const int nk_t = static_cast<int>((tile_kind[T + 1] & 0xFFFFu) - k0);
            const int nq_t = static_cast<int>((tile_kind[T + 1] >> 16) - q0);
            // Pair records (the kept ones) go out from registers: in the kind-row pass when a tile's
            // records and kind rows would fit the staging area together, else in a pass of their own.
            // (Both forms stay in the code: with either one alone the compiler spills the sort's
            // registers at 16 items per thread.)
            const int rec_bytes = a.rec != nullptr ? pcount * 16 : 0;
            const int kind_bytes = nk_t * 16 + (nk_t * 4 + 15) / 16 * 16 + nq_t * 4;
            const bool joint = rec_bytes + kind_bytes <= a.stage_bytes;   // block-uniform
            if (rec_bytes > 0 && !joint) {
                for_tile(T, rpre[T], fpre[T], kpre[T], vv[T], [&](int k, int p, const Entry& e) {
                    if (!e.live || !e.keep) return;
                    a.rec[crow + p] = make_uint4(
                        e.pay | (e.head ? kHead : 0u), __float_as_uint(e.s), __float_as_uint(e.c), __float_as_uint(e.v));
                });
                __asm__ volatile("" ::: "memory");
            }
            unsigned char* st_krec = stage;
            unsigned char* st_spk = st_krec + nk_t * 16;
            unsigned char* st_spq = st_spk + (nk_t * 4 + 15) / 16 * 16;
            for_tile(T, rpre[T], fpre[T], kpre[T], vv[T], [&](int k, int p, const Entry& e) {
                if (!e.live) return;
                if (a.hot != nullptr && e.valid && e.head && e.kg >= static_cast<uint32_t>(a.hot_min)) {
                    hot_buf[atomicAdd(&hot_n, 1u)] = make_uint2(static_cast<uint32_t>(p), e.gsize);
                }
                if (joint && rec_bytes > 0 && e.keep) {
                    a.rec[crow + p] = make_uint4(
                        e.pay | (e.head ? kHead : 0u), __float_as_uint(e.s), __float_as_uint(e.c), __float_as_uint(e.v));
                }
                const uint32_t elem = e.valid ? (e.pay | min(e.bcnt, kDistMax) << kDistShift |
                                                 (e.bcnt == 0 ? kFirst : 0u) | (e.acnt == 0 ? kLast : 0u))
                                              : (e.pay | kFirst | kLast);
                if (e.q) {
                    reinterpret_cast<uint32_t*>(st_spq)[e.jkind - q0] = elem;
                } else {
                    reinterpret_cast<uint32_t*>(st_spk)[e.jkind - k0] = elem;
                    const float sc = e.valid ? e.v * expf(e.rex) : 0.0f;
                    // The slot: the entry's id read again (the chunk's ids are cache-resident by now).
                    const int64_t id = static_cast<int64_t>(a.k_idx[cw + (e.valid ? e.t * W + e.ln : 0)]);
                    const uint32_t slot =
                        e.valid ? static_cast<uint32_t>((static_cast<uint32_t>(id - id_base) & (key_lim - 1u)) + id_base)
                                : 0u;
                    reinterpret_cast<int4*>(st_krec)[e.jkind - k0] =
                        make_int4(static_cast<int32_t>(elem), static_cast<int32_t>(slot), __float_as_int(sc),
                                  __float_as_int(group_exp(e)));
                    if (static_cast<int>(e.jkind) % L == 0) {
                        a.tiles_k[tb + static_cast<int>(e.jkind) / L] =
                            (elem & kFirst) ? static_cast<int>(e.jkind) : min(static_cast<int>(e.jkind + e.acnt + 1u), nk);
                    }
                }
            });
            lds_barrier();
            block_copy_out(a.krec + cw + k0, st_krec, nk_t, 16);
            block_copy_out(a.spay_k + cw + k0, st_spk, nk_t, 4);
            if (a.spay_q != nullptr) block_copy_out(a.spay_q + cr + q0, st_spq, nq_t, 4);
            lds_barrier();
        }
    }
    __syncthreads();   // every hot-group append is done
    if (a.hot != nullptr) {
        // The hot list in position order: each entry's rank is the number of heads before it.
        const int nh = static_cast<int>(hot_n);   // every append happened before the last barrier
        uint2* out = a.hot + static_cast<int64_t>(c) * (a.hot_cap + 1);
        for (int x = threadIdx.x; x < nh; x += kNT) {
            const uint2 me = hot_buf[x];
            int rank = 0;
            for (int y = 0; y < nh; ++y) rank += hot_buf[y].x < me.x ? 1 : 0;
            out[1 + rank] = me;
        }
        if (threadIdx.x == 0) out[0] = make_uint2(static_cast<uint32_t>(nh), 0u);
    }
}

// Pair sums. Block (chunk, triangle): the triangle of the block's matrix lives in LDS and every
// cell has one writer at a time, so no floating-point atomics are needed. Token i's entries of
// the block's kind (K for A, Q for QK) that share a slot sit next to each other in the sorted row
// and share one log-cumsum L, and so do the K entries of any earlier token j in that group. One
// term per (group, run of token i, K run of token j): w_i * k_j * exp(L_i - L_j), the run sums w
// and k taken over the run's values, L as the compensated pair (s, c).
//
// Hot groups (many K entries; listed by the sort/scan kernel) are summed densely: their runs are
// gathered into LDS tables (K runs, and the runs of the block's kind as rows, each with the number
// of K runs before it; L kept in base 2 as a compensated pair), then the threads that own row i
// sweep, group after group, the K runs before each of row i's runs, each term one hardware exp2. The other groups are walked
// by thread i from each flagged run back to the group's head. Terms reach a cell in an order fixed
// by the input (hot groups in position order, then the walks).
struct PairArgs {
    const uint4* rec;
    const uint16_t* inv;
    const uint8_t* walk;
    const uint2* hot;   // per chunk: {count, 0}, then {head position, size} in position order (NULL: none)
    float* a;
    float* qk;
    int C, W, R, first_partial, valid_last, hot_cap, tab_cap;
};

// Threads per pair block: 512, or 1024 where the LDS allows one block per compute unit anyway.
constexpr float kLog2E = 1.44269504088896340736f;
constexpr size_t kPairStaticLds = 256;   // room left for the kernel's static LDS (scan partials)
constexpr int kWalkBatch = 8;

// Hot groups per batch (a group bit in one 32-bit mask per token).
constexpr int kPairBatchGroups = 32;

// LDS of the pair kernel: the triangle, the hot list, per-group table bases, per-token group
// masks, per-group token bitmaps, the two run tables.
struct PairLds {
    size_t tri, hot, gbase, tmask, pres, ktab, rtab, total;
};
__host__ __device__ inline PairLds pair_lds_layout(int C, int hot_cap, int tab_cap) {
    auto up = [](size_t b) { return (b + 15) / 16 * 16; };
    PairLds l;
    l.tri = 0;
    l.hot = up(static_cast<size_t>(C) * (C + 1) / 2 * sizeof(float));
    l.gbase = l.hot + up(static_cast<size_t>(hot_cap) * 2 * sizeof(uint32_t) + 16);   // + batch bounds
    l.tmask = l.gbase + up(static_cast<size_t>(kPairBatchGroups + 1) * 3 * sizeof(uint32_t));
    l.pres = l.tmask + up(static_cast<size_t>(C) * sizeof(uint32_t));
    l.ktab = l.pres + static_cast<size_t>(kPairBatchGroups) * 8 * sizeof(uint32_t);
    l.rtab = l.ktab + static_cast<size_t>(tab_cap) * 16;
    l.total = l.rtab + static_cast<size_t>(tab_cap) * 16;
    return l;
}

template <int kPairThreads>
__global__ void __launch_bounds__(kPairThreads) p1_pairs_kernel(PairArgs a) {
    constexpr int kPairWaves = kPairThreads / kWave;
    extern __shared__ __align__(16) unsigned char smem[];
    const bool q = blockIdx.y == 1;
    float* out = q ? a.qk : a.a;
    if (out == nullptr) return;   // block-uniform
    const int c = blockIdx.x;
    const int C = a.C, W = a.W, R = a.R;
    const int wr = W + R;
    const int n = C * wr;
    const int tv = c >= a.first_partial ? a.valid_last : C;
    const PairLds lay = pair_lds_layout(C, a.hot_cap, a.tab_cap);
    float* tri = reinterpret_cast<float*>(smem + lay.tri);
    uint2* hl = reinterpret_cast<uint2*>(smem + lay.hot);               // hot list of the chunk
    int* bounds = reinterpret_cast<int*>(smem + lay.hot) + 2 * a.hot_cap;   // batch end, positions
    uint32_t* ubase = reinterpret_cast<uint32_t*>(smem + lay.gbase);    // batch-local first position
    uint32_t* gk = ubase + (kPairBatchGroups + 1);                       // first K-run index per group
    uint32_t* gr = gk + (kPairBatchGroups + 1);                          // first row-run index per group
    uint32_t* tmask = reinterpret_cast<uint32_t*>(smem + lay.tmask);     // batch groups with a row run of token t
    uint32_t* pres = reinterpret_cast<uint32_t*>(smem + lay.pres);       // per group: tokens with a row run
    uint4* ktab = reinterpret_cast<uint4*>(smem + lay.ktab);
    uint4* rtab = reinterpret_cast<uint4*>(smem + lay.rtab);
    const int tri_size = C * (C + 1) / 2;
    for (int e = threadIdx.x; e < tri_size; e += kPairThreads) tri[e] = 0.0f;
    const int64_t crow = static_cast<int64_t>(c) * n;
    const uint4* rec = a.rec + crow;
    const uint32_t row_q = q ? kIsQ : 0u;
    const int lane = static_cast<int>(lane_id());
    const int wave = threadIdx.x / kWave;

    // ---- Hot groups, in batches whose runs fit the tables.
    const int nh = a.hot != nullptr ? static_cast<int>(a.hot[static_cast<int64_t>(c) * (a.hot_cap + 1)].x) : 0;
    if (nh > 0) {
        const uint2* hsrc = a.hot + static_cast<int64_t>(c) * (a.hot_cap + 1) + 1;
        for (int g = threadIdx.x; g < nh; g += kPairThreads) hl[g] = hsrc[g];
    }
    __syncthreads();
    for (int g0 = 0; g0 < nh;) {
        if (threadIdx.x == 0) {   // the batch: groups g0 .. g1-1, at most tab_cap runs of each table
            int g1 = g0, runs = 0;
            uint32_t pos = 0;
            while (g1 < nh) {
                const int r = min(static_cast<int>(hl[g1].y), C);   // runs of one kind in a group <= tokens
                if (g1 > g0 && (runs + r > a.tab_cap || g1 - g0 == kPairBatchGroups)) break;
                ubase[g1 - g0] = pos;
                pos += hl[g1].y;
                runs += r;
                ++g1;
            }
            ubase[g1 - g0] = pos;
            bounds[0] = g1;
            bounds[1] = static_cast<int>(pos);
        }
        __syncthreads();
        const int g1 = bounds[0];
        const int np = bounds[1];
        const int ng = g1 - g0;
        // Thread x takes the batch positions [u0, u1) (group by group); run starts are counted, then
        // numbered with one block scan, then written.
        const int per = (np + kPairThreads - 1) / kPairThreads;
        const int u0 = min(np, static_cast<int>(threadIdx.x) * per), u1 = min(np, u0 + per);
        int g = 0;
        while (g + 1 < ng && static_cast<int>(ubase[g + 1]) <= u0) ++g;
        // Positions are read kWin at a time (all loads in flight together). Per window: the sorted
        // position, whether it starts its group, its group, and the group's end position.
        constexpr int kWin = 8;
        constexpr uint32_t kTag = kIsQ | (0xFFu << kTokShift);   // (kind, token) of an entry
        struct Cursor {
            int gg, gstart, gnext, ghead, gend;
        };
        auto cursor_at = [&](int gg) {
            Cursor cu;
            cu.gg = gg;
            cu.gstart = static_cast<int>(ubase[gg]);
            cu.gnext = static_cast<int>(ubase[gg + 1]);
            cu.ghead = static_cast<int>(hl[g0 + gg].x);
            cu.gend = cu.ghead + static_cast<int>(hl[g0 + gg].y);
            return cu;
        };
        auto window = [&](int ub, int cnt, Cursor& cu, int (&rho)[kWin], bool (&fst)[kWin], int (&grp)[kWin],
                          int (&gend)[kWin]) {
#pragma unroll
            for (int b = 0; b < kWin; ++b) {
                const int u = ub + min(b, cnt - 1);
                if (u >= cu.gnext) cu = cursor_at(cu.gg + 1);   // positions advance by at most one group
                rho[b] = cu.ghead + (u - cu.gstart);
                fst[b] = u == cu.gstart && b < cnt;
                grp[b] = cu.gg;
                gend[b] = cu.gend;
            }
        };
        for (int t = threadIdx.x; t < C; t += kPairThreads) tmask[t] = 0u;
        for (int t = threadIdx.x; t < kPairBatchGroups * 8; t += kPairThreads) pres[t] = 0u;
        uint32_t counts = 0;   // K-run starts | row-run starts << 16
        {
            Cursor cu = cursor_at(g);
            uint32_t prev = 0xFFFFFFFFu;
            for (int ub = u0; ub < u1; ub += kWin) {
                const int cnt = min(kWin, u1 - ub);
                int rho[kWin], grp[kWin], gend[kWin];
                bool fst[kWin];
                window(ub, cnt, cu, rho, fst, grp, gend);
                uint32_t x[kWin];
#pragma unroll
                for (int b = 0; b < kWin; ++b) x[b] = rec[rho[b]].x;
                if (prev == 0xFFFFFFFFu && !fst[0]) prev = rec[rho[0] - 1].x;
#pragma unroll
                for (int b = 0; b < kWin; ++b) {
                    if (b >= cnt) break;
                    const bool cont = !fst[b] && (prev & kTag) == (x[b] & kTag);
                    counts += (!(x[b] & kIsQ) && !cont) ? 1u : 0u;
                    counts += ((x[b] & kIsQ) == row_q && !cont) ? (1u << 16) : 0u;
                    prev = x[b];
                }
            }
        }
        __shared__ uint32_t psum[kPairWaves];
        uint32_t incl = counts;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t o = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += o;
        }
        if (lane == kWave - 1) psum[wave] = incl;
        __syncthreads();
        uint32_t base = incl - counts;
        for (int w = 0; w < wave; ++w) base += psum[w];
        {
            Cursor cu = cursor_at(g);
            uint32_t kx = base & 0xFFFFu, rx = base >> 16;
            uint32_t prev = 0xFFFFFFFFu;
            for (int ub = u0; ub < u1; ub += kWin) {
                const int cnt = min(kWin, u1 - ub);
                int rho[kWin], grp[kWin], gend[kWin];
                bool fst[kWin];
                window(ub, cnt, cu, rho, fst, grp, gend);
                uint4 r[kWin];
#pragma unroll
                for (int b = 0; b < kWin; ++b) r[b] = rec[rho[b]];
                // The entry after the window's last, when still in its group (a run may go on).
                const int last_rho = rho[kWin - 1];   // the window's last valid position (clamped)
                const bool more = last_rho + 1 < gend[kWin - 1];
                const uint4 nx0 = rec[more ? last_rho + 1 : last_rho];
                if (prev == 0xFFFFFFFFu && !fst[0]) prev = rec[rho[0] - 1].x;
                // Run sums inside the window, from the back: suf[b] = value of b plus the rest of its run.
                // (Elements past cnt repeat the last one, so r[kWin - 1] is the window's last entry.)
                const uint32_t last_tag = r[kWin - 1].x & kTag;
                float tail = 0.0f;
                if (more && (nx0.x & kTag) == last_tag) {
                    tail = __uint_as_float(nx0.w);
                    for (int p2 = last_rho + 2; p2 < gend[kWin - 1]; ++p2) {
                        const uint4 nx = rec[p2];
                        if ((nx.x & kTag) != last_tag) break;
                        tail = tail + __uint_as_float(nx.w);
                    }
                }
                float suf[kWin];
                float after = tail;   // the run sum that continues past element b
#pragma unroll
                for (int b = kWin - 1; b >= 0; --b) {
                    if (b >= cnt) continue;
                    suf[b] = __uint_as_float(r[b].w) + after;
                    // element b continues the run of element b-1?
                    const bool joins_prev = b > 0 && !fst[b] && (r[b].x & kTag) == (r[b - 1].x & kTag);
                    after = joins_prev ? suf[b] : 0.0f;
                }
#pragma unroll
                for (int b = 0; b < kWin; ++b) {
                    if (b >= cnt) break;
                    if (fst[b]) {   // group bases (the thread holding a group's first position)
                        gk[grp[b]] = kx;
                        gr[grp[b]] = rx;
                    }
                    const bool cont = !fst[b] && (prev & kTag) == (r[b].x & kTag);
                    prev = r[b].x;
                    if (cont) continue;
                    const bool is_k = !(r[b].x & kIsQ), is_row = (r[b].x & kIsQ) == row_q;
                    const uint32_t tok = (r[b].x >> kTokShift) & 0xFFu;
                    // L in base 2 as a compensated pair: hi = s log2(e), lo = the product's rounding error
                    // plus c log2(e). Differences of such pairs keep the exponent as accurate as (s, c).
                    const float ls = __uint_as_float(r[b].y), lc = __uint_as_float(r[b].z);
                    const float l2hi = ls * kLog2E;
                    const float l2lo = fmaf(ls, kLog2E, -l2hi) + lc * kLog2E;
                    if (is_row) {
                        rtab[rx] = make_uint4(tok | (kx << 8), __float_as_uint(suf[b]), __float_as_uint(l2hi),
                                              __float_as_uint(l2lo));
                        atomicOr(tmask + tok, 1u << grp[b]);
                        atomicOr(pres + grp[b] * 8 + (tok >> 5), 1u << (tok & 31u));
                    }
                    if (is_k) ktab[kx] = make_uint4(tok, __float_as_uint(suf[b]), __float_as_uint(l2hi), __float_as_uint(l2lo));
                    kx += is_k ? 1u : 0u;
                    rx += is_row ? 1u : 0u;
                }
            }
        }
        if (threadIdx.x == kPairThreads - 1) {   // end bases: the batch totals
            gk[ng] = (base & 0xFFFFu) + (counts & 0xFFFFu);
            gr[ng] = (base >> 16) + (counts >> 16);
        }
        __syncthreads();
        // Dense terms: kRowThreads threads own row i across every group of the batch (no barrier
        // between groups), each taking every kRowThreads-th K run of the row run's prefix,
        // kColBlock at a time (table reads, then cell reads, then cell writes: the cells of a block
        // are distinct, a group holding one K run per token). A row run's table index is its
        // group's first row index plus the group's row tokens below i.
        constexpr int kRowThreads = kPairThreads / 256, kColBlock = 8;
        for (int i = static_cast<int>(threadIdx.x) / kRowThreads; i < tv; i += kPairThreads / kRowThreads) {
            const int sub = static_cast<int>(threadIdx.x) % kRowThreads;
            float* row = tri + i * (i + 1) / 2;
            for (uint32_t gm = tmask[i]; gm != 0u; gm &= gm - 1u) {
                const int gg = __builtin_ctz(gm);
                const uint32_t* pg = pres + gg * 8;
                int below = 0;
#pragma unroll
                for (int wd = 0; wd < 8; ++wd) {
                    const uint32_t bits = pg[wd];
                    const int lo = wd * 32;
                    below += i >= lo + 32 ? __popc(bits) : (i > lo ? __popc(bits & ((1u << (i - lo)) - 1u)) : 0);
                }
                const uint32_t kb = gk[gg];
                const uint4 me = rtab[gr[gg] + below];
                const int ncol = static_cast<int>((me.x >> 8) - kb);
                const float wi = __uint_as_float(me.y), hi_i = __uint_as_float(me.z), lo_i = __uint_as_float(me.w);
                for (int c0 = sub; c0 < ncol; c0 += kRowThreads * kColBlock) {
                    uint4 kt[kColBlock];
#pragma unroll
                    for (int b = 0; b < kColBlock; ++b) kt[b] = ktab[kb + min(c0 + b * kRowThreads, ncol - 1)];
                    float term[kColBlock], cell[kColBlock];
#pragma unroll
                    for (int b = 0; b < kColBlock; ++b) {
                        // exp(L_i - L_j) = 2^((hi_i - hi_j) + (lo_i - lo_j)); the exponent is <= 0 for
                        // log-sigmoid gates, and underflow to 0 only drops terms below 2^-126.
                        term[b] = (wi * __uint_as_float(kt[b].y)) *
                                  __builtin_amdgcn_exp2f((hi_i - __uint_as_float(kt[b].z)) + (lo_i - __uint_as_float(kt[b].w)));
                        cell[b] = row[kt[b].x];
                    }
#pragma unroll
                    for (int b = 0; b < kColBlock; ++b) {
                        if (c0 + b * kRowThreads < ncol) row[kt[b].x] = cell[b] + term[b];
                    }
                }
            }
        }
        __syncthreads();   // the tables are rebuilt for the next batch
        g0 = g1;
    }

    // ---- Other groups: thread i walks its flagged runs back to the group head.
    const int i = threadIdx.x;
    if (i < tv) {
        float* row = tri + i * (i + 1) / 2;
        const int lanes = q ? R : W;
        const int r0 = i * wr + (q ? W : 0);
        const uint8_t* wf = a.walk + crow + r0;
        const uint16_t* iv = a.inv + crow + r0;
        // Token i's entries of this kind: (Q flag, token) bits of the payload.
        const uint32_t own_tag = (q ? kIsQ : 0u) | (static_cast<uint32_t>(i) << kTokShift);
        const uint32_t tag_mask = kIsQ | (0xFFu << kTokShift);
        for (int lb = 0; lb < lanes; lb += 32) {
          // The flags of up to 32 lanes, loaded together, then only the lanes walked here.
          uint32_t flags = 0;
#pragma unroll
          for (int u = 0; u < 32; ++u) {
              const int ln = lb + u;
              flags |= (ln < lanes && wf[min(ln, lanes - 1)] == 1) ? (1u << u) : 0u;
          }
          for (; flags != 0u; flags &= flags - 1u) {
            const int ln = lb + __builtin_ctz(flags);
            const int rho = iv[ln];
            const uint4 own = rec[rho];
            // Sum the run's values.
            float wi = __uint_as_float(own.w);
            for (int p = rho + 1; p < n; ++p) {
                const uint4 nx = rec[p];
                if ((nx.x & kHead) || (nx.x & tag_mask) != own_tag) break;
                wi = wi + __uint_as_float(nx.w);
            }
            const float se = __uint_as_float(own.y), ce = __uint_as_float(own.z);
            // Walk back to the head; the K runs of earlier tokens are summed, then one term each.
            int cur_j = -1;
            float kj = 0.0f, sj = 0.0f, cj = 0.0f;
            bool done = false;
            for (int top = rho - 1; !done; top -= kWalkBatch) {
                uint4 rb[kWalkBatch];
#pragma unroll
                for (int k = 0; k < kWalkBatch; ++k) rb[k] = rec[max(top - k, 0)];
#pragma unroll
                for (int k = 0; k < kWalkBatch; ++k) {
                    if (done) break;
                    const uint32_t px = rb[k].x;
                    if (!(px & (kIsQ | kInvalid))) {
                        const int jt = static_cast<int>((px >> kTokShift) & 0xFFu);
                        if (jt != cur_j) {
                            if (cur_j >= 0 && (q || cur_j != i)) {
                                row[cur_j] = row[cur_j] + (wi * kj) * expf((se - sj) + (ce - cj));
                            }
                            cur_j = jt;
                            kj = 0.0f;
                            sj = __uint_as_float(rb[k].y);
                            cj = __uint_as_float(rb[k].z);
                        }
                        kj = kj + __uint_as_float(rb[k].w);
                    }
                    done = (px & kHead) != 0;
                }
            }
            if (cur_j >= 0 && (q || cur_j != i)) row[cur_j] = row[cur_j] + (wi * kj) * expf((se - sj) + (ce - cj));
          }
        }
    }
    __syncthreads();
    const int64_t ob = static_cast<int64_t>(c) * C * C;
    if ((C & 3) == 0 && ((reinterpret_cast<uintptr_t>(out + ob) & 15u) == 0)) {
        const int c4 = C >> 2;
        for (int e = threadIdx.x; e < C * c4; e += kPairThreads) {
            const int ii = e / c4;
            const int j0 = (e - ii * c4) << 2;
            const float* trow = tri + ii * (ii + 1) / 2;
            float v4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int jj = j0 + u;
                v4[u] = (q ? jj <= ii : jj < ii) ? trow[jj] : 0.0f;
            }
            reinterpret_cast<float4*>(out + ob)[e] = make_float4(v4[0], v4[1], v4[2], v4[3]);
        }
    } else {
        for (int e = threadIdx.x; e < C * C; e += kPairThreads) {
            const int ii = e / C;
            const int jj = e - ii * C;
            out[ob + e] = (q ? jj <= ii : jj < ii) ? tri[ii * (ii + 1) / 2 + jj] : 0.0f;
        }
    }
}

// Host-side plan of one Phase-1 launch: sort items per thread, digit width, staging rounds.
struct MainPlan {
    int ipt;
    int digit_bits;
    int stage_bytes;
    size_t lds_bytes;
    Rounds rounds;
};

constexpr int kLdsTotal = 160 * 1024;
constexpr int kStaticReserve = 1024;   // static LDS of the kernel (scan totals, tile counts)

int field_count(const sdm_p1_shape* s, int f) {
    const int n = s->C * (s->W + s->R);
    return field_is_all(f) ? n : field_is_q(f) ? s->C * s->R : s->C * s->W;
}

MainPlan plan_main(const sdm_p1_shape* s, const sdm_p1_io* io, bool with_pairs_ws) {
    MainPlan m;
    const int n = s->C * (s->W + s->R);
    m.ipt = n <= kNT ? 1 : n <= 2 * kNT ? 2 : n <= 4 * kNT ? 4 : n <= 8 * kNT ? 8 : 16;
    const int np = kNT * m.ipt;
    // Sorted row, gates and (with pair sums) the chunk's hot-group list.
    const int fixed = np * 2 + 256 * static_cast<int>(sizeof(float)) +
                      (with_pairs_ws ? s->C * s->W / kHotMin * static_cast<int>(sizeof(uint2)) : 0);
    const int cap_max = (kLdsTotal - kStaticReserve - fixed) / 16 * 16;
    // Widest digit (<= 10 bits) whose per-wave counts fit beside the keys.
    int d = 10;
    while (d > 4 && np * 4 + kNW * (1 << d) * 4 > cap_max) --d;
    m.digit_bits = d;
    const int sort_bytes = np * 4 + kNW * (1 << d) * 4;
    const void* dst[kNumFields] = {io->log_k, io->rex, io->cpe, io->k_eff, io->is_last, io->is_only, io->pos_k,
                                   io->log_q, io->q_w, io->pos_q, io->q_last, io->q_only,
                                   with_pairs_ws ? io : nullptr, with_pairs_ws ? io : nullptr};
    int need = 0;
    for (int f = 0; f < kNumFields; ++f) need += (field_count(s, f) * field_bytes(f) + 15) / 16 * 16;
    // With 16 items per thread krec and both kind rows are staged per tile.
    const int sorted_bytes = m.ipt == 16 ? kTile * 20 + 32 : 0;
    int cap = max(max(sort_bytes, sorted_bytes), min(need, cap_max));
    cap = min(cap, cap_max) / 16 * 16;
    // Greedy packing of the requested fields, in order, into rounds of `cap` bytes.
    m.rounds.count = 0;
    m.rounds.flat = 0u;
    for (int r = 0; r < kMaxRounds; ++r) {
        m.rounds.mask[r] = 0u;
        m.rounds.vtotal[r] = 0;
        for (int f = 0; f < kNumFields; ++f) m.rounds.vstart[r][f] = 0x3FFFFFFF;
    }
    int used = cap;   // forces a new round for the first field
    for (int f = 0; f < kNumFields; ++f) {
        m.rounds.offset[f] = 0;
        if (dst[f] == nullptr) continue;
        const int bytes = (field_count(s, f) * field_bytes(f) + 15) / 16 * 16;
        if (used + bytes > cap) {
            if (m.rounds.count == kMaxRounds) {   // cannot happen for n <= 16384 (>= 2 fields a round)
                m.rounds.count = kMaxRounds + 1;
                return m;
            }
            ++m.rounds.count;
            used = 0;
        }
        m.rounds.offset[f] = used;
        m.rounds.mask[m.rounds.count - 1] |= 1u << f;
        m.rounds.vstart[m.rounds.count - 1][f] = used / 16;
        used += bytes;
        m.rounds.vtotal[m.rounds.count - 1] = used / 16;
    }
    m.stage_bytes = cap;
    m.lds_bytes = static_cast<size_t>(cap) + static_cast<size_t>(fixed);
    return m;
}

template <int IPT>
hipError_t launch_main(P1Args args, size_t lds, int N, hipStream_t st, hipEvent_t start, hipEvent_t stop) {
    const void* fn = reinterpret_cast<const void*>(&p1_main_kernel<IPT>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    void* kargs[] = {&args};
    return hipExtLaunchKernel(fn, dim3(N), dim3(kNT), kargs, lds, st, start, stop, 0);
}

}  // namespace

P1Workspace p1_workspace_layout(const sdm_p1_shape* s) {
    const size_t n = static_cast<size_t>(s->C) * static_cast<size_t>(s->W + s->R);
    const size_t N = static_cast<size_t>(s->N);
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    P1Workspace w;
    w.rec_off = 0;
    w.inv_off = up(N * n * sizeof(uint4));
    w.walk_off = w.inv_off + up(N * n * sizeof(uint16_t));
    w.hot_cap = s->C * s->W / kHotMin;
    w.hot_off = w.walk_off + up(N * n);
    w.total = w.hot_off + up(N * static_cast<size_t>(w.hot_cap + 1) * sizeof(uint2));
    return w;
}

size_t p1_pair_lds_min(const sdm_p1_shape* s) {
    return pair_lds_layout(s->C, s->C * s->W / kHotMin, 0).total + kPairStaticLds;
}

size_t p1_lds_bytes(const sdm_p1_shape* s, const sdm_p1_io* io) {
    return plan_main(s, io, io->a != nullptr || io->qk != nullptr).lds_bytes;
}

hipError_t p1_launch(const P1Launch& Lc, hipStream_t st) {
    const sdm_p1_shape* s = Lc.s;
    const sdm_p1_io* io = Lc.io;
    if (s->N == 0) return hipSuccess;
    const bool pairs = io->a != nullptr || io->qk != nullptr;
    P1Args a;
    a.k_idx = io->k_idx;
    a.q_idx = io->q_idx;
    a.k_val = io->k_val;
    a.q_val = io->q_val;
    a.g = io->g;
    void* fields[kNumFields] = {io->log_k, io->rex, io->cpe, io->k_eff, io->is_last, io->is_only, io->pos_k,
                                io->log_q, io->q_w, io->pos_q, io->q_last, io->q_only,
                                pairs ? Lc.inv : nullptr, pairs ? Lc.walk : nullptr};
    for (int f = 0; f < kNumFields; ++f) a.field[f] = fields[f];
    a.spay_k = io->spay_k;
    a.spay_q = io->spay_q;
    a.krec = reinterpret_cast<int4*>(io->krec);
    a.tiles_k = io->tiles_k;
    a.repeats = io->repeats;
    a.rec = pairs ? static_cast<uint4*>(Lc.rec) : nullptr;
    // Hot groups only when the pair kernel's run tables (at least C runs of each kind) fit in LDS.
    const int hot_cap = s->C * s->W / kHotMin;
    // Table capacity: as large as the blocks per compute unit that the smallest tables (C runs of
    // each kind) allow still fit; at least C when hot groups are on.
    const size_t pair_fixed = pair_lds_layout(s->C, hot_cap, 0).total + kPairStaticLds;
    const size_t pair_min = pair_fixed + static_cast<size_t>(s->C) * 32;
    const int blocks_cu = pair_min <= static_cast<size_t>(Lc.lds_max) ? static_cast<int>(Lc.lds_max / pair_min) : 0;
    const int tab_cap = blocks_cu > 0
                            ? min(4096, static_cast<int>((static_cast<size_t>(Lc.lds_max) / blocks_cu - pair_fixed) / 32))
                            : 0;
    const bool hot_on = pairs && hot_cap > 0 && tab_cap >= s->C;
    a.hot = pairs ? static_cast<uint2*>(Lc.hot) : nullptr;
    a.hot_min = hot_on ? kHotMin : 0x7FFFFFFF;
    a.hot_cap = hot_cap;
    a.C = s->C;
    a.W = s->W;
    a.R = s->R;
    a.P = s->P;
    a.key_bits = s->key_bits;
    a.first_partial = s->first_partial;
    a.valid_last = s->valid_last;
    a.tile_len = s->tile_len;
    a.stream_offset = s->stream_offset;
    a.wr_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + static_cast<uint64_t>(s->W + s->R) - 1) /
                                       static_cast<uint64_t>(s->W + s->R));
    const MainPlan m = plan_main(s, io, pairs);
    if (m.rounds.count > kMaxRounds) return hipErrorInvalidValue;
    a.digit_bits = m.digit_bits;
    a.stage_bytes = m.stage_bytes;
    a.rounds = m.rounds;
    // Flat copy-out for the rounds whose fields all have 16-byte aligned rows of whole vectors.
    for (int r = 0; r < a.rounds.count; ++r) {
        bool flat = true;
        for (int f = 0; f < kNumFields; ++f) {
            if (!(a.rounds.mask[r] & (1u << f))) continue;
            flat = flat && (reinterpret_cast<uintptr_t>(a.field[f]) & 15u) == 0 &&
                   (field_count(s, f) * field_bytes(f)) % 16 == 0;
        }
        if (flat) a.rounds.flat |= 1u << r;
    }
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (io->events != nullptr) {
        for (int k = 0; k < 4; ++k) ev[k] = io->events[k];
    }
    hipError_t e;
    switch (m.ipt) {
        case 1: e = launch_main<1>(a, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
        case 2: e = launch_main<2>(a, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
        case 4: e = launch_main<4>(a, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
        case 8: e = launch_main<8>(a, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
        default: e = launch_main<16>(a, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
    }
    if (e != hipSuccess || !pairs) return e;
    PairArgs pa;
    pa.rec = static_cast<const uint4*>(Lc.rec);
    pa.inv = static_cast<const uint16_t*>(Lc.inv);
    pa.walk = static_cast<const uint8_t*>(Lc.walk);
    pa.hot = static_cast<const uint2*>(Lc.hot);
    pa.hot_cap = hot_cap;
    pa.tab_cap = hot_on ? tab_cap : 0;
    pa.a = io->a;
    pa.qk = io->qk;
    pa.C = s->C;
    pa.W = s->W;
    pa.R = s->R;
    pa.first_partial = s->first_partial;
    pa.valid_last = s->valid_last;
    // The pair kernel on its own stream, after the sort/scan kernel, when the caller gives one.
    hipStream_t pst = st;
    if (io->pair_stream != nullptr) {
        if ((e = hipEventRecord(io->pair_ready, st)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(io->pair_stream, io->pair_ready, 0)) != hipSuccess) return e;
        pst = io->pair_stream;
    }
    const size_t lds = pair_lds_layout(s->C, hot_cap, pa.tab_cap).total;
    const int threads = blocks_cu == 1 ? 1024 : 512;
    const void* fn = threads == 1024 ? reinterpret_cast<const void*>(&p1_pairs_kernel<1024>)
                                     : reinterpret_cast<const void*>(&p1_pairs_kernel<512>);
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    void* kargs[] = {&pa};
    return hipExtLaunchKernel(fn, dim3(s->N, 2), dim3(threads), kargs, lds, pst, ev[2], ev[3], 0);
}

}  // namespace sdm
