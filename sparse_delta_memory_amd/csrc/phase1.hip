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
//   4. output sweeps: each thread recomputes its entries once per sweep, writes the sorted-order
//      outputs (kind rows, mover records, pair records, tile bounds) from registers and leaves a
//      compact record per entry in LDS at its entry index; the block then expands the records
//      into the entry-order fields with coalesced stores. One sweep when every record fits in
//      LDS, else one per kind (and token range).
// A second kernel sums the A / QK triangles.
//
// Definitions: page "sparse_delta_memory/cuda/phase1_cuda.py" (module docstring; keys and payloads
// of p1_keys_zw_kernel; the scan semantics of p1_scan_kernel; the pair terms of p1_pairs_kernel).
// Scans combine TwoSum-compensated float sums in a fixed tree; every output element has one
// writer; no floating-point atomics are used, so results are bitwise reproducible.
#include <hip/hip_ext.h>

#include <type_traits>

#include "p1_scan.hpp"
#include "sdm_device.hpp"
#include "sdm_launch.hpp"

namespace sdm {
namespace {

constexpr int kTileItems = 4;     // scan items per thread per tile
constexpr int kTile = kNT * kTileItems;
constexpr uint32_t kFlagHead = 1u << 14;   // group head, kept beside r (< 2^14) in the sorted row
constexpr uint32_t kFlagRep = 1u << 15;    // repeated K entry (its gate is not applied again)
constexpr uint32_t kRMask = kFlagHead - 1u;

// Output sweeps: the entries (kind, token range) whose records one sweep leaves in LDS.
constexpr int kMaxSweeps = 8;
constexpr uint32_t kSweepK = 1u, kSweepQ = 2u;
struct Sweeps {
    int count;
    uint32_t kinds[kMaxSweeps];
    int t0[kMaxSweeps], t1[kMaxSweeps];   // tokens [t0, t1); t0 a multiple of 4
};

// Compact record of an entry, in LDS at its entry index (arrays of a sweep): L = f32 log-cumsum,
// rex (K only), and a metadata word: sorted position (bits 0-13), min(after, 127) (14-20),
// min(peers, 127) (21-27), no own-kind peer before (28), pair-kernel walk code (29-30), valid (31).
constexpr int kMetaAfterShift = 14;
constexpr int kMetaSizeShift = 21;
constexpr uint32_t kMetaFirst = 1u << 28;
constexpr int kMetaWalkShift = 29;
constexpr uint32_t kMetaValid = 1u << 31;
constexpr uint32_t kMetaPos = (1u << 14) - 1u;
// Entry-order workspace word of the pair kernel: sorted position | kInvWalk when the entry starts
// its token's run with earlier valid K entries in an ordinary group, kInvHot when it does so in a
// hot group (walked only if the pair kernel cannot sum that group densely).
constexpr uint32_t kInvWalk = InvBits<uint16_t>::kWalk;
constexpr uint32_t kInvHot = InvBits<uint16_t>::kHot;

// Entry-order destinations, kept in an LDS table from the kernel's start to the sweeps (their
// kernel-argument copies would otherwise hold scalar registers through the sort and the scans).
enum OutPtr : int {
    kOLogK, kORex, kOCpe, kOKEff, kOIsLast, kOIsOnly, kOPosK, kOInvK,
    kOLogQ, kOQW, kOPosQ, kOQLast, kOQOnly, kOInvQ, kNumOut
};

struct P1Args {
    const void* k_idx;   // int32 or int64 ids
    const void* q_idx;
    const void* k_val;   // float32, or bfloat16 (the kernel's VBF)
    const void* q_val;
    const float* g;
    // entry-order outputs (NULL: skipped)
    float* log_k;
    float* rex;
    void* cpe;           // float32, or bfloat16 with VBF (as k_eff and q_w)
    void* k_eff;
    int8_t* is_last;
    int8_t* is_only;
    int32_t* pos_k;
    float* log_q;
    void* q_w;
    int32_t* pos_q;
    int8_t* q_last;
    int8_t* q_only;
    // pair-kernel workspace in entry order, per kind (NULL: no pair sums): the entry's sorted
    // position (bits 0-13) and kInvWalk where the pair kernel walks it
    uint16_t* inv_k;
    uint16_t* inv_q;
    int32_t* spay_k;
    int32_t* spay_q;
    int4* krec;
    int32_t* tiles_k;
    int32_t* repeats;
    int32_t* perm;       // [N, n] entry index at each sorted position (NULL: skipped)
    int32_t* status;     // debug (NULL: off): bit 0 set when a valid entry's slot id is out of range
    uint4* rec;
    uint2* hot;          // per chunk: {count, 0}, then {head position, size} of each hot group (NULL: none)
    int C, W, R, P, key_bits, first_partial, valid_last, tile_len, digit_bits;
    int stage_bytes;     // LDS before the sorted row: sort keys and counts, then the sweeps' records
    // Resident layout (rows of up to 8 items per thread, when LDS holds it): the sorted keys stay
    // in LDS through the sweeps (the mover records take their slots there) and the entries' values
    // are staged in LDS at the start (K values [C*W], then Q values [C*R]); the digit counts and
    // then the records follow them. 0: keys at 0, counts and then records over them.
    int resident;
    int vals_off;        // resident: byte offset of the staged values
    int hist_off;        // byte offsets of the digit counts and (after the scans) the records
    int rec_off;
    uint32_t vec;        // bit 0 (1): K (Q) fields take 4-entry vector stores (aligned rows)
    int hot_min;         // valid K entries that make a group hot for the pair kernel
    int hot_cap;         // hot groups one chunk can have (list entries after the count)
    uint32_t wr_magic;   // ceil(2^32 / (W + R)): r / (W + R) == umulhi(r, wr_magic) for r < 2^17
    int64_t stream_offset;
    Sweeps sweeps;
};

// Stable LSD radix sort of the block's kNT * IPT (key, value) pairs over key bits [0, bits), in
// the fewest passes of at most `dmax` bits, the bits shared out evenly among them. Items live in registers in striped order (item k of lane l of wave
// w is element w * 64 * IPT + k * 64 + l). Per digit: ranks inside the wave from ballot-built
// peer masks, slice by slice (equal digits keep element order); per-wave digit counts in LDS
// (rows of 2^dmax + 1); one block scan over (digit, wave) gives every (wave, digit) its start; a
// scatter into skey / sval. On return skey / sval hold the sorted sequence.
template <int IPT>
__device__ void block_radix_sort(uint32_t (&key)[IPT], uint32_t (&val)[IPT], int bits, int dmax, uint32_t* skey,
                                 uint16_t* sval, uint32_t* hist, uint32_t* wsum, uint32_t& phase) {
    const int lane = static_cast<int>(lane_id());
    const int w = threadIdx.x / kWave;
    const int stride = (1 << dmax) + 1;   // rows padded by a word: the (digit, wave) scan spreads over the banks
    uint32_t* my_hist = hist + w * stride;
    const int passes = (bits + dmax - 1) / dmax;
    const int width = (bits + passes - 1) / passes;   // digits of (nearly) equal width, at most dmax
    for (int pass = 0; pass < passes; ++pass) {
        const int sh = pass * width;
        const int db = min(width, bits - sh);
        const int nd = 1 << db;
        const uint32_t dmask = static_cast<uint32_t>(nd - 1);
        for (int d = lane; d < nd; d += kWave) my_hist[d] = 0u;
        lds_barrier();
        // The rank inside the wave (< 2^16) rides in the upper half of val (values are < 2^16).
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const uint32_t d = (key[k] >> sh) & dmask;
            uint32_t below, cnt;
            digit_peers(d, db, below, cnt);
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
        uint32_t run = block_exclusive_add(local, wsum, phase, tot);
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

// LG: gates per (token, K lane), [N, C, W], read from global memory where a scan needs one;
// otherwise per token, [N, C], staged in LDS. ID64: slot ids are int64 (else int32).
template <int IPT, bool LG, bool ID64, bool VBF>
__global__ void __launch_bounds__(kNT) p1_main_kernel(P1Args a) {
    constexpr int NP = kNT * IPT;
    constexpr int NTILE = (NP + kTile - 1) / kTile;
    // Products of tokens and lane counts: at 16 items per thread on the full-rate 24-bit multiply;
    // at fewer items the plain multiply, which leaves the compiler's scalar registers in a better
    // state there (measured: with the 24-bit form it spilled far more of them into vector lanes).
    auto imul = [](int t, int m) {
        if constexpr (IPT >= 16) {
            return mul24(t, m);
        } else {
            return t * m;
        }
    };
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t* skey = reinterpret_cast<uint32_t*>(smem);                   // sort keys
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + a.hist_off);      // digit counts
    unsigned char* stage = smem + a.rec_off;                              // records, after the scans
    float* vals_k = reinterpret_cast<float*>(smem + a.vals_off);          // resident: staged values
    uint16_t* sval = reinterpret_cast<uint16_t*>(smem + a.stage_bytes);
    float* gates = reinterpret_cast<float*>(smem + a.stage_bytes + NP * 2);
    __shared__ Seg wtot[2 * kNW];
    __shared__ uint32_t wsum[2 * kNW];
    // Alternation of the scan-total buffers, one count per buffer pair (the same in every thread).
    uint32_t seg_phase = 0, add_phase = 0;
    __shared__ uint32_t tile_kind[NTILE + 1];   // kind counts (K | Q << 16) before each tile
    __shared__ uint32_t hot_n;                   // hot groups found so far
    __shared__ uint64_t optr[kNumOut];           // entry-order destinations (0: skipped)
    uint2* hot_buf = reinterpret_cast<uint2*>(smem + a.stage_bytes + NP * 2 + 256 * sizeof(float));

    const int c = blockIdx.x;
    const int C = a.C, W = a.W, R = a.R;
    float* vals_q = vals_k + ((C * W + 3) & ~3);
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
    // A tile position as an index of the sorted row's LDS arrays (NP entries, every one written by
    // the sort): positions past the row are read there too, and their values are not used; tiles
    // longer than the row (fewer than 4 items per thread) read its last entry instead.
    auto in_row = [](int p) {
        if constexpr (NP % kTile == 0) {
            return p;
        } else {
            return min(p, NP - 1);
        }
    };

    if constexpr (!LG) {
        for (int t = threadIdx.x; t < C; t += kNT) gates[t] = t < tv ? a.g[static_cast<int64_t>(c) * C + t] : 0.0f;
    }
    // The gate of valid token t's K lane j (the scans read it for non-repeated valid K entries only).
    auto gate = [&](int t, int j) -> float {
        if constexpr (LG) {
            return a.g[cw + imul(t, W) + j];
        } else {
            return gates[t];
        }
    };
    if (threadIdx.x == 0) hot_n = 0u;
    {
        const void* outs[kNumOut] = {a.log_k, a.rex, a.cpe, a.k_eff, a.is_last, a.is_only, a.pos_k, a.inv_k,
                                     a.log_q, a.q_w, a.pos_q, a.q_last, a.q_only, a.inv_q};
#pragma unroll
        for (int o = 0; o < kNumOut; ++o) {
            if (threadIdx.x == o) optr[o] = reinterpret_cast<uintptr_t>(outs[o]);
        }
    }

    // ---- 1. keys (element i of the striped layout is entry r = i) and the sort.
    {
        uint32_t key[IPT], val[IPT];
        int64_t ids[IPT];
        // Every item loads (padding items re-read entry 0) before any id is used: the asm below
        // keeps the compiler from sinking a load into the select that uses it, where each load
        // would get a wait of its own.
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const int i = w * kWave * IPT + k * kWave + lane;
            val[k] = static_cast<uint32_t>(i);
            const int ic = i < n ? i : 0;
            const int t = token_of_entry(ic, a.wr_magic);
            const int j = ic - imul(t, wr);
            ids[k] = load_id<ID64>(j < W ? a.k_idx : a.q_idx, j < W ? cw + imul(t, W) + j : cr + imul(t, R) + (j - W));
        }
        // Resident layout: the entries' values in entry order (coalesced, issued beside the ids;
        // the invalid tokens' values, which may be anything, are not used).
        float vk[IPT], vq[IPT];   // (C*W, C*R < IPT * kNT)
        const bool res = IPT <= 8 && a.resident;   // block-uniform
        if (res) {
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int i = static_cast<int>(threadIdx.x) + k * kNT;
                vk[k] = load_val(a.k_val, cw + min(i, C * W - 1), VBF);
                vq[k] = load_val(a.q_val, cr + min(i, C * R - 1), VBF);
            }
        }
#pragma unroll
        for (int k = 0; k < IPT; ++k) asm volatile("" ::"v"(ids[k]));   // (64-bit ids: a register pair)
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const int i = w * kWave * IPT + k * kWave + lane;
            const int t = token_of_entry(i < n ? i : 0, a.wr_magic);
            const uint32_t kv =
                t < tv ? static_cast<uint32_t>(ids[k] - id_base) & (key_lim - 1u) : key_lim;
            key[k] = i < n ? kv : pad_key;
        }
        if (a.status != nullptr) {   // debug: every valid entry's local slot in [0, 2^key_bits), id >= 0
            bool bad = false;
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int i = w * kWave * IPT + k * kWave + lane;
                const int t = token_of_entry(i < n ? i : 0, a.wr_magic);
                const int64_t local = ids[k] - id_base;
                bad = bad || (i < n && t < tv && (ids[k] < 0 || local < 0 || local >= static_cast<int64_t>(key_lim)));
            }
            if (__any(bad) && lane == 0) atomicOr(a.status, 1);
        }
        if (res) {
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int i = static_cast<int>(threadIdx.x) + k * kNT;
                if (i < C * W) vals_k[i] = i < tv * W ? vk[k] : 0.0f;
                if (i < C * R) vals_q[i] = i < tv * R ? vq[k] : 0.0f;
            }
        }
        // Invalid entries need one more key bit only in a ragged chunk.
        block_radix_sort<IPT>(key, val, tv < C ? kb + 1 : kb, a.digit_bits, skey, sval, hist, wsum, add_phase);
    }

    // Per-thread state carried from the scans to the output sweeps (registers, tile-indexed).
    Seg rpre[NTILE], fpre[NTILE];
    uint32_t kpre[NTILE];
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
                const uint32_t kv = skey[in_row(p)], sv = sval[in_row(p)];
                kk[k] = p < n ? kv : pad_key;
                rr[k] = p < n ? (sv & kRMask) : 0u;
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
                const int j = static_cast<int>(rr[k]) - imul(t, wr);
                const bool is_k = valid && j < W;
                const int pt = token_of_entry(static_cast<int>(pr), a.wr_magic);
                const int pj = static_cast<int>(pr) - imul(pt, wr);
                const bool rep = !head && is_k && pj < W && pt == t;
                heads |= (head ? 1u : 0u) << k;
                reps |= (rep ? 1u : 0u) << k;
                x[k] = (is_k && !rep) ? gate(t, j) : 0.0f;
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
                const bool q = static_cast<int>(rr[k]) - imul(t, wr) >= W;
                agg = seg_combine(agg, Seg{x[k], 0.0f, (valid ? (q ? kSegQOne : 1u) : 0u) |
                                                           (((ends >> k) & 1u) ? kSegHead : 0u)});
            }
            Seg total;
            rpre[T] = seg_combine(rcarry, block_exclusive_seg<true>(agg, wtot, seg_phase, total));
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
    if (a.perm != nullptr) {   // the sorted order itself: entry index at each sorted position
        for (int p = threadIdx.x; p < n; p += kNT) a.perm[crow + p] = static_cast<int32_t>(sval[p] & kRMask);
    }

    // The thread index as the recomputations see it: each output sweep makes it opaque again, so the
    // compiler cannot hoist per-position address arithmetic out of the sweeps (registers it would
    // hold through them).
    int otid = static_cast<int>(threadIdx.x);
    // The tile's entries as the scans see them, from the flagged sorted row.
    auto load_tile = [&](int T, uint32_t (&rr)[kTileItems], float (&x)[kTileItems], uint32_t& heads,
                         uint32_t& ends) {
        const int p0 = T * kTile + otid * kTileItems;
        heads = 0;
        ends = 0;
#pragma unroll
        for (int k = 0; k < kTileItems; ++k) {
            const int p = p0 + k;
            const uint32_t sv = sval[in_row(p)];
            rr[k] = p < n ? sv : kFlagHead;   // padding: a group of its own
            const int r = static_cast<int>(rr[k] & kRMask);
            const int t = token_of_entry(r, a.wr_magic);
            const bool q = r - imul(t, wr) >= W;
            const bool valid = p < n && t < tv;
            x[k] = (valid && !q && !(rr[k] & kFlagRep)) ? gate(t, r - imul(t, wr)) : 0.0f;
            heads |= ((rr[k] & kFlagHead) ? 1u : 0u) << k;
        }
        const int pn = p0 + kTileItems;
        const uint32_t svn = sval[min(pn, NP - 1)];
        const bool next_head = pn >= n || (svn & kFlagHead);
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
        const bool q = r - imul(t, wr) >= W;
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
                if (p0 + k < n) kind_cnt += (r - imul(t, wr) >= W) ? kSegQOne : 1u;
            }
            Seg total;
            fpre[T] = seg_combine(fcarry, block_exclusive_seg<false>(agg, wtot, seg_phase, total));
            fcarry = seg_combine(fcarry, total);
            uint32_t kind_total;
            kpre[T] = kind_carry + block_exclusive_add(kind_cnt, wsum, add_phase, kind_total);
            if (threadIdx.x == 0) tile_kind[T] = kind_carry;
            kind_carry += kind_total;
        }
        if (threadIdx.x == 0) tile_kind[ntiles] = kind_carry;
        uint32_t rep_total;
        (void)block_exclusive_add(repeat_count, wsum, add_phase, rep_total);
        if (threadIdx.x == 0 && a.repeats != nullptr) a.repeats[c] = static_cast<int32_t>(rep_total);
    }
    lds_barrier();   // LDS only: the repeats (and perm) stores stay in flight; nothing here reads them

    // Recomputes the four entries of tile T owned by this thread and calls f(k, entry).
    auto for_tile = [&](int T, const Seg& rp, const Seg& fp, uint32_t kp, const float (&vl)[kTileItems], auto&& f) {
        const int p0 = T * kTile + otid * kTileItems;
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
        const uint32_t svp = sval[in_row(max(p0 - 1, 0))];
        const uint32_t prev_raw = p0 > 0 && p0 <= n ? svp : (0xFFFFu & ~kFlagHead);
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
            const int j = e.r - imul(e.t, wr);
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
            // (an invalid token's value, which may be anything, is dropped here, where the entry is
            // first used: a select right after the loads would wait for them before the recompute)
            e.v = e.valid ? vl[k] : 0.0f;
            // Same token and kind as the previous position (inside the group): not a run start.
            const uint32_t pr = k ? (rr[k - 1] & kRMask) : prev_r;
            const int pt = token_of_entry(static_cast<int>(pr), a.wr_magic);
            const bool pq = static_cast<int>(pr) - imul(pt, wr) >= W;
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

    // ---- 4. Outputs, in sweeps. A sweep recomputes the thread's entries from its tile prefixes;
    // for the entries of the sweep (its kinds, its token range) it writes the sorted-order outputs
    // straight from registers (a thread owns consecutive sorted positions, and its K (Q) entries
    // have consecutive kind indices, so these stores stay close to contiguous) and leaves a
    // compact record in LDS at the entry's index. After a barrier the block expands the records
    // into the entry-order fields, each thread four consecutive entries at a time.
    // Tile bounds of the K-only row (values computed where they are used, to keep scalar
    // registers free through the sweeps).
    auto tile_bounds = [&](int& nk, int& L, int64_t& tb) {
        nk = C * W;
        L = a.tile_len;
        const int ntk = (nk + L - 1) / L;
        tb = static_cast<int64_t>(c) * (ntk + 1);
    };
    if (threadIdx.x == 0) {
        int nk, L;
        int64_t tb;
        tile_bounds(nk, L, tb);
        a.tiles_k[tb + (nk + L - 1) / L] = nk;
    }
    // One sweep over tokens [t0, t1) of the kinds KINDS (a compile-time set: a sweep of one kind
    // carries only that kind's code, which keeps registers free at 16 items per thread).
    auto sweep = [&](auto kinds_c, int t0, int t1) {
        constexpr uint32_t kinds = decltype(kinds_c)::value;
        constexpr bool sk = (kinds & kSweepK) != 0u, sq = (kinds & kSweepQ) != 0u;
        asm volatile("" : "+v"(otid));
        // Record arrays of the sweep (16-byte aligned, lengths padded to 4 entries).
        const int nke = sk ? (t1 - t0) * W : 0, nqe = sq ? (t1 - t0) * R : 0;
        const int nkp = (nke + 3) & ~3, nqp = (nqe + 3) & ~3;
        float* kl = reinterpret_cast<float*>(stage);
        float* kx = kl + nkp;
        uint32_t* km = reinterpret_cast<uint32_t*>(kx + nkp);
        float* ql = reinterpret_cast<float*>(km + nkp);
        uint32_t* qm = reinterpret_cast<uint32_t*>(ql + nqp);
#pragma unroll
        for (int T = 0; T < NTILE; ++T) {
            if (T >= ntiles) continue;
            // The values of this thread's entries in the tile and the ids of its K entries (for the
            // mover-record slots), issued before the tile's recomputation (their waits fall at the
            // first use, inside it).
            int32_t kid[kTileItems];
            float vl[kTileItems];
            const bool res = IPT <= 8 && a.resident;   // block-uniform
            {
                const int p0 = T * kTile + static_cast<int>(threadIdx.x) * kTileItems;
#pragma unroll
                for (int k = 0; k < kTileItems; ++k) {
                    const int p = p0 + k;
                    const uint32_t sv = sval[in_row(p)];
                    const int r = p < n ? static_cast<int>(sv & kRMask) : 0;
                    const int t = token_of_entry(r, a.wr_magic);
                    const int j = r - imul(t, wr);
                    const bool q = j >= W;
                    if (res) {   // staged values (zero for invalid tokens); the slot from the sorted key
                        vl[k] = q ? vals_q[imul(t, R) + (j - W)] : vals_k[imul(t, W) + j];
                        if constexpr (sk) kid[k] = static_cast<int32_t>(p < n ? skey[p] : 0u);
                    } else {
                        // Selects of the array and of the element (a K entry's index in its kind's rows
                        // is t W + j = r - t R, a Q entry's t R + j - W = r - (t + 1) W), then one load.
                        // At 16 items per thread the compiler's branch over the two address forms
                        // measured faster; at fewer items the selects (far fewer scalar registers
                        // spilled into vector lanes).
                        const int ek = r - imul(t, R);
                        if constexpr (IPT >= 16) {
                            // (a sweep of one kind loads only that kind's values: the others are
                            // never used in it)
                            using VT = std::conditional_t<VBF, uint16_t, float>;
                            if ((sk && !sq && q) || (sq && !sk && !q)) {
                                vl[k] = 0.0f;
                            } else {
                                const VT* vp = q ? static_cast<const VT*>(a.q_val) + cr + imul(t, R) + (j - W)
                                                 : static_cast<const VT*>(a.k_val) + cw + ek;
                                vl[k] = load_val(vp, 0, VBF);
                            }
                        } else {
                            const int64_t e = q ? cr + (r - imul(t + 1, W)) : cw + ek;
                            const uintptr_t vb = q ? reinterpret_cast<uintptr_t>(a.q_val) : reinterpret_cast<uintptr_t>(a.k_val);
                            vl[k] = load_val(reinterpret_cast<const void*>(vb), e, VBF);
                        }
                        if constexpr (sk) kid[k] = static_cast<int32_t>(load_id<ID64>(a.k_idx, cw + ((!q && t < tv) ? ek : 0)));
                    }
                }
            }
            for_tile(T, rpre[T], fpre[T], kpre[T], vl, [&](int k, int p, const Entry& e) {
                if (!e.live || (sk && !sq && e.q) || (sq && !sk && !e.q) || e.t < t0 || e.t >= t1) return;
                const uint32_t walk = e.walk ? (e.kg >= static_cast<uint32_t>(a.hot_min) ? 2u : 1u) : 0u;
                const uint32_t meta = static_cast<uint32_t>(p) | min(e.acnt, kPosCountMax) << kMetaAfterShift |
                                      min(e.bcnt + 1u + e.acnt, kPosCountMax) << kMetaSizeShift |
                                      (e.bcnt == 0u ? kMetaFirst : 0u) | walk << kMetaWalkShift |
                                      (e.valid ? kMetaValid : 0u);
                const float Lv = e.s + e.c;
                // Hot groups (the pair kernel sums them densely): appended in any order, sorted below.
                if (a.hot != nullptr && e.valid && e.head && e.kg >= static_cast<uint32_t>(a.hot_min)) {
                    hot_buf[atomicAdd(&hot_n, 1u)] = make_uint2(static_cast<uint32_t>(p), e.gsize);
                }
                if (a.rec != nullptr && e.keep) {   // pair records {payload | head, log-cumsum s, c, value}
                    gstore<u32x4>(a.rec + crow, static_cast<uint32_t>(p),
                                  u32x4{e.pay | (e.head ? kHead : 0u), __float_as_uint(e.s), __float_as_uint(e.c),
                                        __float_as_uint(e.v)});
                }
                const uint32_t elem = e.valid ? (e.pay | min(e.bcnt, kDistMax) << kDistShift |
                                                 (e.bcnt == 0 ? kFirst : 0u) | (e.acnt == 0 ? kLast : 0u))
                                              : (e.pay | kFirst | kLast);
                if (sq && (!sk || e.q)) {
                    const int o = imul(e.t - t0, R) + e.ln;
                    ql[o] = Lv;
                    qm[o] = meta;
                    if (a.spay_q != nullptr) gstore<uint32_t>(a.spay_q + cr, e.jkind, elem);
                } else {
                    const int o = imul(e.t - t0, W) + e.ln;
                    kl[o] = Lv;
                    kx[o] = e.rex;
                    km[o] = meta;
                    gstore<uint32_t>(a.spay_k + cw, e.jkind, elem);
                    const float sc = e.valid ? e.v * expf(e.rex) : 0.0f;
                    // kid: the entry's id, or (resident layout) its sorted key, the local slot.
                    const uint32_t local = res ? static_cast<uint32_t>(kid[k])
                                               : static_cast<uint32_t>(static_cast<int64_t>(kid[k]) - id_base) & (key_lim - 1u);
                    const uint32_t slot = e.valid ? static_cast<uint32_t>(local + id_base) : 0u;
                    gstore<u32x4>(a.krec + cw, e.jkind,
                                  u32x4{elem, slot, __float_as_uint(sc), val_bits32(group_exp(e), VBF)});
                    int nk, L;
                    int64_t tb;
                    tile_bounds(nk, L, tb);
                    // Does the entry start a tile (and which)? A power-of-two tile length (a uniform
                    // test) takes a mask and a shift instead of a division.
                    const uint32_t uL = static_cast<uint32_t>(L);
                    bool tile_start;
                    uint32_t ti;
                    if ((uL & (uL - 1u)) == 0u) {
                        tile_start = (e.jkind & (uL - 1u)) == 0u;
                        ti = e.jkind >> __builtin_ctz(uL);
                    } else {
                        tile_start = e.jkind % uL == 0u;
                        ti = e.jkind / uL;
                    }
                    if (tile_start) {
                        gstore<int32_t>(a.tiles_k + tb, ti,
                                        (elem & kFirst) ? static_cast<int>(e.jkind)
                                                        : min(static_cast<int>(e.jkind + e.acnt + 1u), nk));
                    }
                }
            });
        }
        lds_barrier();
        // Entry-order fields from the records: entries i0 .. i0 + 3 of the sweep's kind rows.
        auto pos_of = [](uint32_t m) {
            const uint32_t p = m & kMetaPos;
            return (m & kMetaValid) ? (p | ((m >> kMetaAfterShift) & kPosCountMax) << kPosAfterShift |
                                       ((m >> kMetaSizeShift) & kPosCountMax) << kPosSizeShift)
                                    : p;
        };
        auto is_last_of = [](uint32_t m) { return (m & kMetaValid) && ((m >> kMetaAfterShift) & kPosCountMax) == 0u; };
        // A destination from the table, as a wave-uniform pointer (nullptr: skipped).
        // The sweep's first entry of the row is element `first` (es bytes each) of the chunk's row.
        auto out_ptr = [&](int o, int64_t first, int es) {
            const uint64_t v = optr[o];
            const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
            const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
            const uintptr_t b = static_cast<uintptr_t>(lo) | static_cast<uintptr_t>(hi) << 32;
            return b != 0 ? reinterpret_cast<void*>(b + static_cast<uintptr_t>(first * es)) : nullptr;
        };
        if constexpr (sk) {
            const int64_t gb = cw + static_cast<int64_t>(t0) * W;   // the chunk's entry index of record 0
            void* const log_k = out_ptr(kOLogK, gb, 4);
            void* const rex_o = out_ptr(kORex, gb, 4);
            const int ves = (VBF ? 2 : 4);   // value-typed fields: cpe, k_eff
            void* const cpe_o = out_ptr(kOCpe, gb, ves);
            void* const k_eff = out_ptr(kOKEff, gb, ves);
            void* const is_last = out_ptr(kOIsLast, gb, 1);
            void* const is_only = out_ptr(kOIsOnly, gb, 1);
            void* const pos_k = out_ptr(kOPosK, gb, 4);
            void* const inv_k = out_ptr(kOInvK, gb, 2);
            const bool vec = (a.vec & 1u) != 0u;
            for (int i0 = 4 * static_cast<int>(threadIdx.x); i0 < nke; i0 += 4 * kNT) {
                const int cnt = min(4, nke - i0);
                const f32x4 L4 = *reinterpret_cast<const f32x4*>(kl + i0);
                const f32x4 X4 = *reinterpret_cast<const f32x4*>(kx + i0);
                const u32x4 M4 = *reinterpret_cast<const u32x4*>(km + i0);
                const uint32_t g = static_cast<uint32_t>(i0);
                f32x4 v4;
                if (IPT <= 8 && a.resident) {   // (one sweep from token 0 here: record i is K entry i)
                    v4 = *reinterpret_cast<const f32x4*>(vals_k + g);
                } else if (vec && cnt == 4) {
                    v4 = load_val4(a.k_val, gb + g, VBF);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) v4[u] = load_val(a.k_val, gb + g + min(u, cnt - 1), VBF);
                }
                f32x4 cp, ke;
                u32x4 ps;
                uint32_t fl = 0u, fo = 0u;
                uint32_t iw[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t m = M4[u];
                    const bool valid = (m & kMetaValid) != 0u;
                    cp[u] = valid ? expf(L4[u] + X4[u]) : 1.0f;
                    ke[u] = valid ? v4[u] * expf(L4[u]) : 0.0f;
                    ps[u] = pos_of(m);
                    const bool last = is_last_of(m);
                    fl |= (last ? 1u : 0u) << (8 * u);
                    fo |= ((last && (m & kMetaFirst)) ? 1u : 0u) << (8 * u);
                    const uint32_t wc = (m >> kMetaWalkShift) & 3u;
                    iw[u] = (m & kMetaPos) | (wc == 1u ? kInvWalk : 0u) | (wc == 2u ? kInvHot : 0u);
                }
                if (vec && cnt == 4) {   // (non-temporal: nothing in the step reads these fields back;
                                         // the pair kernel reads inv_k, which keeps plain stores)
                    const uint32_t g4 = g / 4;
                    if (log_k != nullptr) gstore_nt<f32x4>(log_k, g4, L4);
                    if (rex_o != nullptr) gstore_nt<f32x4>(rex_o, g4, X4);
                    if (cpe_o != nullptr) store_val4(cpe_o, g4, cp, VBF);
                    if (k_eff != nullptr) store_val4(k_eff, g4, ke, VBF);
                    if (pos_k != nullptr) gstore_nt<u32x4>(pos_k, g4, ps);
                    if (is_last != nullptr) gstore_nt<uint32_t>(is_last, g4, fl);
                    if (is_only != nullptr) gstore_nt<uint32_t>(is_only, g4, fo);
                    if (inv_k != nullptr) gstore<u32x2>(inv_k, g4, u32x2{iw[0] | iw[1] << 16, iw[2] | iw[3] << 16});
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (u >= cnt) break;
                        if (log_k != nullptr) gstore<float>(log_k, g + u, L4[u]);
                        if (rex_o != nullptr) gstore<float>(rex_o, g + u, X4[u]);
                        if (cpe_o != nullptr) store_val(cpe_o, g + u, cp[u], VBF);
                        if (k_eff != nullptr) store_val(k_eff, g + u, ke[u], VBF);
                        if (pos_k != nullptr) gstore<uint32_t>(pos_k, g + u, ps[u]);
                        if (is_last != nullptr) gstore<uint8_t>(is_last, g + u, static_cast<uint8_t>((fl >> (8 * u)) & 1u));
                        if (is_only != nullptr) gstore<uint8_t>(is_only, g + u, static_cast<uint8_t>((fo >> (8 * u)) & 1u));
                        if (inv_k != nullptr) gstore<uint16_t>(inv_k, g + u, static_cast<uint16_t>(iw[u]));
                    }
                }
            }
        }
        if constexpr (sq) {
            const int64_t gb = cr + static_cast<int64_t>(t0) * R;
            void* const log_q = out_ptr(kOLogQ, gb, 4);
            void* const q_w = out_ptr(kOQW, gb, (VBF ? 2 : 4));
            void* const pos_q = out_ptr(kOPosQ, gb, 4);
            void* const q_last = out_ptr(kOQLast, gb, 1);
            void* const q_only = out_ptr(kOQOnly, gb, 1);
            void* const inv_q = out_ptr(kOInvQ, gb, 2);
            const bool vec = (a.vec & 2u) != 0u;
            for (int i0 = 4 * static_cast<int>(threadIdx.x); i0 < nqe; i0 += 4 * kNT) {
                const int cnt = min(4, nqe - i0);
                const f32x4 L4 = *reinterpret_cast<const f32x4*>(ql + i0);
                const u32x4 M4 = *reinterpret_cast<const u32x4*>(qm + i0);
                const uint32_t g = static_cast<uint32_t>(i0);
                f32x4 v4;
                if (IPT <= 8 && a.resident) {
                    v4 = *reinterpret_cast<const f32x4*>(vals_q + g);
                } else if (vec && cnt == 4) {
                    v4 = load_val4(a.q_val, gb + g, VBF);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) v4[u] = load_val(a.q_val, gb + g + min(u, cnt - 1), VBF);
                }
                f32x4 qw;
                u32x4 ps;
                uint32_t fl = 0u, fo = 0u;
                uint32_t iw[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t m = M4[u];
                    const bool valid = (m & kMetaValid) != 0u;
                    qw[u] = valid ? v4[u] * expf(L4[u]) : 0.0f;
                    ps[u] = pos_of(m);
                    const bool last = is_last_of(m);
                    fl |= (last ? 1u : 0u) << (8 * u);
                    fo |= ((last && (m & kMetaFirst)) ? 1u : 0u) << (8 * u);
                    const uint32_t wc = (m >> kMetaWalkShift) & 3u;
                    iw[u] = (m & kMetaPos) | (wc == 1u ? kInvWalk : 0u) | (wc == 2u ? kInvHot : 0u);
                }
                if (vec && cnt == 4) {
                    const uint32_t g4 = g / 4;
                    if (log_q != nullptr) gstore_nt<f32x4>(log_q, g4, L4);
                    if (q_w != nullptr) store_val4(q_w, g4, qw, VBF);
                    if (pos_q != nullptr) gstore_nt<u32x4>(pos_q, g4, ps);
                    if (q_last != nullptr) gstore_nt<uint32_t>(q_last, g4, fl);
                    if (q_only != nullptr) gstore_nt<uint32_t>(q_only, g4, fo);
                    if (inv_q != nullptr) gstore<u32x2>(inv_q, g4, u32x2{iw[0] | iw[1] << 16, iw[2] | iw[3] << 16});
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (u >= cnt) break;
                        if (log_q != nullptr) gstore<float>(log_q, g + u, L4[u]);
                        if (q_w != nullptr) store_val(q_w, g + u, qw[u], VBF);
                        if (pos_q != nullptr) gstore<uint32_t>(pos_q, g + u, ps[u]);
                        if (q_last != nullptr) gstore<uint8_t>(q_last, g + u, static_cast<uint8_t>((fl >> (8 * u)) & 1u));
                        if (q_only != nullptr) gstore<uint8_t>(q_only, g + u, static_cast<uint8_t>((fo >> (8 * u)) & 1u));
                        if (inv_q != nullptr) gstore<uint16_t>(inv_q, g + u, static_cast<uint16_t>(iw[u]));
                    }
                }
            }
        }
        lds_barrier();   // the records are read before the next sweep writes its own
    };
    if constexpr (IPT <= 8) {   // every record fits in LDS (the host checks): one sweep
        sweep(std::integral_constant<uint32_t, kSweepK | kSweepQ>{}, 0, C);
    } else {   // one kind per sweep (a planned joint sweep runs as its K part, then its Q part)
        for (int sw = 0; sw < a.sweeps.count; ++sw) {
            const uint32_t kinds = a.sweeps.kinds[sw];
            if (kinds & kSweepK) sweep(std::integral_constant<uint32_t, kSweepK>{}, a.sweeps.t0[sw], a.sweeps.t1[sw]);
            if (kinds & kSweepQ) sweep(std::integral_constant<uint32_t, kSweepQ>{}, a.sweeps.t0[sw], a.sweeps.t1[sw]);
        }
    }
    lds_barrier();   // every hot-group append is done (the sweeps' global stores stay in flight)
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
// Hot groups (many K entries; listed by the sort/scan kernel) are summed as a dense contraction. A
// token has at most one run of each kind in a group, and earlier tokens come first in it, so a
// group's terms are the lower triangle of the outer product x y^T with x[i] = w_i 2^(L_i - c) over
// the row runs and y[j] = k_j 2^(c - L_j) over the K runs (L in base 2 as a compensated pair, c
// the midpoint of the group's L range, so neither factor leaves the float range). A batch of hot
// groups fills x and y tables in LDS; each thread then adds sum_g x_g y_g^T into its own 4 x 4
// blocks of the triangle. A group whose L range is too wide for this is walked instead, as are the
// other groups: thread i walks each flagged run back to the group's head. Terms reach a cell in an
// order fixed by the input (hot batches in position order, then the walks).
struct PairArgs {
    const uint4* rec;
    const void* inv_k;   // entry-order words per kind (InvBits: 16-bit, or 32-bit for long rows)
    const void* inv_q;
    const uint2* hot;   // per chunk: {count, 0}, then {head position, size} in position order (NULL: none)
    float* a;
    float* qk;
    int C, W, R, first_partial, valid_last, hot_cap;
    int gb;             // hot groups per batch (x and y tables in LDS); 0: hot groups off
};

// Threads per pair block: 512, or 1024 where the LDS allows one block per compute unit anyway.
constexpr float kLog2E = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr size_t kPairStaticLds = 256;   // room left for the kernel's static LDS (scan partials)
constexpr int kWalkBatch = 8;

// Hot groups per batch at most.
constexpr int kPairBatchGroups = 32;
// A hot group whose L range (base 2) exceeds this is walked: the factors 2^(+-range/2) stay finite.
constexpr float kDenseRange = 200.0f;
constexpr uint32_t kHotWide = 0x80000000u;   // in a hot-list size word: the group is walked

// The triangle in LDS: row i holds cells 0..i padded to a multiple of 4 floats, so that every row
// starts 16-byte aligned (4-cell reads of the write-out); rows 4a .. 4a+3 take 4(a+1) floats each.
__host__ __device__ constexpr int tri_row(int i) { return 4 * ((i >> 2) + 1) * (2 * (i >> 2) + (i & 3)); }

// LDS of the pair kernel: the triangle, the hot list (+ batch bounds), the reference c of every
// hot group, per batch group its first batch position and its 4-token block masks (x, y), then
// the x and y tables (gb groups of Cp = C rounded up to 4 floats each).
struct PairLds {
    size_t tri, hot, gbase, gref, bmask, xt, yt, total;
};
__host__ __device__ inline PairLds pair_lds_layout(int C, int hot_cap, int gb) {
    auto up = [](size_t b) { return (b + 15) / 16 * 16; };
    const size_t cp = static_cast<size_t>((C + 3) & ~3);
    PairLds l;
    l.tri = 0;
    l.hot = up(static_cast<size_t>(tri_row(C)) * sizeof(float));
    l.gref = l.hot + up(static_cast<size_t>(hot_cap) * 2 * sizeof(uint32_t) + 16);   // + batch bounds
    l.gbase = l.gref + up(static_cast<size_t>(hot_cap) * sizeof(float));
    l.bmask = l.gbase + up(static_cast<size_t>(kPairBatchGroups + 1) * sizeof(uint32_t));
    l.xt = l.bmask + static_cast<size_t>(kPairBatchGroups) * 4 * sizeof(uint32_t);
    l.yt = l.xt + static_cast<size_t>(gb) * cp * sizeof(float);
    l.total = l.yt + static_cast<size_t>(gb) * cp * sizeof(float);
    return l;
}

template <int kPairThreads, typename InvT>
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
    const PairLds lay = pair_lds_layout(C, a.hot_cap, a.gb);
    const int cp = (C + 3) & ~3;
    float* tri = reinterpret_cast<float*>(smem + lay.tri);
    uint2* hl = reinterpret_cast<uint2*>(smem + lay.hot);               // hot list of the chunk
    int* bounds = reinterpret_cast<int*>(smem + lay.hot) + 2 * a.hot_cap;   // batch end, positions, any wide
    uint32_t* ubase = reinterpret_cast<uint32_t*>(smem + lay.gbase);    // batch-local first position
    float* gref = reinterpret_cast<float*>(smem + lay.gref);            // reference c per hot group
    uint32_t* bmask = reinterpret_cast<uint32_t*>(smem + lay.bmask);    // per group: x blocks (2 words), y blocks (2)
    float* xt = reinterpret_cast<float*>(smem + lay.xt);
    float* yt = reinterpret_cast<float*>(smem + lay.yt);
    // The walkers' first 32 entry-order words (16-bit words, rows of a multiple of 8 lanes): loaded
    // before anything else, so that the walks find them in registers.
    const int pre_lanes = q ? R : W;
    const bool pre = sizeof(InvT) == 2 && pre_lanes % 8 == 0 && static_cast<int>(threadIdx.x) < tv;
    uint4 ivp[4] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u),
                    make_uint4(0u, 0u, 0u, 0u)};
    if (pre) {
        const uint4* src = reinterpret_cast<const uint4*>(static_cast<const InvT*>(q ? a.inv_q : a.inv_k) +
                                                          (static_cast<int64_t>(c) * C + threadIdx.x) * pre_lanes);
#pragma unroll
        for (int v = 0; v < 4; ++v) ivp[v] = v * 8 < pre_lanes ? src[v] : make_uint4(0u, 0u, 0u, 0u);
    }
    const int tri_size = tri_row(C);
    for (int e = threadIdx.x; e < tri_size / 4; e += kPairThreads) reinterpret_cast<float4*>(tri)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t crow = static_cast<int64_t>(c) * n;
    const uint4* rec = a.rec + crow;
    const uint32_t row_q = q ? kIsQ : 0u;

    // ---- Hot groups, in batches of at most gb groups.
    const int nh = a.hot != nullptr ? static_cast<int>(a.hot[static_cast<int64_t>(c) * (a.hot_cap + 1)].x) : 0;
    // L of a record in base 2 as a compensated pair: hi = s log2(e), lo = the product's rounding
    // error plus c log2(e). Sums and differences of such pairs keep the exponent accurate.
    auto l2pair = [](const uint4& r, float& hi, float& lo) {
        const float ls = __uint_as_float(r.y), lc = __uint_as_float(r.z);
        hi = ls * kLog2E;
        lo = fmaf(ls, kLog2E, -hi) + lc * kLog2E;
    };
    if (threadIdx.x == 0) bounds[2] = 0;   // any group walked instead
    __syncthreads();
    if (nh > 0) {   // the hot list, each group's reference c (its L range's midpoint) and range check
        const uint2* hsrc = a.hot + static_cast<int64_t>(c) * (a.hot_cap + 1) + 1;
        for (int g = threadIdx.x; g < nh; g += kPairThreads) {
            uint2 h = hsrc[g];
            float h0, l0, h1, l1;
            l2pair(rec[h.x], h0, l0);
            l2pair(rec[h.x + h.y - 1u], h1, l1);
            gref[g] = 0.5f * (h0 + h1);
            if (fabsf(h0 - h1) > kDenseRange) {
                h.y |= kHotWide;
                bounds[2] = 1;
            }
            hl[g] = h;
        }
    }
    __syncthreads();
    // 2^(hi + lo - c) to about two ulps: hi - c is split exactly (TwoSum) into its rounded value d,
    // whose power of two the hardware takes, and an error that joins lo in a first-order factor
    // (|err + lo| is below an ulp of hi).
    auto pow2 = [](float hi, float lo, float cg) {
        const float d = hi - cg;
        const float bb = d - hi;
        const float err = (hi - (d - bb)) + (-cg - bb);
        return __builtin_amdgcn_exp2f(d) * fmaf(err + lo, kLn2, 1.0f);
    };
    for (int g0 = 0; g0 < nh;) {
        if (threadIdx.x == 0) {   // the batch: groups g0 .. g1-1
            const int g1 = min(nh, g0 + a.gb);
            uint32_t pos = 0;
            for (int g = g0; g < g1; ++g) {
                ubase[g - g0] = pos;
                pos += hl[g].y & ~kHotWide;
            }
            ubase[g1 - g0] = pos;
            bounds[0] = g1;
            bounds[1] = static_cast<int>(pos);
        }
        if (threadIdx.x < kPairBatchGroups) {
#pragma unroll
            for (int w = 0; w < 4; ++w) bmask[threadIdx.x * 4 + w] = 0u;
        }
        for (int e = threadIdx.x; e < a.gb * cp; e += kPairThreads) {
            xt[e] = 0.0f;
            yt[e] = 0.0f;
        }
        __syncthreads();
        const int g1 = bounds[0];
        const int np = bounds[1];
        const int ng = g1 - g0;
        // Thread x takes the batch positions [u0, u1) (group by group) and writes the x (y) entry of
        // every row (K) run that starts there: the run's value sum times 2^(L - c) (2^(c - L)).
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
            cu.gend = cu.ghead + static_cast<int>(hl[g0 + gg].y & ~kHotWide);
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
        {
            Cursor cu = cursor_at(g);
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
                    const bool cont = !fst[b] && (prev & kTag) == (r[b].x & kTag);
                    prev = r[b].x;
                    if (cont || (hl[g0 + grp[b]].y & kHotWide)) continue;
                    const bool is_k = !(r[b].x & kIsQ), is_row = (r[b].x & kIsQ) == row_q;
                    const uint32_t tok = (r[b].x >> kTokShift) & 0xFFu;
                    float hi, lo;
                    l2pair(r[b], hi, lo);
                    const float cg = gref[g0 + grp[b]];
                    uint32_t* bm = bmask + grp[b] * 4;
                    if (is_row) {
                        xt[grp[b] * cp + tok] = suf[b] * pow2(hi, lo, cg);
                        atomicOr(bm + (tok >> 7), 1u << ((tok >> 2) & 31u));
                    }
                    if (is_k) {
                        yt[grp[b] * cp + tok] = suf[b] * pow2(-hi, -lo, -cg);
                        atomicOr(bm + 2 + (tok >> 7), 1u << ((tok >> 2) & 31u));
                    }
                }
            }
        }
        __syncthreads();
        // Each thread owns 4 x 4 blocks (bi >= bj) of the triangle and adds sum_g x_g y_g^T into them,
        // skipping groups with no row run in the block's rows or no K run in its columns.
        {
            const int nbr = (C + 3) >> 2;
            const int nblk = nbr * (nbr + 1) / 2;
            for (int blk = threadIdx.x; blk < nblk; blk += kPairThreads) {
                int bi = static_cast<int>((sqrtf(8.0f * static_cast<float>(blk) + 1.0f) - 1.0f) * 0.5f);
                while (bi * (bi + 1) / 2 > blk) --bi;
                while ((bi + 1) * (bi + 2) / 2 <= blk) ++bi;
                const int bj = blk - bi * (bi + 1) / 2;
                float acc[4][4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0f;
                }
                bool any = false;
                for (int gg = 0; gg < ng; ++gg) {
                    const uint32_t* bm = bmask + gg * 4;
                    if (!((bm[bi >> 5] >> (bi & 31)) & 1u) || !((bm[2 + (bj >> 5)] >> (bj & 31)) & 1u)) continue;
                    any = true;
                    const float4 x4 = *reinterpret_cast<const float4*>(xt + gg * cp + 4 * bi);
                    const float4 y4 = *reinterpret_cast<const float4*>(yt + gg * cp + 4 * bj);
                    const float xs[4] = {x4.x, x4.y, x4.z, x4.w}, ys[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(xs[u], ys[v], acc[u][v]);
                    }
                }
                if (!any) continue;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int ii = 4 * bi + u;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int jj = 4 * bj + v;
                        if (ii < C && (q ? jj <= ii : jj < ii)) {
                            float* cell = tri + tri_row(ii) + jj;
                            *cell = *cell + acc[u][v];
                        }
                    }
                }
            }
        }
        __syncthreads();   // the tables are rebuilt for the next batch
        g0 = g1;
    }
    const bool any_wide = bounds[2] != 0;   // (set before the last barrier)

    // ---- Other groups: thread i walks its flagged runs back to the group head. The entry words of
    // 32 lanes are loaded together; walks go two at a time, each with the record window around its
    // start (one record after, the own record, four before) loaded in one go, which covers a small
    // group; longer groups read eight more records at a time.
    const int i = threadIdx.x;
    if (i < tv) {
        float* row = tri + tri_row(i);
        const int lanes = q ? R : W;
        const InvT* iv = static_cast<const InvT*>(q ? a.inv_q : a.inv_k) + (static_cast<int64_t>(c) * C + i) * lanes;
        // Token i's entries of this kind: (Q flag, token) bits of the payload.
        const uint32_t own_tag = (q ? kIsQ : 0u) | (static_cast<uint32_t>(i) << kTokShift);
        const uint32_t tag_mask = kIsQ | (0xFFu << kTokShift);
        // The sorted position of the walk starting at lane ln, or -1 for a hot group's run whose
        // group was summed densely.
        auto walk_start = [&](int ln) {
            const uint32_t word = iv[ln];
            // A walk start has an earlier entry in its group, so 1 <= rho (the clamp only guards).
            const int rho = min(static_cast<int>(word & InvBits<InvT>::kPos), n - 1);
            if (word & InvBits<InvT>::kHot) {   // walked only if its group was too wide for the dense pass
                int lo_g = 0, hi_g = nh - 1;   // the last hot group with head <= rho
                while (lo_g < hi_g) {
                    const int mid = (lo_g + hi_g + 1) >> 1;
                    if (static_cast<int>(hl[mid].x) <= rho) lo_g = mid; else hi_g = mid - 1;
                }
                if (!(hl[lo_g].y & kHotWide)) return -1;
            }
            return rho;
        };
        // The record window of a walk: positions rho + 1, rho, rho - 1, ..., rho - kBack.
        constexpr int kBack = 4, kWin = kBack + 2;
        auto load_window = [&](int rho, uint4 (&rb)[kWin]) {
            const int r = max(rho, 0);
#pragma unroll
            for (int k = 0; k < kWin; ++k) rb[k] = rec[min(max(r + 1 - k, 0), n - 1)];
        };
        auto walk = [&](int rho, const uint4 (&rb)[kWin]) {
            const uint4 own = rb[1];
            // Sum the run's values (the run goes on past rho only for repeated lanes of the token).
            float wi = __uint_as_float(own.w);
            if (rho + 1 < n && !(rb[0].x & kHead) && (rb[0].x & tag_mask) == own_tag) {
                wi = wi + __uint_as_float(rb[0].w);
                for (int p = rho + 2; p < n; ++p) {
                    const uint4 nx = rec[p];
                    if ((nx.x & kHead) || (nx.x & tag_mask) != own_tag) break;
                    wi = wi + __uint_as_float(nx.w);
                }
            }
            const float se = __uint_as_float(own.y), ce = __uint_as_float(own.z);
            // Walk back to the head; the K runs of earlier tokens are summed, then one term each.
            int cur_j = -1;
            float kj = 0.0f, sj = 0.0f, cj = 0.0f;
            bool done = false;
            auto visit = [&](const uint4& r) {
                const uint32_t px = r.x;
                if (!(px & (kIsQ | kInvalid))) {
                    const int jt = static_cast<int>((px >> kTokShift) & 0xFFu);
                    if (jt != cur_j) {
                        if (cur_j >= 0 && (q || cur_j != i)) {
                            row[cur_j] = row[cur_j] + (wi * kj) * expf((se - sj) + (ce - cj));
                        }
                        cur_j = jt;
                        kj = 0.0f;
                        sj = __uint_as_float(r.y);
                        cj = __uint_as_float(r.z);
                    }
                    kj = kj + __uint_as_float(r.w);
                }
                done = (px & kHead) != 0;
            };
#pragma unroll
            for (int k = 2; k < kWin; ++k) {
                if (done) break;
                visit(rb[k]);
            }
            for (int top = rho - 1 - kBack; !done; top -= kWalkBatch) {
                uint4 rc[kWalkBatch];
#pragma unroll
                for (int k = 0; k < kWalkBatch; ++k) rc[k] = rec[max(top - k, 0)];
#pragma unroll
                for (int k = 0; k < kWalkBatch; ++k) {
                    if (done) break;
                    visit(rc[k]);
                }
            }
            if (cur_j >= 0 && (q || cur_j != i)) row[cur_j] = row[cur_j] + (wi * kj) * expf((se - sj) + (ce - cj));
        };
        for (int lb = 0; lb < lanes; lb += 32) {
          uint32_t flags = 0;
          const uint32_t walk_bits = any_wide ? (InvBits<InvT>::kWalk | InvBits<InvT>::kHot) : InvBits<InvT>::kWalk;
          if (pre && lb == 0) {   // (the preloaded words: lanes 0..31, zeros past the row)
#pragma unroll
              for (int u = 0; u < 32; ++u) {
                  const uint4 v4 = ivp[u / 8];
                  const uint32_t w2 = (u % 8) < 2 ? v4.x : (u % 8) < 4 ? v4.y : (u % 8) < 6 ? v4.z : v4.w;
                  const uint32_t word = (u % 2) ? (w2 >> 16) : (w2 & 0xFFFFu);
                  flags |= (u < lanes && (word & walk_bits)) ? (1u << u) : 0u;
              }
          } else {   // (all 32 words loaded before any is tested, so that they are in flight together)
              uint32_t wd[32];
#pragma unroll
              for (int u = 0; u < 32; ++u) wd[u] = iv[min(lb + u, lanes - 1)];
#pragma unroll
              for (int u = 0; u < 32; ++u) flags |= (lb + u < lanes && (wd[u] & walk_bits)) ? (1u << u) : 0u;
          }
          // Walks three at a time: their record windows in flight before any is walked (the terms
          // still reach the row in lane order).
          for (; flags != 0u;) {
            int rh[3];
#pragma unroll
            for (int q3 = 0; q3 < 3; ++q3) {
                const int ln = flags != 0u ? lb + __builtin_ctz(flags) : -1;
                if (flags != 0u) flags &= flags - 1u;
                rh[q3] = ln >= 0 ? walk_start(ln) : -1;
            }
            uint4 w1[kWin], w2[kWin], w3[kWin];
            load_window(rh[0], w1);
            load_window(rh[1], w2);
            load_window(rh[2], w3);
            if (rh[0] >= 0) walk(rh[0], w1);
            if (rh[1] >= 0) walk(rh[1], w2);
            if (rh[2] >= 0) walk(rh[2], w3);
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
            // Cells past the triangle read as zeros: the row padding is never written, and A's
            // diagonal cell is never written either.
            f32x4 v4 = f32x4{0.f, 0.f, 0.f, 0.f};
            if (j0 <= ii) v4 = *reinterpret_cast<const f32x4*>(tri + tri_row(ii) + j0);
            // Non-temporal: the matrices stream past the caches (nothing in the step reads them back).
            __builtin_nontemporal_store(v4, reinterpret_cast<f32x4*>(out + ob) + e);
        }
    } else {
        for (int e = threadIdx.x; e < C * C; e += kPairThreads) {
            const int ii = e / C;
            const int jj = e - ii * C;
            out[ob + e] = (q ? jj <= ii : jj < ii) ? tri[tri_row(ii) + jj] : 0.0f;
        }
    }
}

// Host-side plan of one Phase-1 launch: sort items per thread, digit width, output sweeps.
struct MainPlan {
    int ipt;
    int digit_bits;
    int stage_bytes;
    int resident, vals_off, hist_off, rec_off;
    size_t lds_bytes;
    Sweeps sweeps;
};

constexpr int kLdsTotal = 160 * 1024;
constexpr int kStaticReserve = 1024;   // static LDS of the kernel (scan totals, tile counts)

// LDS bytes of the records of one sweep (arrays padded to 4 entries): K 12 B, Q 8 B per entry.
int sweep_bytes(const sdm_p1_shape* s, uint32_t kinds, int tokens) {
    const int nk = (kinds & kSweepK) ? (tokens * s->W + 3) & ~3 : 0;
    const int nq = (kinds & kSweepQ) ? (tokens * s->R + 3) & ~3 : 0;
    return nk * 12 + nq * 8;
}

// LDS bytes of the per-wave digit counts: kNW rows of 2^d counts, each padded by one word.
int hist_bytes(int d) { return kNW * ((1 << d) + 1) * 4; }

MainPlan plan_main(const sdm_p1_shape* s, bool with_pairs_ws) {
    MainPlan m;
    const int n = s->C * (s->W + s->R);
    m.ipt = n <= kNT ? 1 : n <= 2 * kNT ? 2 : n <= 4 * kNT ? 4 : n <= 8 * kNT ? 8 : 16;
    const int np = kNT * m.ipt;
    // Sorted row, gates and (with pair sums) the chunk's hot-group list.
    const int fixed = np * 2 + 256 * static_cast<int>(sizeof(float)) +
                      (with_pairs_ws ? s->C * s->W / kHotMin * static_cast<int>(sizeof(uint2)) : 0);
    const int total = s->lds_budget > 0 ? min(kLdsTotal, s->lds_budget) : kLdsTotal;   // (a test budget)
    const int cap_max = (total - kStaticReserve - fixed) / 16 * 16;
    // Widest digit (<= 10 bits) whose per-wave counts fit beside the keys (and, in the resident
    // layout, beside the keys and the staged values, with the records fitting there too).
    const int vals_bytes = (((s->C * s->W + 3) & ~3) + ((s->C * s->R + 3) & ~3)) * 4;
    m.resident = 0;
    int d = 10;
    if (m.ipt <= 8) {
        while (d > 4 && np * 4 + vals_bytes + hist_bytes(d) > cap_max) --d;
        m.resident = np * 4 + vals_bytes + max(hist_bytes(d), sweep_bytes(s, kSweepK | kSweepQ, s->C)) <= cap_max;
    }
    if (!m.resident) {
        d = 10;
        while (d > 4 && np * 4 + hist_bytes(d) > cap_max) --d;
    }
    m.digit_bits = d;
    m.vals_off = np * 4;
    m.hist_off = np * 4 + (m.resident ? vals_bytes : 0);
    m.rec_off = m.resident ? m.hist_off : 0;
    int cap = m.hist_off + hist_bytes(d);
    // Sweeps: every record at once up to 8 items per thread, else each kind in token ranges
    // (multiples of 4 tokens, so every range starts 16-byte aligned in the entry-order rows).
    Sweeps& sw = m.sweeps;
    sw.count = 0;
    auto add = [&](uint32_t kinds, int t0, int t1) {
        if (sw.count < kMaxSweeps) {
            sw.kinds[sw.count] = kinds;
            sw.t0[sw.count] = t0;
            sw.t1[sw.count] = t1;
            cap = max(cap, m.rec_off + sweep_bytes(s, kinds, t1 - t0));
        }
        ++sw.count;
    };
    if (m.ipt <= 8) {   // fits: n <= 8192 entries of at most 12 B beside at most 21 KB of the rest
        add(kSweepK | kSweepQ, 0, s->C);
        if (m.rec_off + sweep_bytes(s, kSweepK | kSweepQ, s->C) > cap_max) sw.count = kMaxSweeps + 1;   // refused
    } else {   // the kernel sweeps one kind at a time here
        for (uint32_t kind : {kSweepK, kSweepQ}) {
            int step = 4;
            while (step + 4 <= s->C && sweep_bytes(s, kind, step + 4) <= cap_max) step += 4;
            for (int t0 = 0; t0 < s->C; t0 += step) add(kind, t0, min(s->C, t0 + step));
        }
    }
    m.stage_bytes = (cap + 15) / 16 * 16;
    m.lds_bytes = static_cast<size_t>(m.stage_bytes) + static_cast<size_t>(fixed);
    return m;
}

template <int IPT, bool VBF>
const void* main_fn(bool lane_gates, bool id64) {
    return lane_gates ? (id64 ? reinterpret_cast<const void*>(&p1_main_kernel<IPT, true, true, VBF>)
                              : reinterpret_cast<const void*>(&p1_main_kernel<IPT, true, false, VBF>))
                      : (id64 ? reinterpret_cast<const void*>(&p1_main_kernel<IPT, false, true, VBF>)
                              : reinterpret_cast<const void*>(&p1_main_kernel<IPT, false, false, VBF>));
}

template <int IPT>
hipError_t launch_main(P1Args args, bool lane_gates, bool id64, bool vbf, size_t lds, int N, hipStream_t st,
                       hipEvent_t start, hipEvent_t stop) {
    // (The value type is a template parameter: a run-time switch in the staging loads costs the
    // float32 path about a sixth of its time.)
    const void* fn = vbf ? main_fn<IPT, true>(lane_gates, id64) : main_fn<IPT, false>(lane_gates, id64);
    void* kargs[] = {&args};
    return hipExtLaunchKernel(fn, dim3(N), dim3(kNT), kargs, lds, st, start, stop, 0);
}

// Dense group ordinals of one chunk's K-only row (gord_k): a valid position gets the number of
// valid FIRSTs at or before it, minus one (the ordinal of its group among the chunk's groups with a
// valid write, in slot order); padding gets -1. One block per chunk walks the row 256 positions at
// a time (coalesced): a block-wide inclusive scan of the FIRST flags plus the running count.
constexpr int kOrdThreads = 256;

__global__ void __launch_bounds__(kOrdThreads) p1_ordinal_kernel(const uint32_t* spay_k, int32_t* gord, int CW) {
    __shared__ int wsum[kOrdThreads / kWave];
    const int64_t base = static_cast<int64_t>(blockIdx.x) * CW;
    const int lane = static_cast<int>(lane_id());
    const int w = static_cast<int>(threadIdx.x) / kWave;
    int carry = 0;
    for (int j0 = 0; j0 < CW; j0 += kOrdThreads) {
        const int j = j0 + static_cast<int>(threadIdx.x);
        const uint32_t x = j < CW ? spay_k[base + j] : kInvalid;
        const bool valid = (x & kInvalid) == 0u;
        int v = (valid && (x & kFirst)) ? 1 : 0;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(v, d, kWave);
            if (lane >= d) v += o;
        }
        if (lane == kWave - 1) wsum[w] = v;
        __syncthreads();
        int before = carry, total = 0;
#pragma unroll
        for (int k = 0; k < kOrdThreads / kWave; ++k) {
            before += k < w ? wsum[k] : 0;
            total += wsum[k];
        }
        if (j < CW) gord[base + j] = valid ? before + v - 1 : -1;
        carry += total;
        __syncthreads();   // wsum is rewritten by the next round
    }
}

}  // namespace

thread_local const char* g_p1_stage = "";

bool p1_tiled(const sdm_p1_shape* s) {
    return s->tiled != 0 || static_cast<int64_t>(s->C) * (s->W + s->R) > kP1MaxRow;
}

P1Workspace p1_workspace_layout(const sdm_p1_shape* s) {
    const size_t n = static_cast<size_t>(s->C) * static_cast<size_t>(s->W + s->R);
    const size_t N = static_cast<size_t>(s->N);
    const size_t nk = N * static_cast<size_t>(s->C) * static_cast<size_t>(s->W);
    const size_t nq = N * static_cast<size_t>(s->C) * static_cast<size_t>(s->R);
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    P1Workspace w;
    w.tiled = p1_tiled(s);
    const size_t ib = w.tiled ? sizeof(uint32_t) : sizeof(uint16_t);   // entry-order pair words
    w.rec_off = 0;
    w.inv_k_off = up(N * n * sizeof(uint4));
    w.inv_q_off = w.inv_k_off + up(nk * ib);
    w.hot_cap = s->C * s->W / kHotMin;
    w.hot_off = w.inv_q_off + up(nq * ib);
    w.total = w.hot_off + up(N * static_cast<size_t>(w.hot_cap + 1) * sizeof(uint2));
    w.sort_off = w.rev_off = 0;
    if (w.tiled) {   // the tiled path's sort buffers (keys and entry indices, two of each) and reverse-scan results
        w.sort_off = w.total;
        w.rev_off = w.sort_off + up(N * n * 4 * sizeof(uint32_t));
        w.total = w.rev_off + up(N * n * 3 * sizeof(uint32_t));
    }
    return w;
}

// (Without hot groups the pair kernel keeps only its triangle and a few words in LDS.)
size_t p1_pair_lds_min(const sdm_p1_shape* s) { return pair_lds_layout(s->C, 0, 0).total + kPairStaticLds; }

size_t p1_lds_bytes(const sdm_p1_shape* s, const sdm_p1_io* io) {
    if (p1_tiled(s)) return p1_tiled_lds_bytes(s);
    const MainPlan m = plan_main(s, io->a != nullptr || io->qk != nullptr);
    const size_t budget = s->lds_budget > 0 ? static_cast<size_t>(min(kLdsTotal, s->lds_budget)) : static_cast<size_t>(kLdsTotal);
    // (a plan over the budget, or with more sweeps than the kernel takes, is refused)
    if (m.sweeps.count > kMaxSweeps || m.lds_bytes + kStaticReserve > budget) return SIZE_MAX;
    return m.lds_bytes;
}

PairPlan pair_plan(const sdm_p1_shape* s, bool pairs, int lds_max) {
    // Hot groups only when the pair kernel's x and y tables hold at least 4 groups beside the rest.
    // Groups per batch: as many as the blocks per compute unit that 4 groups allow still fit.
    PairPlan pp;
    pp.hot_cap = s->C * s->W / kHotMin;
    const size_t pair_fixed = pair_lds_layout(s->C, pp.hot_cap, 0).total + kPairStaticLds;
    const size_t per_group = 2 * static_cast<size_t>((s->C + 3) & ~3) * sizeof(float);
    const size_t pair_min = pair_fixed + 4 * per_group;
    pp.blocks_cu = pair_min <= static_cast<size_t>(lds_max) ? static_cast<int>(lds_max / pair_min) : 0;
    pp.gb = pp.blocks_cu > 0 ? min(kPairBatchGroups,
                                   static_cast<int>((static_cast<size_t>(lds_max) / pp.blocks_cu - pair_fixed) / per_group))
                             : 0;
    // (A hot list too long for LDS beside the triangle, as with C = 256, W = 256: every group walked.)
    pp.hot_on = pairs && pp.hot_cap > 0 && pp.gb >= 4 && s->pair_walk == 0;   // (pair_walk: every group walked)
    if (!pp.hot_on) {   // the triangle alone per block
        pp.gb = 0;
        pp.blocks_cu = max(1, static_cast<int>(static_cast<size_t>(lds_max) / (pair_lds_layout(s->C, 0, 0).total + kPairStaticLds)));
    }
    return pp;
}

hipError_t p1_ordinal_launch(const sdm_p1_shape* s, const sdm_p1_io* io, hipStream_t st) {
    if (io->gord_k == nullptr) return hipSuccess;   // (on st, after the kernel that writes spay_k)
    g_p1_stage = "group ordinal kernel";
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(io->spay_k);
    int32_t* gord = io->gord_k;
    int cw = s->C * s->W;
    void* kargs[] = {&sp, &gord, &cw};
    // (the launch's own status: a pending error of an earlier call is not this launch's)
    return hipLaunchKernel(reinterpret_cast<const void*>(&p1_ordinal_kernel), dim3(s->N), dim3(kOrdThreads), kargs, 0, st);
}

hipError_t pair_launch(const P1Launch& Lc, const PairPlan& pp, bool inv32, hipStream_t st) {
    const sdm_p1_shape* s = Lc.s;
    const sdm_p1_io* io = Lc.io;
    PairArgs pa;
    pa.rec = static_cast<const uint4*>(Lc.rec);
    pa.inv_k = Lc.inv_k;
    pa.inv_q = Lc.inv_q;
    // Hot groups off: no list (the Phase-1 kernels flag no entry as hot), and no LDS for one.
    pa.hot = pp.hot_on ? static_cast<const uint2*>(Lc.hot) : nullptr;
    pa.hot_cap = pp.hot_on ? pp.hot_cap : 0;
    pa.gb = pp.hot_on ? pp.gb : 0;
    pa.a = io->a;
    pa.qk = io->qk;
    pa.C = s->C;
    pa.W = s->W;
    pa.R = s->R;
    pa.first_partial = s->first_partial;
    pa.valid_last = s->valid_last;
    const size_t lds = pair_lds_layout(s->C, pa.hot_cap, pa.gb).total;
    const int threads = pp.blocks_cu == 1 ? 1024 : 512;
    const void* fn = inv32 ? (threads == 1024 ? reinterpret_cast<const void*>(&p1_pairs_kernel<1024, uint32_t>)
                                              : reinterpret_cast<const void*>(&p1_pairs_kernel<512, uint32_t>))
                           : (threads == 1024 ? reinterpret_cast<const void*>(&p1_pairs_kernel<1024, uint16_t>)
                                              : reinterpret_cast<const void*>(&p1_pairs_kernel<512, uint16_t>));
    void* kargs[] = {&pa};
    g_p1_stage = "pair kernel";
    hipEvent_t e0 = io->events != nullptr ? io->events[2] : nullptr, e1 = io->events != nullptr ? io->events[3] : nullptr;
    return hipExtLaunchKernel(fn, dim3(s->N, 2), dim3(threads), kargs, lds, st, e0, e1, 0);
}

hipError_t p1_launch(const P1Launch& Lc, hipStream_t st) {
    const sdm_p1_shape* s = Lc.s;
    const sdm_p1_io* io = Lc.io;
    if (s->N == 0) return hipSuccess;
    if (p1_tiled(s)) return p1_tiled_launch(Lc, st);
    g_p1_stage = "sort/scan kernel";
    const bool pairs = io->a != nullptr || io->qk != nullptr;
    P1Args a;
    a.k_idx = io->k_idx;
    a.q_idx = io->q_idx;
    a.k_val = io->k_val;
    a.q_val = io->q_val;
    a.g = io->g;
    a.log_k = io->log_k;
    a.rex = io->rex;
    a.cpe = io->cpe;
    a.k_eff = io->k_eff;
    a.is_last = io->is_last;
    a.is_only = io->is_only;
    a.pos_k = io->pos_k;
    a.log_q = io->log_q;
    a.q_w = io->q_w;
    a.pos_q = io->pos_q;
    a.q_last = io->q_last;
    a.q_only = io->q_only;
    a.inv_k = pairs ? static_cast<uint16_t*>(Lc.inv_k) : nullptr;
    a.inv_q = pairs ? static_cast<uint16_t*>(Lc.inv_q) : nullptr;
    // Four-entry vector stores where every row of the kind's fields is 16-byte aligned (4-byte for
    // the flag bytes; the workspace rows follow from C * W or C * R being a multiple of 4).
    auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
    // (Value-typed fields, bfloat16 values: four entries are 8 bytes.)
    const bool vbf = s->val_bytes == 2;
    const uintptr_t va = vbf ? 8 : 16;
    const bool vk = (s->C * s->W) % 4 == 0 && al(io->k_val, va) && al(io->log_k, 16) && al(io->rex, 16) &&
                    al(io->cpe, va) && al(io->k_eff, va) && al(io->pos_k, 16) && al(io->is_last, 4) &&
                    al(io->is_only, 4);
    const bool vq = (s->C * s->R) % 4 == 0 && al(io->q_val, va) && al(io->log_q, 16) && al(io->q_w, va) &&
                    al(io->pos_q, 16) && al(io->q_last, 4) && al(io->q_only, 4);
    a.vec = (vk ? 1u : 0u) | (vq ? 2u : 0u);
    a.spay_k = io->spay_k;
    a.spay_q = io->spay_q;
    a.krec = reinterpret_cast<int4*>(io->krec);
    a.tiles_k = io->tiles_k;
    a.repeats = io->repeats;
    a.perm = io->perm;
    a.status = io->status;
    a.rec = pairs ? static_cast<uint4*>(Lc.rec) : nullptr;
    const PairPlan pp = pair_plan(s, pairs, Lc.lds_max);
    a.hot = pairs ? static_cast<uint2*>(Lc.hot) : nullptr;
    a.hot_min = pp.hot_on ? kHotMin : 0x7FFFFFFF;
    a.hot_cap = pp.hot_cap;
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
    const MainPlan m = plan_main(s, pairs);
    if (m.sweeps.count > kMaxSweeps) return hipErrorInvalidValue;
    a.digit_bits = m.digit_bits;
    a.stage_bytes = m.stage_bytes;
    a.resident = m.resident;
    a.vals_off = m.vals_off;
    a.hist_off = m.hist_off;
    a.rec_off = m.rec_off;
    a.sweeps = m.sweeps;
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if (io->events != nullptr) {
        for (int k = 0; k < 4; ++k) ev[k] = io->events[k];
    }
    hipError_t e;
    switch (m.ipt) {
        case 1: e = launch_main<1>(a, s->g_lane_stride != 0, s->idx_bytes == 8, vbf, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
        case 2: e = launch_main<2>(a, s->g_lane_stride != 0, s->idx_bytes == 8, vbf, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
        case 4: e = launch_main<4>(a, s->g_lane_stride != 0, s->idx_bytes == 8, vbf, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
        case 8: e = launch_main<8>(a, s->g_lane_stride != 0, s->idx_bytes == 8, vbf, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
        default: e = launch_main<16>(a, s->g_lane_stride != 0, s->idx_bytes == 8, vbf, m.lds_bytes, s->N, st, ev[0], ev[1]); break;
    }
    if (e == hipSuccess) e = p1_ordinal_launch(s, io, st);
    if (e != hipSuccess || !pairs || io->defer_pairs) return e;
    return pair_launch(Lc, pp, false, st);
}

hipError_t p1_pairs_launch(const P1Launch& Lc, hipStream_t st) {
    // The plan the sort/scan (or tiled) kernel of the same shape followed (it is a function of the
    // shape and the device alone), so the hot-group lists it left are read as it wrote them.
    const PairPlan pp = pair_plan(Lc.s, true, Lc.lds_max);
    return pair_launch(Lc, pp, p1_tiled(Lc.s), st);
}

int p1_lds_kernels(const void** fns, int cap) {
    int n = 0;
    auto add = [&](const void* f) {
        if (n < cap) fns[n++] = f;
    };
    for (int lg = 0; lg < 2; ++lg) {
        for (int id64 = 0; id64 < 2; ++id64) {
            add(main_fn<1, false>(lg, id64));
            add(main_fn<2, false>(lg, id64));
            add(main_fn<4, false>(lg, id64));
            add(main_fn<8, false>(lg, id64));
            add(main_fn<16, false>(lg, id64));
            add(main_fn<1, true>(lg, id64));
            add(main_fn<2, true>(lg, id64));
            add(main_fn<4, true>(lg, id64));
            add(main_fn<8, true>(lg, id64));
            add(main_fn<16, true>(lg, id64));
        }
    }
    add(reinterpret_cast<const void*>(&p1_pairs_kernel<1024, uint16_t>));
    add(reinterpret_cast<const void*>(&p1_pairs_kernel<512, uint16_t>));
    add(reinterpret_cast<const void*>(&p1_pairs_kernel<1024, uint32_t>));
    add(reinterpret_cast<const void*>(&p1_pairs_kernel<512, uint32_t>));
    n += p1_tiled_lds_kernels(fns + n, cap - n);
    return n;
}

}  // namespace sdm
