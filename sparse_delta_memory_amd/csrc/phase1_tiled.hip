// Phase 1 of a chunk through the tiled path: rows longer than one workgroup sorts on chip (up to
// 2^17 entries), or any row when the shape asks for it (shape->tiled).
//
// One 1024-thread workgroup per chunk works from global memory (the workspace) in tiles of 8192
// entries, 8 per thread:
//   1. keys: every entry's key (its local slot, or the invalid key for a masked token) and its entry
//      index go to buffer 0;
//   2. a stable LSD radix sort between the two buffers, passes of at most 6 key bits. Per pass,
//      each wave ranks the items of each tile by ballot-built peer masks (stable, no atomics) and
//      counts its digits; one exclusive scan over (digit, wave of the row) gives every wave its
//      first position per digit; a second sweep recomputes the ranks and scatters. Rows this long
//      are sorted by merge rounds of on-chip sorts on the pages; here the whole row takes global
//      radix passes, which need no merge path and keep the order of equal keys by construction;
//   3. a reverse scan over the tiles, last first (a thread owns 16 consecutive sorted positions of
//      a tile): per position the gate sum after it in its group, its valid K and Q peers after it
//      and its valid peers of either kind after it, kept in the workspace;
//   4. a forward scan over the tiles in order: per position every output. Entry-order fields are
//      stored at the entry's index; the pair records and the (32-bit) entry-order words feed the
//      pair kernel as those of the on-chip kernel do.
// Definitions and readings are those of the on-chip kernel (page
// "sparse_delta_memory/cuda/phase1_cuda.py": keys and payloads of p1_keys_zw_kernel, the scan
// semantics of p1_scan_kernel, the records of its Outputs / Records comments). Scans combine
// compensated sums in a fixed tree and every output element has one writer: results are bitwise
// reproducible, and the integer outputs equal the on-chip kernel's bit for bit.
#include <hip/hip_ext.h>

#include <climits>

#include "p1_scan.hpp"
#include "sdm_device.hpp"
#include "sdm_launch.hpp"

namespace sdm {
namespace {

constexpr int kTI = 8;                                    // items per thread per tile
constexpr int kTT = kNT * kTI;                            // entries per tile
constexpr int kTDigit = 6;                                // key bits per radix pass
constexpr int kTUnits = (kP1MaxTiledRow / kTT) * kNW;     // (tile, wave) units of the longest row
constexpr uint32_t kTPad = 0xFFFFFFFFu;                   // key past the row: sorts last, never stored
constexpr uint32_t kTWalk = InvBits<uint32_t>::kWalk, kTHot = InvBits<uint32_t>::kHot;

struct TiledArgs {
    const void* k_idx;
    const void* q_idx;
    const void* k_val;
    const void* q_val;
    const float* g;
    float* log_k;
    float* rex;
    void* cpe;
    void* k_eff;
    int8_t* is_last;
    int8_t* is_only;
    int32_t* pos_k;
    float* log_q;
    void* q_w;
    int32_t* pos_q;
    int8_t* q_last;
    int8_t* q_only;
    uint32_t* spay_k;
    uint32_t* spay_q;
    uint4* krec;
    int32_t* tiles_k;
    int32_t* repeats;
    int32_t* perm;
    int32_t* status;
    uint4* rec;          // pair records (NULL: no pair sums)
    uint32_t* inv_k;     // 32-bit entry-order pair words (InvBits<uint32_t>)
    uint32_t* inv_q;
    uint2* hot;          // per chunk: {count, 0}, then {head position, size} of each hot group
    uint32_t* sort;      // [N, 4, n]: keys and entry indices, two buffers of each
    uint32_t* rev;       // [N, n, 3]: per sorted position the reverse-scan results
    int64_t stream_offset;
    int C, W, R, P, key_bits, first_partial, valid_last, tile_len, hot_min, hot_cap;
    uint32_t wr_magic;
    int lane_gates, id64, vbf;
};

// exp of the group total from the compensated log-cumsum (s, c) and the sum after (TwoSum).
__device__ __forceinline__ float tiled_group_exp(float s, float c, float rex) {
    const float gs = s + rex;
    const float gb = gs - s;
    const float ge = (s - (gs - gb)) + (rex - gb);
    return expf(gs + (c + ge));
}

__global__ void __launch_bounds__(kNT) p1_tiled_kernel(TiledArgs a) {
    __shared__ uint32_t hist[kTUnits << kTDigit];   // per (unit, digit): counts, then first positions
    __shared__ SegW wtot[2 * kNW];
    __shared__ uint32_t wsum[2 * kNW];
    __shared__ float gates[256];
    __shared__ uint32_t hot_n;
    extern __shared__ __align__(16) unsigned char tsmem[];
    uint2* hot_buf = reinterpret_cast<uint2*>(tsmem);   // hot_cap entries

    const int c = blockIdx.x;
    const int C = a.C, W = a.W, R = a.R;
    const int wr = W + R;
    const int n = C * wr;
    const int ntiles = (n + kTT - 1) / kTT;
    const int tv = c >= a.first_partial ? a.valid_last : C;
    const uint32_t key_lim = 1u << a.key_bits;
    const int64_t id_base = static_cast<int64_t>(c % a.P) * a.stream_offset;
    const int64_t cw = static_cast<int64_t>(c) * C * W;
    const int64_t cr = static_cast<int64_t>(c) * C * R;
    const int64_t crow = static_cast<int64_t>(c) * n;
    const int tid = static_cast<int>(threadIdx.x);
    const int lane = static_cast<int>(lane_id());
    const int w = tid / kWave;
    uint32_t* keys0 = a.sort + crow * 4;
    uint32_t* rr0 = keys0 + n;
    uint32_t* keys1 = rr0 + n;
    uint32_t* rr1 = keys1 + n;
    uint32_t* rev = a.rev + crow * 3;
    uint32_t seg_phase = 0, add_phase = 0;

    if (!a.lane_gates) {
        for (int t = tid; t < C; t += kNT) gates[t] = t < tv ? a.g[static_cast<int64_t>(c) * C + t] : 0.0f;
    }
    if (tid == 0) hot_n = 0u;
    auto gate = [&](int t, int j) -> float { return a.lane_gates ? a.g[cw + t * W + j] : gates[t]; };
    auto slot_id = [&](int t, int j) -> int64_t {
        const bool k = j < W;
        const int64_t i = k ? cw + t * W + j : cr + t * R + (j - W);
        const void* ids = k ? a.k_idx : a.q_idx;
        return a.id64 ? static_cast<const int64_t*>(ids)[i] : static_cast<int64_t>(static_cast<const int32_t*>(ids)[i]);
    };

    // ---- 1. keys, in entry order.
    bool bad = false;
    for (int i = tid; i < n; i += kNT) {
        const int t = token_of_entry(i, a.wr_magic);
        const int j = i - t * wr;
        uint32_t key = key_lim;
        if (t < tv) {
            const int64_t id = slot_id(t, j);
            const int64_t local = id - id_base;
            key = static_cast<uint32_t>(local) & (key_lim - 1u);
            bad = bad || id < 0 || local < 0 || local >= static_cast<int64_t>(key_lim);
        }
        keys0[i] = key;
        rr0[i] = static_cast<uint32_t>(i);
    }
    if (a.status != nullptr && __any(bad) && lane == 0) atomicOr(a.status, 1);
    __syncthreads();

    // ---- 2. stable LSD radix sort between the two buffers (invalid entries need one more key bit,
    // in a ragged chunk only).
    const int bits = tv < C ? a.key_bits + 1 : a.key_bits;
    const int passes = (bits + kTDigit - 1) / kTDigit;
    const int width = (bits + passes - 1) / passes;
    const int units = ntiles * kNW;
    uint32_t* ks = keys0;
    uint32_t* rs = rr0;
    uint32_t* kd = keys1;
    uint32_t* rd = rr1;
    for (int pass = 0; pass < passes; ++pass) {
        const int sh = pass * width;
        const int db = min(width, bits - sh);
        const int nd = 1 << db;
        const uint32_t dmask = static_cast<uint32_t>(nd - 1);
        for (int e = tid; e < units * nd; e += kNT) hist[e] = 0u;
        __syncthreads();
        // Item k of lane l of wave w in tile T is element T kTT + w 64 kTI + k 64 + l: ranks inside
        // the wave's unit follow the element order, so the sort is stable.
        for (int sweep = 0; sweep < 2; ++sweep) {
            for (int T = 0; T < ntiles; ++T) {
                uint32_t* uh = hist + (T * kNW + w) * nd;
                // The tile's keys (and, when scattering, entry indices) all loaded before the first
                // is ranked, from clamped positions past the row: one round trip per tile.
                uint32_t kt[kTI], rt[kTI];
#pragma unroll
                for (int k = 0; k < kTI; ++k) {
                    const int i = min(T * kTT + w * kWave * kTI + k * kWave + lane, n - 1);
                    kt[k] = ks[i];
                    rt[k] = sweep == 1 ? rs[i] : 0u;
                }
#pragma unroll
                for (int k = 0; k < kTI; ++k) {
                    const int i = T * kTT + w * kWave * kTI + k * kWave + lane;
                    const uint32_t key = i < n ? kt[k] : kTPad;
                    const uint32_t d = (key >> sh) & dmask;
                    uint32_t below, cnt;
                    digit_peers(d, db, below, cnt);
                    const uint32_t base = uh[d];
                    if (sweep == 1 && i < n) {
                        kd[base + below] = key;
                        rd[base + below] = rt[k];
                    }
                    if (below == 0) uh[d] = base + cnt;   // the lowest lane of the digit in this item
                }
            }
            __syncthreads();
            if (sweep == 0) {
                // Exclusive scan of the counts in (digit, unit) order: thread x owns `per`
                // consecutive elements e = x per + u, element e being (digit e / units, unit e % units).
                const int total = nd * units;
                const int per = (total + kNT - 1) / kNT;
                uint32_t local = 0;
                for (int u = 0; u < per; ++u) {
                    const int e = tid * per + u;
                    if (e < total) local += hist[(e % units) * nd + e / units];
                }
                uint32_t tot;
                uint32_t run = block_exclusive_add(local, wsum, add_phase, tot);
                for (int u = 0; u < per; ++u) {
                    const int e = tid * per + u;
                    if (e < total) {
                        uint32_t* h = hist + (e % units) * nd + e / units;
                        const uint32_t cnt = *h;
                        *h = run;
                        run += cnt;
                    }
                }
                __syncthreads();
            }
        }
        uint32_t* t0 = ks;
        ks = kd;
        kd = t0;
        t0 = rs;
        rs = rd;
        rd = t0;
    }
    const uint32_t* skey = ks;   // the sorted row
    const uint32_t* sr = rs;

    // Items of thread tid in tile T: positions p0 .. p0 + kTI - 1 (consecutive).
    struct Items {
        uint32_t key[kTI], rr[kTI];
        float x[kTI];
        uint32_t valid, isk, head, end, rep;   // bit k per item
        uint32_t prev_r;                        // the entry index before p0 (p0 > 0)
    };
    auto load_items = [&](int T, Items& it) {
        const int p0 = T * kTT + tid * kTI;
        // (every load issued from a clamped position, the values past the row dropped after: the
        // loads are in flight together)
#pragma unroll
        for (int k = 0; k < kTI; ++k) {
            const int pc = min(p0 + k, n - 1);
            it.key[k] = skey[pc];
            it.rr[k] = sr[pc];
        }
        const bool has_prev = p0 > 0 && p0 <= n;
        const int pp = min(max(p0 - 1, 0), n - 1);
        const uint32_t pkey_l = skey[pp], prev_l = sr[pp];
        const uint32_t nkey_l = skey[min(p0 + kTI, n - 1)];
#pragma unroll
        for (int k = 0; k < kTI; ++k) {
            if (p0 + k >= n) {
                it.key[k] = kTPad;
                it.rr[k] = 0u;
            }
        }
        const uint32_t pkey = has_prev ? pkey_l : kTPad;
        it.prev_r = has_prev ? prev_l : 0u;
        const uint32_t nkey = p0 + kTI < n ? nkey_l : kTPad;
        it.valid = it.isk = it.head = it.end = it.rep = 0u;
#pragma unroll
        for (int k = 0; k < kTI; ++k) {
            const uint32_t pk = k ? it.key[k - 1] : pkey;
            const uint32_t pr = k ? it.rr[k - 1] : it.prev_r;
            const bool valid = it.key[k] < key_lim;
            const bool head = !valid || !(pk < key_lim) || pk != it.key[k];
            const int r = static_cast<int>(it.rr[k]);
            const int t = token_of_entry(r, a.wr_magic);
            const int j = r - t * wr;
            const bool is_k = valid && j < W;
            const int pt = token_of_entry(static_cast<int>(pr), a.wr_magic);
            const int pj = static_cast<int>(pr) - pt * wr;
            const bool rep = !head && is_k && pj < W && pt == t;
            it.x[k] = (is_k && !rep) ? gate(t, j) : 0.0f;
            it.valid |= (valid ? 1u : 0u) << k;
            it.isk |= (is_k ? 1u : 0u) << k;
            it.head |= (head ? 1u : 0u) << k;
            it.rep |= (rep ? 1u : 0u) << k;
        }
#pragma unroll
        for (int k = 0; k < kTI; ++k) {
            const bool end = k + 1 < kTI ? ((it.head >> (k + 1)) & 1u)
                                         : (!(it.key[k] < key_lim) || !(nkey < key_lim) || nkey != it.key[k]);
            it.end |= (end ? 1u : 0u) << k;
        }
    };
    // The scan element of item k; `start` marks a segment start in scan order.
    auto elem = [&](const Items& it, int k, bool start) {
        const bool valid = (it.valid >> k) & 1u;
        const bool is_k = (it.isk >> k) & 1u;
        return SegW{it.x[k], 0.0f, valid ? (is_k ? 1u : 1u << 16) : 0u, (valid ? 1u : 0u) | (start ? kSegWHead : 0u)};
    };

    // ---- 3. reverse scan: the sums and counts after each position in its group.
    {
        SegW rcarry{};
        for (int T = ntiles - 1; T >= 0; --T) {
            Items it;
            load_items(T, it);
            SegW agg{};
#pragma unroll
            for (int k = kTI - 1; k >= 0; --k) agg = seg_combine(agg, elem(it, k, (it.end >> k) & 1u));
            SegW total;
            SegW run = seg_combine(rcarry, block_exclusive_seg<true>(agg, wtot, seg_phase, total));
            rcarry = seg_combine(rcarry, total);
            const int p0 = T * kTT + tid * kTI;
#pragma unroll
            for (int k = kTI - 1; k >= 0; --k) {
                const bool end = (it.end >> k) & 1u;
                const SegW after = end ? SegW{} : run;
                const int p = p0 + k;
                if (p < n) {
                    rev[3 * static_cast<int64_t>(p)] = __float_as_uint(after.s + after.c);
                    rev[3 * static_cast<int64_t>(p) + 1] = after.kq;
                    rev[3 * static_cast<int64_t>(p) + 2] = after.all & ~kSegWHead;
                }
                run = seg_combine(run, elem(it, k, end));
            }
        }
    }
    __syncthreads();   // every position's reverse results are stored

    // ---- 4. forward scan and every output.
    const int CW = C * W;
    const int L = a.tile_len;
    const int ntk = (CW + L - 1) / L;
    const int64_t tb = static_cast<int64_t>(c) * (ntk + 1);
    if (tid == 0) a.tiles_k[tb + ntk] = CW;
    uint32_t reps = 0;
    {
        SegW fcarry{};
        uint32_t kcar = 0, qcar = 0;   // K- and Q-row entries before the tile
        for (int T = 0; T < ntiles; ++T) {
            Items it;
            load_items(T, it);
            const int p0 = T * kTT + tid * kTI;
            SegW agg{};
            uint32_t nk = 0, nq = 0;   // this thread's entries of each kind (padding included)
#pragma unroll
            for (int k = 0; k < kTI; ++k) {
                agg = seg_combine(agg, elem(it, k, (it.head >> k) & 1u));
                if (p0 + k < n) {
                    const int r = static_cast<int>(it.rr[k]);
                    const int t = token_of_entry(r, a.wr_magic);
                    if (r - t * wr < W) ++nk;
                    else ++nq;
                }
            }
            SegW total;
            SegW run = seg_combine(fcarry, block_exclusive_seg<false>(agg, wtot, seg_phase, total));
            fcarry = seg_combine(fcarry, total);
            uint32_t ktot, qtot;
            uint32_t jk = kcar + block_exclusive_add(nk, wsum, add_phase, ktot);
            uint32_t jq = qcar + block_exclusive_add(nq, wsum, add_phase, qtot);
            kcar += ktot;
            qcar += qtot;
#pragma unroll
            for (int k = 0; k < kTI; ++k) {
                const int p = p0 + k;
                if (p >= n) break;
                const bool head = (it.head >> k) & 1u;
                const SegW before = head ? SegW{} : run;
                run = seg_combine(run, elem(it, k, head));
                const int r = static_cast<int>(it.rr[k]);
                const int t = token_of_entry(r, a.wr_magic);
                const int j = r - t * wr;
                const bool q = j >= W;
                const int ln = q ? j - W : j;
                const bool valid = (it.valid >> k) & 1u;
                const uint32_t pay = static_cast<uint32_t>(ln) | (q ? kIsQ : 0u) | (static_cast<uint32_t>(t) << kTokShift) |
                                     (valid ? 0u : kInvalid);
                const uint32_t* rv = rev + 3 * static_cast<int64_t>(p);
                const float rexv = __uint_as_float(rv[0]);
                const uint32_t akq = rv[1], aall = rv[2];
                const uint32_t bK = before.kq & 0xFFFFu, bQ = before.kq >> 16;
                const uint32_t aK = akq & 0xFFFFu, aQ = akq >> 16;
                const uint32_t bcnt = q ? bQ : bK, acnt = q ? aQ : aK;
                const uint32_t kg = min(bK + aK + ((valid && !q) ? 1u : 0u), 0xFFFFu);
                const uint32_t gsize = (before.all & ~kSegWHead) + aall + (valid ? 1u : 0u);
                const float s = run.s, cc = run.c;
                const float Lv = s + cc;
                const uint32_t pr = k ? it.rr[k - 1] : it.prev_r;
                const int pt = token_of_entry(static_cast<int>(pr), a.wr_magic);
                const bool pq = static_cast<int>(pr) - pt * wr >= W;
                const bool same_run = !head && pt == t && pq == q;
                const bool walk = valid && !same_run && bK != 0u;
                float v = 0.0f;
                if (valid) v = q ? load_val(a.q_val, cr + t * R + ln, a.vbf) : load_val(a.k_val, cw + t * W + ln, a.vbf);
                const uint32_t pos = valid ? (static_cast<uint32_t>(p) | min(acnt, kPosCountMax) << kPosAfterShift |
                                              min(bcnt + 1u + acnt, kPosCountMax) << kPosSizeShift)
                                           : static_cast<uint32_t>(p);
                const uint32_t el = valid ? (pay | min(bcnt, kDistMax) << kDistShift | (bcnt == 0u ? kFirst : 0u) |
                                             (acnt == 0u ? kLast : 0u))
                                          : (pay | kFirst | kLast);
                const uint32_t inv = static_cast<uint32_t>(p) |
                                     (walk ? (kg >= static_cast<uint32_t>(a.hot_min) ? kTHot : kTWalk) : 0u);
                if (a.rec != nullptr) {
                    a.rec[crow + p] = make_uint4(pay | (head ? kHead : 0u), __float_as_uint(s), __float_as_uint(cc),
                                                 __float_as_uint(v));
                }
                if (a.perm != nullptr) a.perm[crow + p] = r;
                if (a.hot != nullptr && valid && head && kg >= static_cast<uint32_t>(a.hot_min)) {
                    hot_buf[atomicAdd(&hot_n, 1u)] = make_uint2(static_cast<uint32_t>(p), gsize);
                }
                const bool last = valid && acnt == 0u;
                const bool only = last && bcnt == 0u;
                if (!q) {
                    const int64_t e = cw + t * W + ln;
                    const float cpe = valid ? tiled_group_exp(s, cc, rexv) : 1.0f;
                    const float sc = valid ? v * expf(rexv) : 0.0f;
                    const uint32_t slot = valid ? static_cast<uint32_t>(static_cast<int64_t>(it.key[k]) + id_base) : 0u;
                    a.spay_k[cw + jk] = el;
                    a.krec[cw + jk] = make_uint4(el, slot, __float_as_uint(sc), a.vbf ? f32_to_bf16_rne(cpe) << 16 : __float_as_uint(cpe));
                    if (jk % static_cast<uint32_t>(L) == 0u) {
                        a.tiles_k[tb + jk / static_cast<uint32_t>(L)] =
                            (el & kFirst) ? static_cast<int>(jk) : min(static_cast<int>(jk + acnt + 1u), CW);
                    }
                    if (a.log_k != nullptr) a.log_k[e] = Lv;
                    if (a.rex != nullptr) a.rex[e] = rexv;
                    if (a.cpe != nullptr) {
                        if (a.vbf) static_cast<uint16_t*>(a.cpe)[e] = static_cast<uint16_t>(f32_to_bf16_rne(cpe));
                        else static_cast<float*>(a.cpe)[e] = cpe;
                    }
                    if (a.k_eff != nullptr) {
                        const float ke = valid ? v * expf(Lv) : 0.0f;
                        if (a.vbf) static_cast<uint16_t*>(a.k_eff)[e] = static_cast<uint16_t>(f32_to_bf16_rne(ke));
                        else static_cast<float*>(a.k_eff)[e] = ke;
                    }
                    if (a.is_last != nullptr) a.is_last[e] = last ? 1 : 0;
                    if (a.is_only != nullptr) a.is_only[e] = only ? 1 : 0;
                    if (a.pos_k != nullptr) a.pos_k[e] = static_cast<int32_t>(pos);
                    if (a.inv_k != nullptr) a.inv_k[e] = inv;
                    reps += (it.rep >> k) & 1u;
                    ++jk;
                } else {
                    const int64_t e = cr + t * R + ln;
                    if (a.spay_q != nullptr) a.spay_q[cr + jq] = el;
                    if (a.log_q != nullptr) a.log_q[e] = Lv;
                    if (a.q_w != nullptr) {
                        const float qw = valid ? v * expf(Lv) : 0.0f;
                        if (a.vbf) static_cast<uint16_t*>(a.q_w)[e] = static_cast<uint16_t>(f32_to_bf16_rne(qw));
                        else static_cast<float*>(a.q_w)[e] = qw;
                    }
                    if (a.pos_q != nullptr) a.pos_q[e] = static_cast<int32_t>(pos);
                    if (a.q_last != nullptr) a.q_last[e] = last ? 1 : 0;
                    if (a.q_only != nullptr) a.q_only[e] = only ? 1 : 0;
                    if (a.inv_q != nullptr) a.inv_q[e] = inv;
                    ++jq;
                }
            }
        }
    }
    uint32_t rep_total;
    (void)block_exclusive_add(reps, wsum, add_phase, rep_total);
    if (tid == 0 && a.repeats != nullptr) a.repeats[c] = static_cast<int32_t>(rep_total);
    __syncthreads();   // every hot-group append is done
    if (a.hot != nullptr) {   // the hot list in position order
        const int nh = static_cast<int>(hot_n);
        uint2* out = a.hot + static_cast<int64_t>(c) * (a.hot_cap + 1);
        for (int x = tid; x < nh; x += kNT) {
            const uint2 me = hot_buf[x];
            int rank = 0;
            for (int y = 0; y < nh; ++y) rank += hot_buf[y].x < me.x ? 1 : 0;
            out[1 + rank] = me;
        }
        if (tid == 0) out[0] = make_uint2(static_cast<uint32_t>(nh), 0u);
    }
}

}  // namespace

size_t p1_tiled_lds_bytes(const sdm_p1_shape* s) {
    const size_t dyn = static_cast<size_t>(s->C * s->W / kHotMin) * sizeof(uint2);
    return dyn + sizeof(uint32_t) * (kTUnits << kTDigit) + 4096;   // dynamic part + the static arrays
}

int p1_tiled_lds_kernels(const void** fns, int cap) {
    if (cap < 1) return 0;
    fns[0] = reinterpret_cast<const void*>(&p1_tiled_kernel);
    return 1;
}

hipError_t p1_tiled_launch(const P1Launch& Lc, hipStream_t st) {
    const sdm_p1_shape* s = Lc.s;
    const sdm_p1_io* io = Lc.io;
    const bool pairs = io->a != nullptr || io->qk != nullptr;
    const PairPlan pp = pair_plan(s, pairs, Lc.lds_max);
    TiledArgs a;
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
    a.spay_k = reinterpret_cast<uint32_t*>(io->spay_k);
    a.spay_q = reinterpret_cast<uint32_t*>(io->spay_q);
    a.krec = reinterpret_cast<uint4*>(io->krec);
    a.tiles_k = io->tiles_k;
    a.repeats = io->repeats;
    a.perm = io->perm;
    a.status = io->status;
    a.rec = pairs ? static_cast<uint4*>(Lc.rec) : nullptr;
    a.inv_k = pairs ? static_cast<uint32_t*>(Lc.inv_k) : nullptr;
    a.inv_q = pairs ? static_cast<uint32_t*>(Lc.inv_q) : nullptr;
    a.hot = pairs ? static_cast<uint2*>(Lc.hot) : nullptr;
    a.sort = static_cast<uint32_t*>(Lc.sort);
    a.rev = static_cast<uint32_t*>(Lc.rev);
    a.stream_offset = s->stream_offset;
    a.C = s->C;
    a.W = s->W;
    a.R = s->R;
    a.P = s->P;
    a.key_bits = s->key_bits;
    a.first_partial = s->first_partial;
    a.valid_last = s->valid_last;
    a.tile_len = s->tile_len;
    a.hot_min = pp.hot_on ? kHotMin : INT_MAX;
    a.hot_cap = pp.hot_cap;
    a.wr_magic = static_cast<uint32_t>(((uint64_t(1) << 32) + static_cast<uint64_t>(s->W + s->R) - 1) /
                                       static_cast<uint64_t>(s->W + s->R));
    a.lane_gates = s->g_lane_stride != 0;
    a.id64 = s->idx_bytes == 8;
    a.vbf = s->val_bytes == 2;
    const size_t lds = static_cast<size_t>(pp.hot_cap) * sizeof(uint2);
    hipEvent_t e0 = io->events != nullptr ? io->events[0] : nullptr, e1 = io->events != nullptr ? io->events[1] : nullptr;
    void* kargs[] = {&a};
    g_p1_stage = "tiled kernel";
    hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(&p1_tiled_kernel), dim3(s->N), dim3(kNT), kargs, lds, st,
                                      e0, e1, 0);
    if (e == hipSuccess) e = p1_ordinal_launch(s, io, st);
    if (e != hipSuccess || !pairs || io->defer_pairs) return e;
    return pair_launch(Lc, pp, true, st);
}

}  // namespace sdm
