// Phase 1 of the chunked SDM recurrence on gfx950: one workgroup per chunk sorts the chunk's
// entries by slot in LDS, runs the two segmented scans and writes every per-entry output, the
// sorted kind rows, the mover records and the tile bounds; a second kernel sums the A / QK
// triangles.
//
// Definitions: page "sparse_delta_memory/cuda/phase1_cuda.py" (module docstring; keys and payloads
// of p1_keys_zw_kernel; the scan semantics of p1_scan_kernel; the pair terms of p1_pairs_kernel).
// The kernels here are an independent gfx950 design: a wave64 LSD radix sort whose ranks come
// from ballot-built peer masks (stable by construction, no atomics), TwoSum-compensated
// segmented scans combined in a fixed tree, and a pair kernel with one writer per output cell.
#include "sdm_device.hpp"
#include "sdm_launch.hpp"

namespace sdm {
namespace {

constexpr int kNT = kP1Threads;   // 1024 threads = 16 waves per chunk
constexpr int kNW = kNT / kWave;
constexpr int kRadix = 256;       // 8-bit digits

struct P1Args {
    const int32_t* k_idx;
    const int32_t* q_idx;
    const float* k_val;
    const float* q_val;
    const float* g;
    float* log_k;
    float* rex;
    float* cpe;
    float* k_eff;
    int8_t* is_last;
    int8_t* is_only;
    int32_t* pos_k;
    float* log_q;
    float* q_w;
    int32_t* pos_q;
    int8_t* q_last;
    int8_t* q_only;
    int32_t* spay_k;
    int32_t* spay_q;
    int4* krec;
    int32_t* tiles_k;
    int32_t* repeats;
    uint4* rec;
    uint32_t* inv;
    int C, W, R, P, key_bits, first_partial, valid_last, tile_len;
    int64_t stream_offset;
};

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

// Exclusive segmented scan of one element per thread over the block, in thread order
// (REV: descending thread order). Fixed combine tree: lane doubling, then the wave totals in
// wave order. wtot: kNW elements of LDS.
template <bool REV>
__device__ __forceinline__ Seg block_exclusive_seg(Seg agg, Seg* wtot) {
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
    __syncthreads();
    Seg pre = seg_zero();
    if (REV) {
        for (int ww = kNW - 1; ww > w; --ww) pre = seg_combine(pre, wtot[ww]);
    } else {
        for (int ww = 0; ww < w; ++ww) pre = seg_combine(pre, wtot[ww]);
    }
    __syncthreads();
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
    __syncthreads();
    uint32_t pre = 0, tot = 0;
    for (int ww = 0; ww < kNW; ++ww) {
        const uint32_t x = wsum[ww];
        pre += ww < w ? x : 0u;
        tot += x;
    }
    __syncthreads();
    total = tot;
    return pre + incl - v;
}

// Stable LSD radix sort of the block's kNT * IPT (key, value) pairs over bits [0, bits).
// Items live in registers in striped order (item k of lane l of wave w is element
// w * 64 * IPT + k * 64 + l). Per 8-bit digit: ranks inside the wave from ballot-built peer
// masks processed item slice by item slice (so equal digits keep element order), per-wave digit
// counts in LDS, their exclusive prefix over (digit, wave), then a scatter into skey / sval.
// On return skey / sval hold the sorted sequence.
template <int IPT>
__device__ void block_radix_sort(uint32_t (&key)[IPT], uint32_t (&val)[IPT], int bits, uint32_t* skey,
                                 uint16_t* sval, uint32_t* hist, uint32_t* dtot, uint32_t* wsum) {
    const int lane = static_cast<int>(lane_id());
    const int w = threadIdx.x / kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    uint32_t* my_hist = hist + w * kRadix;
    for (int sh = 0; sh < bits; sh += 8) {
        const int db = min(8, bits - sh);
        const uint32_t dmask = (1u << db) - 1u;
        for (int d = lane; d < kRadix; d += kWave) my_hist[d] = 0u;
        __syncthreads();
        uint32_t rank[IPT];
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
            rank[k] = base + below;
            if (below == 0) my_hist[d] = base + cnt;   // the slice's lowest lane of this digit
        }
        __syncthreads();
        if (threadIdx.x < kRadix) {
            const int d = threadIdx.x;
            uint32_t run = 0;
            for (int ww = 0; ww < kNW; ++ww) {
                const uint32_t cnt = hist[ww * kRadix + d];
                hist[ww * kRadix + d] = run;
                run += cnt;
            }
            dtot[d] = run;
        }
        __syncthreads();
        uint32_t dv = 0, dincl = 0;
        if (threadIdx.x < kRadix) {
            dv = dtot[threadIdx.x];
            dincl = dv;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const uint32_t x = __shfl_up(dincl, o, kWave);
                if (lane >= o) dincl += x;
            }
            if (lane == kWave - 1) wsum[w] = dincl;
        }
        __syncthreads();
        if (threadIdx.x < kRadix) {
            const int d = threadIdx.x;
            uint32_t pre = 0;
            for (int ww = 0; ww < w; ++ww) pre += wsum[ww];
            const uint32_t base = pre + dincl - dv;   // exclusive start of digit d
            for (int ww = 0; ww < kNW; ++ww) hist[ww * kRadix + d] += base;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const uint32_t d = (key[k] >> sh) & dmask;
            const uint32_t pos = my_hist[d] + rank[k];
            skey[pos] = key[k];
            sval[pos] = static_cast<uint16_t>(val[k]);
        }
        __syncthreads();
        if (sh + 8 < bits) {
#pragma unroll
            for (int k = 0; k < IPT; ++k) {
                const int i = w * kWave * IPT + k * kWave + lane;
                key[k] = skey[i];
                val[k] = sval[i];
            }
            __syncthreads();
        }
    }
}

template <int IPT>
__global__ void __launch_bounds__(kNT) p1_main_kernel(P1Args a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NP = kNT * IPT;
    uint32_t* skey = reinterpret_cast<uint32_t*>(smem);
    uint16_t* sval = reinterpret_cast<uint16_t*>(skey + NP);
    uint32_t* hist = reinterpret_cast<uint32_t*>(sval + NP);
    float* gates = reinterpret_cast<float*>(hist + kNW * kRadix);
    __shared__ Seg wtot[kNW];
    __shared__ uint32_t wsum[kNW];
    __shared__ uint32_t dtot[kRadix];

    const int c = blockIdx.x;
    const int C = a.C, W = a.W, R = a.R;
    const int wr = W + R;
    const int n = C * wr;
    const int tv = c >= a.first_partial ? a.valid_last : C;
    const int kb = a.key_bits;
    const uint32_t key_lim = 1u << kb;          // valid keys are below; invalid = key_lim
    const uint32_t pad_key = (2u << kb) - 1u;   // padding past the row sorts last
    const int64_t id_base = static_cast<int64_t>(c % a.P) * a.stream_offset;
    const int64_t cw = static_cast<int64_t>(c) * C * W;
    const int64_t cr = static_cast<int64_t>(c) * C * R;
    const int64_t crow = static_cast<int64_t>(c) * n;
    const int lane = static_cast<int>(lane_id());
    const int w = threadIdx.x / kWave;

    for (int t = threadIdx.x; t < C; t += kNT) gates[t] = t < tv ? a.g[static_cast<int64_t>(c) * C + t] : 0.0f;

    // ---- keys: element i of the striped layout is entry r = i of the chunk.
    uint32_t key[IPT], val[IPT];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        const int i = w * kWave * IPT + k * kWave + lane;
        val[k] = static_cast<uint32_t>(i);
        key[k] = pad_key;
        if (i < n) {
            const int t = i / wr;
            const int j = i - t * wr;
            const int64_t id = j < W ? static_cast<int64_t>(a.k_idx[cw + t * W + j])
                                     : static_cast<int64_t>(a.q_idx[cr + t * R + (j - W)]);
            key[k] = t < tv ? static_cast<uint32_t>(id - id_base) & (key_lim - 1u) : key_lim;
        }
    }
    block_radix_sort<IPT>(key, val, kb + 1, skey, sval, hist, dtot, wsum);

    // ---- scans over the sorted row, blocked layout: thread x holds positions x*IPT .. +IPT-1.
    const int p0 = threadIdx.x * IPT;
    uint32_t kk[IPT], rr[IPT];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        kk[k] = skey[p0 + k];
        rr[k] = sval[p0 + k];
    }
    const uint32_t prev_key = p0 > 0 ? skey[p0 - 1] : pad_key;
    const uint32_t prev_r = p0 > 0 ? sval[p0 - 1] : 0u;
    const uint32_t next_key = p0 + IPT < NP ? skey[p0 + IPT] : pad_key;

    // Group heads and ends, gate contributions, repeats.
    uint32_t heads = 0, ends = 0, repeat_count = 0;
    float x[IPT];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        const uint32_t pk = k ? kk[k - 1] : prev_key;
        const uint32_t pr = k ? rr[k - 1] : prev_r;
        const bool valid = kk[k] < key_lim;
        const bool pvalid = pk < key_lim && (p0 + k) > 0;
        const bool head = !valid || !pvalid || kk[k] != pk;
        heads |= (head ? 1u : 0u) << k;
        const int t = static_cast<int>(rr[k]) / wr;
        const int j = static_cast<int>(rr[k]) - t * wr;
        const bool is_k = valid && j < W;
        const int pt = static_cast<int>(pr) / wr;
        const int pj = static_cast<int>(pr) - pt * wr;
        const bool rep = !head && is_k && pj < W && pt == t;
        repeat_count += rep ? 1u : 0u;
        x[k] = (is_k && !rep) ? gates[t] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        bool end;
        if (k + 1 < IPT) {
            end = (heads >> (k + 1)) & 1u;
        } else {
            end = !(kk[k] < key_lim) || !(next_key < key_lim) || next_key != kk[k];
        }
        ends |= (end ? 1u : 0u) << k;
    }
    auto item = [&](int k, bool seg_start) {
        const bool valid = kk[k] < key_lim;
        const int t = static_cast<int>(rr[k]) / wr;
        const bool q = static_cast<int>(rr[k]) - t * wr >= W;
        const uint32_t f = (valid ? (q ? kSegQOne : 1u) : 0u) | (seg_start ? kSegHead : 0u);
        return Seg{x[k], 0.0f, f};
    };

    // Reverse pass: sums and peer counts after each entry inside its group.
    Seg agg = seg_zero();
#pragma unroll
    for (int k = IPT - 1; k >= 0; --k) agg = seg_combine(agg, item(k, (ends >> k) & 1u));
    Seg run = block_exclusive_seg<true>(agg, wtot);
    float rexv[IPT];
    uint32_t aft[IPT];
#pragma unroll
    for (int k = IPT - 1; k >= 0; --k) {
        const Seg after = ((ends >> k) & 1u) ? seg_zero() : run;
        rexv[k] = after.s + after.c;
        aft[k] = after.f & ~kSegHead;
        run = seg_combine(run, item(k, (ends >> k) & 1u));
    }

    // Forward pass: inclusive log-cumsums, peers before, and every output.
    agg = seg_zero();
#pragma unroll
    for (int k = 0; k < IPT; ++k) agg = seg_combine(agg, item(k, (heads >> k) & 1u));
    run = block_exclusive_seg<false>(agg, wtot);
    // Index of each entry in its kind's sorted row: plain counts of K-kind and Q-kind entries.
    uint32_t kind_cnt = 0;
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        if (p0 + k < n) {
            const int t = static_cast<int>(rr[k]) / wr;
            kind_cnt += (static_cast<int>(rr[k]) - t * wr >= W) ? kSegQOne : 1u;
        }
    }
    uint32_t kind_total;
    const uint32_t kind_base = block_exclusive_add(kind_cnt, wsum, kind_total);
    uint32_t jk = kind_base & 0xFFFFu, jq = kind_base >> 16;
    uint32_t rep_total;
    (void)block_exclusive_add(repeat_count, wsum, rep_total);
    if (threadIdx.x == 0 && a.repeats != nullptr) a.repeats[c] = static_cast<int32_t>(rep_total);

    const int nk = C * W;
    const int L = a.tile_len;
    const int ntk = (nk + L - 1) / L;
    const int64_t tb = static_cast<int64_t>(c) * (ntk + 1);
    if (threadIdx.x == 0) a.tiles_k[tb + ntk] = nk;

#pragma unroll
    for (int k = 0; k < IPT; ++k) {
        const bool head = (heads >> k) & 1u;
        const Seg before = head ? seg_zero() : run;
        run = seg_combine(run, item(k, head));
        const int rho = p0 + k;
        if (rho >= n) continue;
        const bool valid = kk[k] < key_lim;
        const int t = static_cast<int>(rr[k]) / wr;
        const int j = static_cast<int>(rr[k]) - t * wr;
        const bool q = j >= W;
        const int ln = q ? j - W : j;
        const uint32_t bcnt = q ? ((before.f >> 16) & 0x7FFFu) : (before.f & 0xFFFFu);
        const uint32_t acnt = q ? ((aft[k] >> 16) & 0x7FFFu) : (aft[k] & 0xFFFFu);
        const uint32_t pay = static_cast<uint32_t>(ln) | (q ? kIsQ : 0u) | (static_cast<uint32_t>(t) << kTokShift) |
                             (valid ? 0u : kInvalid);
        const uint32_t packed = valid ? (static_cast<uint32_t>(rho) | min(acnt, kPosCountMax) << kPosAfterShift |
                                         min(bcnt + 1u + acnt, kPosCountMax) << kPosSizeShift)
                                      : static_cast<uint32_t>(rho);
        const uint32_t elem = valid ? ((pay & kEntryMask) | min(bcnt, kDistMax) << kDistShift |
                                       (bcnt == 0 ? kFirst : 0u) | (acnt == 0 ? kLast : 0u))
                                    : (pay | kFirst | kLast);
        const float Lv = run.s + run.c;
        const float v = valid ? (q ? a.q_val[cr + t * R + ln] : a.k_val[cw + t * W + ln]) : 0.0f;
        const float ef = expf(Lv);
        if (q) {
            const int64_t o = cr + t * R + ln;
            if (a.log_q) a.log_q[o] = Lv;
            if (a.q_w) a.q_w[o] = v * ef;
            if (a.pos_q) a.pos_q[o] = static_cast<int32_t>(packed);
            const bool ql = valid && acnt == 0;
            if (a.q_last) a.q_last[o] = ql ? 1 : 0;
            if (a.q_only) a.q_only[o] = (ql && bcnt == 0) ? 1 : 0;
            if (a.spay_q) a.spay_q[cr + jq] = static_cast<int32_t>(elem);
            ++jq;
        } else {
            const int64_t o = cw + t * W + ln;
            // exp of the group total: the compensated log-cumsum plus the sum after (TwoSum).
            const float gs = run.s + rexv[k];
            const float gb = gs - run.s;
            const float ge = (run.s - (gs - gb)) + (rexv[k] - gb);
            const float G = gs + (run.c + ge);
            const float cpe_v = valid ? expf(G) : 1.0f;
            const bool last = valid && acnt == 0;
            if (a.log_k) a.log_k[o] = Lv;
            if (a.rex) a.rex[o] = rexv[k];
            if (a.cpe) a.cpe[o] = cpe_v;
            if (a.k_eff) a.k_eff[o] = v * ef;
            if (a.is_last) a.is_last[o] = last ? 1 : 0;
            if (a.is_only) a.is_only[o] = (last && bcnt == 0) ? 1 : 0;
            if (a.pos_k) a.pos_k[o] = static_cast<int32_t>(packed);
            a.spay_k[cw + jk] = static_cast<int32_t>(elem);
            const float sc = valid ? v * expf(rexv[k]) : 0.0f;
            const int32_t slot = valid ? static_cast<int32_t>(static_cast<int64_t>(kk[k]) + id_base) : 0;
            a.krec[cw + jk] = make_int4(static_cast<int32_t>(elem), slot, __float_as_int(sc), __float_as_int(cpe_v));
            if (static_cast<int>(jk) % L == 0) {
                const int ti = static_cast<int>(jk) / L;
                a.tiles_k[tb + ti] = (elem & kFirst) ? static_cast<int>(jk) : min(static_cast<int>(jk + acnt + 1u), nk);
            }
            ++jk;
        }
        a.rec[crow + rho] = make_uint4(pay | (head ? kHead : 0u), __float_as_uint(run.s), __float_as_uint(run.c),
                                       __float_as_uint(v));
        a.inv[crow + rr[k]] = static_cast<uint32_t>(rho);
    }
}

// Pair sums. Block (chunk, triangle): one thread per row i walks the entries of token i of its
// kind (K for A, Q for QK) in lane order; each walk goes from the entry's nearest earlier entry of
// its group back to the group head and adds, per earlier K entry f of token j (j != i for A),
// val_e * val_f * exp(L_e - L_f) to cell (i, j) with its own rounding. Every cell has one writer
// thread and a fixed term order. The triangle lives in LDS and is written out as a dense [C, C]
// matrix with zeros outside it.
struct PairArgs {
    const uint4* rec;
    const uint32_t* inv;
    float* a;
    float* qk;
    int C, W, R, first_partial, valid_last;
};

constexpr int kPairThreads = 256;

__global__ void __launch_bounds__(kPairThreads) p1_pairs_kernel(PairArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* tri = reinterpret_cast<float*>(smem);
    const bool q = blockIdx.y == 1;
    float* out = q ? a.qk : a.a;
    if (out == nullptr) return;   // block-uniform
    const int c = blockIdx.x;
    const int C = a.C, W = a.W, R = a.R;
    const int wr = W + R;
    const int n = C * wr;
    const int tv = c >= a.first_partial ? a.valid_last : C;
    const int tri_size = C * (C + 1) / 2;
    for (int e = threadIdx.x; e < tri_size; e += kPairThreads) tri[e] = 0.0f;
    __syncthreads();
    const int64_t crow = static_cast<int64_t>(c) * n;
    const uint4* rec = a.rec + crow;
    const int i = threadIdx.x;
    if (i < tv) {
        float* row = tri + i * (i + 1) / 2;
        const int lanes = q ? R : W;
        for (int ln = 0; ln < lanes; ++ln) {
            const int r = i * wr + (q ? W + ln : ln);
            const uint32_t rho = a.inv[crow + r];
            const uint4 own = rec[rho];
            if (own.x & kHead) continue;
            const float se = __uint_as_float(own.y), ce = __uint_as_float(own.z), ve = __uint_as_float(own.w);
            for (int p = static_cast<int>(rho) - 1; p >= 0; --p) {
                const uint4 f = rec[p];
                if (!(f.x & (kIsQ | kInvalid))) {
                    const int jt = static_cast<int>((f.x >> kTokShift) & 0xFFu);
                    if (q || jt != i) {
                        const float d = (se - __uint_as_float(f.y)) + (ce - __uint_as_float(f.z));
                        const float term = (ve * __uint_as_float(f.w)) * expf(d);
                        row[jt] = row[jt] + term;
                    }
                }
                if (f.x & kHead) break;
            }
        }
    }
    __syncthreads();
    const int64_t ob = static_cast<int64_t>(c) * C * C;
    for (int e = threadIdx.x; e < C * C; e += kPairThreads) {
        const int ii = e / C;
        const int jj = e - ii * C;
        const bool inside = q ? (jj <= ii) : (jj < ii);
        out[ob + e] = inside ? tri[ii * (ii + 1) / 2 + jj] : 0.0f;
    }
}

template <int IPT>
size_t main_lds_bytes() {
    return static_cast<size_t>(kNT) * IPT * (sizeof(uint32_t) + sizeof(uint16_t)) + kNW * kRadix * sizeof(uint32_t) +
           256 * sizeof(float);
}

template <int IPT>
hipError_t launch_main(const P1Args& args, int N, hipStream_t st) {
    const size_t lds = main_lds_bytes<IPT>();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&p1_main_kernel<IPT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(p1_main_kernel<IPT>, dim3(N), dim3(kNT), lds, st, args);
    return hipGetLastError();
}

}  // namespace

P1Workspace p1_workspace_layout(const sdm_p1_shape* s) {
    const size_t n = static_cast<size_t>(s->C) * static_cast<size_t>(s->W + s->R);
    const size_t N = static_cast<size_t>(s->N);
    P1Workspace w;
    w.rec_off = 0;
    const size_t rec_bytes = N * n * sizeof(uint4);
    w.inv_off = (rec_bytes + 255) / 256 * 256;
    const size_t inv_bytes = N * n * sizeof(uint32_t);
    w.total = w.inv_off + (inv_bytes + 255) / 256 * 256;
    return w;
}

hipError_t p1_launch(const P1Launch& Lc, hipStream_t st) {
    const sdm_p1_shape* s = Lc.s;
    const sdm_p1_io* io = Lc.io;
    if (s->N == 0) return hipSuccess;
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
    a.spay_k = io->spay_k;
    a.spay_q = io->spay_q;
    a.krec = reinterpret_cast<int4*>(io->krec);
    a.tiles_k = io->tiles_k;
    a.repeats = io->repeats;
    a.rec = static_cast<uint4*>(Lc.rec);
    a.inv = static_cast<uint32_t*>(Lc.inv);
    a.C = s->C;
    a.W = s->W;
    a.R = s->R;
    a.P = s->P;
    a.key_bits = s->key_bits;
    a.first_partial = s->first_partial;
    a.valid_last = s->valid_last;
    a.tile_len = s->tile_len;
    a.stream_offset = s->stream_offset;
    const int n = s->C * (s->W + s->R);
    hipError_t e;
    if (io->events != nullptr && (e = hipEventRecord(io->events[0], st)) != hipSuccess) return e;
    if (n <= kNT) {
        e = launch_main<1>(a, s->N, st);
    } else if (n <= 2 * kNT) {
        e = launch_main<2>(a, s->N, st);
    } else if (n <= 4 * kNT) {
        e = launch_main<4>(a, s->N, st);
    } else if (n <= 8 * kNT) {
        e = launch_main<8>(a, s->N, st);
    } else {
        e = launch_main<16>(a, s->N, st);
    }
    if (e != hipSuccess) return e;
    if (io->events != nullptr && (e = hipEventRecord(io->events[1], st)) != hipSuccess) return e;
    if (io->a == nullptr && io->qk == nullptr) {
        return io->events != nullptr ? hipEventRecord(io->events[2], st) : hipSuccess;
    }
    PairArgs pa;
    pa.rec = a.rec;
    pa.inv = a.inv;
    pa.a = io->a;
    pa.qk = io->qk;
    pa.C = s->C;
    pa.W = s->W;
    pa.R = s->R;
    pa.first_partial = s->first_partial;
    pa.valid_last = s->valid_last;
    const size_t lds = static_cast<size_t>(s->C) * (s->C + 1) / 2 * sizeof(float);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&p1_pairs_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(p1_pairs_kernel, dim3(s->N, 2), dim3(kPairThreads), lds, st, pa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return io->events != nullptr ? hipEventRecord(io->events[2], st) : hipSuccess;
}

}  // namespace sdm
