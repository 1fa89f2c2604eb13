// Device helpers shared by the Phase-1 kernels (the on-chip kernel and the long-row kernel):
// workgroup constants, output stores, the segmented-scan elements with their TwoSum-compensated
// combine, and wave / block scans on DPP lane moves with a fixed combine tree.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdm_device.hpp"
#include "sdm_launch.hpp"

namespace sdm {
namespace {

constexpr int kNT = kP1Threads;   // 1024 threads = 16 waves per chunk
constexpr int kNW = kNT / kWave;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Store of element i (a 32-bit index) of a T array in the global address space (a pointer read from
// the LDS table would otherwise make a flat store, and a 64-bit index 64-bit address arithmetic).
template <typename T>
__device__ __forceinline__ void gstore(const void* base, uint32_t i, T v) {
    typedef __attribute__((address_space(1))) T GT;
    reinterpret_cast<GT*>(reinterpret_cast<uintptr_t>(base))[i] = v;
}

// The same store marked non-temporal (outputs that nothing in the step reads back).
template <typename T>
__device__ __forceinline__ void gstore_nt(const void* base, uint32_t i, T v) {
    typedef __attribute__((address_space(1))) T GT;
    __builtin_nontemporal_store(v, reinterpret_cast<GT*>(reinterpret_cast<uintptr_t>(base)) + i);
}

// Value-typed outputs (cpe, k_eff, q_w) with bfloat16 values: the float32 result rounded to
// bfloat16, nearest even.
__device__ __forceinline__ uint32_t bf16_rn(float x) { return f32_to_bf16_rne(x); }
// Four values from element i (a multiple of 4; 16-byte / 8-byte aligned rows).
__device__ __forceinline__ f32x4 load_val4(const void* p, int64_t i, int bf) {
    if (bf) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p) + i);
        return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xFFFF0000u)};
    }
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
}
// The 32-bit pattern a float32 record field holds for a value-typed quantity.
__device__ __forceinline__ uint32_t val_bits32(float x, int bf) { return bf ? bf16_rn(x) << 16 : __float_as_uint(x); }
__device__ __forceinline__ void store_val(const void* base, uint32_t i, float v, int bf) {
    if (bf) gstore<uint16_t>(base, i, static_cast<uint16_t>(bf16_rn(v)));
    else gstore<float>(base, i, v);
}
// Entries 4 i4 .. 4 i4 + 3 (non-temporal stores).
__device__ __forceinline__ void store_val4(const void* base, uint32_t i4, f32x4 v, int bf) {
    if (bf) gstore_nt<u32x2>(base, i4, u32x2{bf16_rn(v.x) | bf16_rn(v.y) << 16, bf16_rn(v.z) | bf16_rn(v.w) << 16});
    else gstore_nt<f32x4>(base, i4, v);
}

// r / (W + R) for entry indices r < 2^17 and W + R <= 512 (multiply-high by a rounded-up
// reciprocal; the error term r / 2^32 stays below 1 / (W + R)).
__device__ __forceinline__ int token_of_entry(int r, uint32_t magic) {
    return static_cast<int>(__umulhi(static_cast<uint32_t>(r), magic));
}

// t * m for the factors of entry decoding and row offsets (tokens and lane counts: both below 2^24,
// the product below 2^31), on the full-rate 24-bit multiply.
__device__ __forceinline__ int mul24(int t, int m) {
    return static_cast<int>(__umul24(static_cast<unsigned>(t), static_cast<unsigned>(m)));
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

// Lane moves by DPP (GFX9 encodings): inside rows of 16 lanes row_shr:n (0x110 + n) reads lane
// l - n and row_shl:n (0x100 + n) lane l + n; row_bcast:15 (0x142) gives rows 1 and 3 the last lane
// of the row before, row_bcast:31 (0x143) gives rows 2 and 3 lane 31; wave_shr:1 (0x138) and
// wave_shl:1 (0x130) move the whole wave by one lane. A lane with no source (or in a row the mask
// leaves out) reads 0, which is the zero scan element: seg_combine(zero, b) == b bit for bit.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, true));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ Seg seg_dpp(const Seg& v) {
    return Seg{__uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(v.s))),
               __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(v.c))), dpp_u32<CTRL, ROWS>(v.f)};
}
__device__ __forceinline__ Seg seg_from_lane(const Seg& v, int src) {
    return Seg{__shfl(v.s, src, kWave), __shfl(v.c, src, kWave), static_cast<uint32_t>(__shfl(static_cast<int>(v.f), src, kWave))};
}

// Inclusive segmented scan over the lanes of a wave in scan order (REV: descending lanes). Fixed
// tree: doubling steps inside each row of 16 lanes, then the rows in order (forward: the last lane
// of the row before, by row broadcasts; reverse: the first lane of the row after, then lane 32).
template <bool REV, class T>
__device__ __forceinline__ T wave_inclusive_seg(T x) {
    if constexpr (!REV) {
        x = seg_combine(seg_dpp<0x111, 0xF>(x), x);
        x = seg_combine(seg_dpp<0x112, 0xF>(x), x);
        x = seg_combine(seg_dpp<0x114, 0xF>(x), x);
        x = seg_combine(seg_dpp<0x118, 0xF>(x), x);
        x = seg_combine(seg_dpp<0x142, 0xA>(x), x);
        x = seg_combine(seg_dpp<0x143, 0xC>(x), x);
    } else {
        const int lane = static_cast<int>(lane_id());
        x = seg_combine(seg_dpp<0x101, 0xF>(x), x);
        x = seg_combine(seg_dpp<0x102, 0xF>(x), x);
        x = seg_combine(seg_dpp<0x104, 0xF>(x), x);
        x = seg_combine(seg_dpp<0x108, 0xF>(x), x);
        T o = seg_from_lane(x, (lane | 15) + 1);   // rows 0 and 2: the first lane of the next row
        if ((lane & 16) == 0) x = seg_combine(o, x);
        o = seg_from_lane(x, 32);                    // rows 0 and 1: lane 32 (rows 2 and 3 summed)
        if (lane < 32) x = seg_combine(o, x);
    }
    return x;
}

// Inclusive sum over the lanes of a wave (the same doubling steps and row order).
__device__ __forceinline__ uint32_t wave_inclusive_add(uint32_t x) {
    x += dpp_u32<0x111, 0xF>(x);
    x += dpp_u32<0x112, 0xF>(x);
    x += dpp_u32<0x114, 0xF>(x);
    x += dpp_u32<0x118, 0xF>(x);
    x += dpp_u32<0x142, 0xA>(x);
    x += dpp_u32<0x143, 0xC>(x);
    return x;
}

__device__ __forceinline__ Seg seg_readlane(const Seg& v, int l) {
    return Seg{__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v.s), l)),
               __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v.c), l)),
               static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v.f), l))};
}

// Segmented-scan element of the long-row path (rows up to 2^17 entries): a compensated float sum,
// the valid K and Q counts saturating at 65535 each (bits 0-15, 16-31 of kq; saturating sums of
// non-negative counts stay associative, and every use of a count reads it through a cap of at
// most 4095 or a test against zero), and the exact count of valid entries of either kind with the
// segment-start flag (bits 0-17 and 31 of all).
struct SegW {
    float s;
    float c;
    uint32_t kq;
    uint32_t all;
};
constexpr uint32_t kSegWHead = 0x80000000u;

__device__ __forceinline__ uint32_t sat_add16x2(uint32_t a, uint32_t b) {
    const uint32_t lo = min((a & 0xFFFFu) + (b & 0xFFFFu), 0xFFFFu);
    const uint32_t hi = min((a >> 16) + (b >> 16), 0xFFFFu);
    return lo | hi << 16;
}

__device__ __forceinline__ SegW seg_combine(const SegW& a, const SegW& b) {
    if (b.all & kSegWHead) return b;
    const float s = a.s + b.s;
    const float bb = s - a.s;
    const float err = (a.s - (s - bb)) + (b.s - bb);
    return SegW{s, (a.c + b.c) + err, sat_add16x2(a.kq, b.kq), ((a.all & ~kSegWHead) + (b.all & ~kSegWHead)) | (a.all & kSegWHead)};
}
template <int CTRL, int ROWS>
__device__ __forceinline__ SegW seg_dpp(const SegW& v) {
    return SegW{__uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(v.s))), __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(v.c))),
                dpp_u32<CTRL, ROWS>(v.kq), dpp_u32<CTRL, ROWS>(v.all)};
}
__device__ __forceinline__ SegW seg_from_lane(const SegW& v, int src) {
    return SegW{__shfl(v.s, src, kWave), __shfl(v.c, src, kWave), static_cast<uint32_t>(__shfl(static_cast<int>(v.kq), src, kWave)),
                static_cast<uint32_t>(__shfl(static_cast<int>(v.all), src, kWave))};
}
__device__ __forceinline__ SegW seg_readlane(const SegW& v, int l) {
    return SegW{__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v.s), l)),
                __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v.c), l)),
                static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v.kq), l)),
                static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v.all), l))};
}

// Exclusive segmented scan of one element per thread over the block, in thread order
// (REV: descending). Fixed tree: the wave scans above; then every wave scans the 16 wave totals
// itself in the first row of its lanes (doubling steps in scan order) and takes its own prefix by
// readlane, so one barrier suffices. The totals alternate between two LDS buffers (`phase`, the
// same count in every thread): a wave that runs ahead writes the other buffer, and cannot get two
// scans ahead, since writing again needs every wave past the barrier of the scan in between.
// `total` receives the block's combined element. wtot: 2 kNW elements of LDS.
template <bool REV, class T>
__device__ __forceinline__ T block_exclusive_seg(T agg, T* wtot, uint32_t& phase, T& total) {
    static_assert(kNW == 16, "one DPP row of wave totals");
    const int lane = static_cast<int>(lane_id());
    const int w = threadIdx.x / kWave;
    T* buf = wtot + (phase & 1u) * kNW;
    ++phase;
    const T incl = wave_inclusive_seg<REV>(agg);
    const T ex = REV ? seg_dpp<0x130, 0xF>(incl) : seg_dpp<0x138, 0xF>(incl);
    if (REV ? (lane == 0) : (lane == kWave - 1)) buf[w] = incl;
    lds_barrier();
    // Lane i < 16 holds the i-th wave total in scan order.
    const T v = lane < kNW ? buf[REV ? kNW - 1 - lane : lane] : T{};
    T inc = seg_combine(seg_dpp<0x111, 0xF>(v), v);
    inc = seg_combine(seg_dpp<0x112, 0xF>(inc), inc);
    inc = seg_combine(seg_dpp<0x114, 0xF>(inc), inc);
    inc = seg_combine(seg_dpp<0x118, 0xF>(inc), inc);
    const T exw = seg_dpp<0x111, 0xF>(inc);
    total = seg_readlane(inc, kNW - 1);
    return seg_combine(seg_readlane(exw, REV ? kNW - 1 - w : w), ex);
}

// Exclusive integer sum over the block in thread order; `total` receives the block sum.
// wsum: 2 kNW words of LDS, used in alternation as in block_exclusive_seg.
__device__ __forceinline__ uint32_t block_exclusive_add(uint32_t v, uint32_t* wsum, uint32_t& phase, uint32_t& total) {
    const int lane = static_cast<int>(lane_id());
    const int w = threadIdx.x / kWave;
    uint32_t* buf = wsum + (phase & 1u) * kNW;
    ++phase;
    const uint32_t incl = wave_inclusive_add(v);
    if (lane == kWave - 1) buf[w] = incl;
    lds_barrier();
    const uint32_t x = lane < kNW ? buf[lane & (kNW - 1)] : 0u;
    uint32_t inc = x;
    inc += dpp_u32<0x111, 0xF>(inc);
    inc += dpp_u32<0x112, 0xF>(inc);
    inc += dpp_u32<0x114, 0xF>(inc);
    inc += dpp_u32<0x118, 0xF>(inc);
    total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(inc), kNW - 1));
    const uint32_t pre = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(inc - x), w));
    return pre + incl - v;
}

// Slot id i of an int32 or int64 id array (absolute slots are below 2^31 either way).
template <bool ID64>
__device__ __forceinline__ int64_t load_id(const void* ids, int64_t i) {
    if constexpr (ID64) {
        return static_cast<const int64_t*>(ids)[i];
    } else {
        return static_cast<const int32_t*>(ids)[i];
    }
}

// Entry-order words the pair kernel reads per kind: the entry's sorted position, a walk bit where
// the entry starts its token's run with earlier valid K entries in an ordinary group, and a hot bit
// where it does so in a hot group (walked only when that group cannot be summed densely). 16-bit
// words for rows of up to 2^14 entries (the on-chip kernel), 32-bit words for longer rows.
template <typename InvT>
struct InvBits;
template <>
struct InvBits<uint16_t> {
    static constexpr uint32_t kPos = (1u << 14) - 1u, kHot = 1u << 14, kWalk = 1u << 15;
};
template <>
struct InvBits<uint32_t> {
    static constexpr uint32_t kPos = (1u << 17) - 1u, kHot = 1u << 30, kWalk = 1u << 31;
};

}  // namespace
}  // namespace sdm
