// Device-side constants and helpers shared by the Phase-1, DW and read-side kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdm {

// Payload word of an entry (page "sparse_delta_memory/cuda/phase1_cuda.py", p1_keys_zw_kernel and
// the sorted-row element comment of p1_scan_kernel): lane bits 0-7, Q bit 8, token bits 9-16,
// invalid bit 17; the sorted kind rows add the distance to the kind's first entry of the group
// (bits 18-29), LAST (bit 30) and FIRST (bit 31).
constexpr uint32_t kFirst = 0x80000000u;
constexpr uint32_t kLast = 0x40000000u;
constexpr uint32_t kInvalid = 0x20000u;
constexpr uint32_t kIsQ = 0x100u;
constexpr int kTokShift = 9;
constexpr uint32_t kEntryMask = 0x3FFFFu;
constexpr int kDistShift = 18;
constexpr uint32_t kDistMax = 4095u;
// Packed positions: sorted position bits 0-16, peers after bits 17-23, peers in group 24-30.
constexpr int kPosAfterShift = 17;
constexpr int kPosSizeShift = 24;
constexpr uint32_t kPosCountMax = 127u;
// Head-of-group flag kept in bit 31 of the pair records' payload word.
constexpr uint32_t kHead = 0x80000000u;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) { return __uint_as_float(h16 << 16); }

// float32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
// Branch-free (a select), so that callers can keep several conversions in one basic block.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? ((u >> 16) | 0x40u) : rounded;
}

// Element i of a value array: float32, or bfloat16 (bf set) widened exactly to float32.
__device__ __forceinline__ float load_val(const void* p, int64_t i, int bf) {
    if (bf) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

// The lanes of the wave whose digit (the db low bits of d, db < 32) equals this lane's: `below` of
// them in lower lanes, `cnt` in all (every lane of the wave active). One ballot per bit: with the
// lane's bit replicated over a word (sel), it keeps the ballot's lanes that agree with it,
// peers &= ~(ballot ^ sel) per 32-lane half (one 3-input bit operation each on gfx950).
__device__ __forceinline__ void digit_peers(uint32_t d, int db, uint32_t& below, uint32_t& cnt) {
    uint32_t plo = ~0u, phi = ~0u;
    for (int b = 0; b < db; ++b) {
        const uint32_t sel = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int32_t>(d), b, 1));
        const uint64_t m = __ballot(sel != 0u);
        plo &= ~(static_cast<uint32_t>(m) ^ sel);
        phi &= ~(static_cast<uint32_t>(m >> 32) ^ sel);
    }
    below = __builtin_amdgcn_mbcnt_hi(phi, __builtin_amdgcn_mbcnt_lo(plo, 0u));   // set bits under the lane
    cnt = static_cast<uint32_t>(__popc(plo) + __popc(phi));
}

// The compute dies (XCDs) of the device: a launch's workgroups are dealt to them in turn
// (workgroup b runs on XCD b % kXcds), and each has its own L2.
constexpr int kXcds = 8;

// Logical block of workgroup b among nb: consecutive logical blocks run on one XCD, so work laid
// out by logical block keeps neighbouring data (rows that several blocks read) in one L2. XCD x
// takes the logical blocks [x q + min(x, r), ...) of length q + (x < r), with q = nb / 8,
// r = nb % 8: a bijection of [0, nb).
__device__ __forceinline__ int xcd_block(int b, int nb) {
    const int x = b % kXcds, k = b / kXcds;
    const int q = nb / kXcds, r = nb % kXcds;
    return x * q + min(x, r) + k;
}

// Barrier for LDS hazards only: LDS operations complete, global stores may stay in flight.
__device__ __forceinline__ void lds_barrier() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace sdm
