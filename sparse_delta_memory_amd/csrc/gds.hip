// GDS on gfx950: the backward of the read gather q0[t] = sum_r q_w[t, r] M0[q_idx[t, r]] for the
// chunks of one step (page "sparse_delta_memory/cuda/mover_da2_cuda.py": the GDS part of the module
// docstring and the comment of its scatter role).
//
// gds_dots_kernel: d_q_w[t, r] = <gr[t], M0[q_idx[t, r]]>, token order, one wave per token: each
// lane takes 4 columns of every 256, and a wave reduction gives each dot (no atomics).
// gds_scatter_kernel: the gradient rows in sorted order, one wave per position of the Q-only rows:
// at a valid group FIRST the wave walks the group's members in sorted order, acc = fma(q_w, gr[t],
// acc) from +0, and at LAST adds acc to grad[slot] with one read-modify-write (the wave is that
// row's only writer in the launch, so the result is deterministic).

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
    int64_t rows, chunk0, row0;
    int P, C, R, hd, first_partial, valid_last, id64, vbf, bank_bf16, grad_bf16;
};

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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

__global__ void __launch_bounds__(kGdsThreads) gds_dots_kernel(GdsArgs a) {
    const int wv = static_cast<int>(threadIdx.x) / kWave;
    const int lane = static_cast<int>(lane_id());
    const int64_t tok = static_cast<int64_t>(blockIdx.x) * kGdsWaves + wv;   // (p, t) of the step
    if (tok >= static_cast<int64_t>(a.P) * a.C) return;
    const int p = static_cast<int>(tok / a.C), t = static_cast<int>(tok % a.C);
    const int64_t c = a.chunk0 + p;
    const int tv = c >= a.first_partial ? a.valid_last : a.C;
    const int64_t eo = (c * a.C + t) * a.R;   // the token's first Q entry
    if (t >= tv) {   // masked: no reads, dots 0
        for (int r = lane; r < a.R; r += kWave) a.d_q_w[eo + r] = 0.0f;
        return;
    }
    const int64_t grow = a.row0 + static_cast<int64_t>(p) * a.C + t;
    for (int r = 0; r < a.R; ++r) {
        const int64_t s = gds_id(a, eo + r);
        float acc = 0.0f;
        if (s >= 0 && s < a.rows) {   // (a slot outside the bank contributes nothing)
            for (int col = 4 * lane; col < a.hd; col += 4 * kWave) {
                const float4 g = load4(a.gr, 0, grow, a.hd, col);
                const float4 m = load4(a.bank, a.bank_bf16, s, a.hd, col);
                acc = fmaf(g.w, m.w, fmaf(g.z, m.z, fmaf(g.y, m.y, fmaf(g.x, m.x, acc))));
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) a.d_q_w[eo + r] = acc;
    }
}

__global__ void __launch_bounds__(kGdsThreads) gds_scatter_kernel(GdsArgs a) {
    const int wv = static_cast<int>(threadIdx.x) / kWave;
    const int lane = static_cast<int>(lane_id());
    const int n = a.C * a.R;
    const int64_t pos = static_cast<int64_t>(blockIdx.x) * kGdsWaves + wv;   // p * C * R + j
    if (pos >= static_cast<int64_t>(a.P) * n) return;
    const int p = static_cast<int>(pos / n), j = static_cast<int>(pos % n);
    const int64_t c = a.chunk0 + p;
    const uint32_t* row = a.spay_q + c * n;
    const uint32_t e0 = row[j];
    if (!(e0 & kFirst) || (e0 & kInvalid)) return;   // a valid group starts here
    // The group's slot (every member reads it) and its bounds.
    const int64_t qbase = c * n;   // entry-order Q index of (t, lane) is t * R + lane
    auto entry = [&](uint32_t el) { return static_cast<int64_t>((el >> kTokShift) & 0xFFu) * a.R + (el & 0xFFu); };
    const int64_t slot = gds_id(a, qbase + entry(e0));
    if (slot < 0 || slot >= a.rows) return;
    const int64_t grow0 = a.row0 + static_cast<int64_t>(p) * a.C;
    for (int col = 4 * lane; col < a.hd; col += 4 * kWave) {
        float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int m = j; m < n; ++m) {   // the members in sorted order, up to LAST
            const uint32_t el = row[m];
            const int64_t ei = entry(el);
            const float w = load_val(a.q_w, qbase + ei, a.vbf);
            const float4 g = load4(a.gr, 0, grow0 + ((el >> kTokShift) & 0xFFu), a.hd, col);
            acc.x = fmaf(w, g.x, acc.x);
            acc.y = fmaf(w, g.y, acc.y);
            acc.z = fmaf(w, g.z, acc.z);
            acc.w = fmaf(w, g.w, acc.w);
            if (el & kLast) break;
        }
        // One read-modify-write of the lane's columns (this wave is the row's only writer).
        if (a.grad_bf16) {
            uint2* gp = reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.grad) + slot * a.hd + col);
            const uint2 o = *gp;
            const float x = bf16_bits_to_f32(o.x & 0xFFFFu) + acc.x, y = bf16_bits_to_f32(o.x >> 16) + acc.y;
            const float z = bf16_bits_to_f32(o.y & 0xFFFFu) + acc.z, u = bf16_bits_to_f32(o.y >> 16) + acc.w;
            *gp = make_uint2(f32_to_bf16_rne(x) | f32_to_bf16_rne(y) << 16, f32_to_bf16_rne(z) | f32_to_bf16_rne(u) << 16);
        } else {
            float4* gp = reinterpret_cast<float4*>(static_cast<float*>(a.grad) + slot * a.hd + col);
            const float4 o = *gp;
            *gp = make_float4(o.x + acc.x, o.y + acc.y, o.z + acc.z, o.w + acc.w);
        }
    }
}

}  // namespace

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
    const int64_t toks = static_cast<int64_t>(io->P) * io->C;
    const int64_t poss = toks * io->R;
    void* kargs[] = {&a};
    hipError_t e = hipSuccess;
    if (io->d_q_w != nullptr) {
        e = hipLaunchKernel(reinterpret_cast<const void*>(&gds_dots_kernel),
                            dim3(static_cast<unsigned>((toks + kGdsWaves - 1) / kGdsWaves)), dim3(kGdsThreads), kargs, 0, st);
        if (e != hipSuccess) return e;
    }
    if (io->grad != nullptr) {
        e = hipLaunchKernel(reinterpret_cast<const void*>(&gds_scatter_kernel),
                            dim3(static_cast<unsigned>((poss + kGdsWaves - 1) / kGdsWaves)), dim3(kGdsThreads), kargs, 0, st);
    }
    return e;
}

}  // namespace sdm
