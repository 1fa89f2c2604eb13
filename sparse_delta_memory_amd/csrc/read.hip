// Forward read side of a DW step on gfx950: the token gather of the pre-step rows, the delta-rule
// forward substitution that gives the step's token rows, and the reads.
//
// Per chunk (definitions: page "sparse_delta_memory/cuda/phase1_cuda.py", module docstring, for
// k_eff, q_w, A and QK; the delta rule dv = beta (v - prediction) is read from the write scale
// -beta k exp(log_k) of the backward records, same page, p1_scan_kernel, and page
// "sparse_delta_memory/cuda/pa_dc_cuda.py", module docstring):
//   p0[t] = sum_e k_eff[t,e] M0[k_idx[t,e]],  q0[t] = sum_r q_w[t,r] M0[q_idx[t,r]]
//   dv[t] = beta[t] (v[t] - p0[t] - sum_{j<t} A[t,j] dv[j])
//   pred[t] = p0[t] + sum_{j<t} A[t,j] dv[j],  read[t] = q0[t] + sum_{j<=t} QK[t,j] dv[j]
//
// Two kernels per step. read_gather_kernel: a team of 16 lanes per token, 8 columns per lane (16-byte
// bf16 or two 16-byte float32 loads per row), entries taken 8 at a time with every row load in flight
// before the first is used; p0 and q0 go to the pred and read outputs. read_solve_kernel: one block
// per (chunk, 4 columns). It first inverts every 16 x 16 diagonal block of I + diag(beta) A (one
// column of one block per lane, by substitution), then takes the tokens in blocks of 16: the
// block's A and QK rows (loaded two blocks ahead) go to LDS; four lanes share each (token, column)
// dot, every fourth term each, added by a fixed butterfly; the scaled right-hand side times the
// block inverse's row gives dv, then the pred and read terms. Sums run in a fixed order: results
// are reproducible.
#include <hip/hip_ext.h>

#include "sdm_device.hpp"
#include "sdm_launch.hpp"

namespace sdm {
namespace {

constexpr int kGTeam = 16;          // lanes per token in the gather
constexpr int kGCols = 8;           // columns per lane
constexpr int kGTok = 256 / kGTeam; // tokens per gather block
constexpr int kGBatch = 8;          // entries whose rows are in flight together
constexpr int kSB = 16;             // tokens per substitution block

struct ReadArgs {
    const void* bank;
    int64_t rows;
    const void* k_idx;   // int32 or int64 ids
    const void* q_idx;
    const float* k_eff;
    const float* q_w;
    const float* a;
    const float* qk;
    const float* v;
    const float* beta;
    float* dv;
    float* pred;
    float* read;
    int64_t chunk0;      // ti * P
    int64_t row0;        // ti * step_rows: row of (p, t) is row0 + p * C + t
    int P, C, W, R, hd, first_partial, valid_last;
};

template <bool BF16>
__device__ __forceinline__ void load_row8(const void* bank, int64_t slot, int hd, int col0, uint4 (&raw)[BF16 ? 1 : 2]) {
    const unsigned char* p = static_cast<const unsigned char*>(bank) + (slot * hd + col0) * (BF16 ? 2 : 4);
    raw[0] = *reinterpret_cast<const uint4*>(p);
    if constexpr (!BF16) raw[1] = *reinterpret_cast<const uint4*>(p + 16);
}

template <bool BF16>
__device__ __forceinline__ void widen_row8(const uint4 (&raw)[BF16 ? 1 : 2], float (&x)[kGCols]) {
    if constexpr (BF16) {
        const uint32_t w[4] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            x[2 * h] = bf16_bits_to_f32(w[h] & 0xFFFFu);
            x[2 * h + 1] = bf16_bits_to_f32(w[h] >> 16);
        }
    } else {
        const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
        for (int h = 0; h < 8; ++h) x[h] = __uint_as_float(w[h]);
    }
}

// sum_e w[e] M0[idx[e]] over n entries (idx: int32, or int64 when ID64), 8 columns of one token;
// entries kGBatch at a time.
template <bool BF16, bool ID64>
__device__ __forceinline__ void gather_sum(const ReadArgs& a, const void* idx, const float* w, int n, int col0,
                                           float (&acc)[kGCols]) {
    for (int e0 = 0; e0 < n; e0 += kGBatch) {
        int64_t s[kGBatch];
        float ws[kGBatch];
#pragma unroll
        for (int b = 0; b < kGBatch; ++b) {
            const int e = min(e0 + b, n - 1);
            if constexpr (ID64) {
                s[b] = static_cast<const int64_t*>(idx)[e];
            } else {
                s[b] = static_cast<const int32_t*>(idx)[e];
            }
            ws[b] = e0 + b < n ? w[e] : 0.0f;
        }
        uint4 raw[kGBatch][BF16 ? 1 : 2];
#pragma unroll
        for (int b = 0; b < kGBatch; ++b) {
            // A slot outside the bank contributes nothing (its row is not read).
            const bool ok = s[b] >= 0 && s[b] < a.rows;
            load_row8<BF16>(a.bank, ok ? s[b] : 0, a.hd, col0, raw[b]);
            if (!ok) ws[b] = 0.0f;
        }
#pragma unroll
        for (int b = 0; b < kGBatch; ++b) {
            float x[kGCols];
            widen_row8<BF16>(raw[b], x);
#pragma unroll
            for (int q = 0; q < kGCols; ++q) acc[q] = fmaf(ws[b], x[q], acc[q]);
        }
    }
}

template <bool BF16, bool ID64>
__global__ void __launch_bounds__(256) read_gather_kernel(ReadArgs a) {
    const int tok_blocks = (a.C + kGTok - 1) / kGTok;
    const int col_blocks = (a.hd + kGTeam * kGCols - 1) / (kGTeam * kGCols);
    const int b = blockIdx.x;
    const int p = b / (tok_blocks * col_blocks);
    const int rem = b - p * tok_blocks * col_blocks;
    const int t = (rem / col_blocks) * kGTok + static_cast<int>(threadIdx.x) / kGTeam;
    const int col0 = ((rem % col_blocks) * kGTeam + static_cast<int>(threadIdx.x) % kGTeam) * kGCols;
    if (t >= a.C || col0 >= a.hd) return;
    const int64_t c = a.chunk0 + p;
    const int tv = c >= a.first_partial ? a.valid_last : a.C;
    const int64_t row = a.row0 + static_cast<int64_t>(p) * a.C + t;
    float pk[kGCols], pq[kGCols];
#pragma unroll
    for (int q = 0; q < kGCols; ++q) pk[q] = pq[q] = 0.0f;
    if (t < tv) {
        const int64_t ko = (c * a.C + t) * a.W, qo = (c * a.C + t) * a.R;
        const int es = ID64 ? 8 : 4;
        gather_sum<BF16, ID64>(a, static_cast<const char*>(a.k_idx) + ko * es, a.k_eff + ko, a.W, col0, pk);
        gather_sum<BF16, ID64>(a, static_cast<const char*>(a.q_idx) + qo * es, a.q_w + qo, a.R, col0, pq);
    }
    float4* op = reinterpret_cast<float4*>(a.pred + row * a.hd + col0);
    float4* oq = reinterpret_cast<float4*>(a.read + row * a.hd + col0);
    op[0] = make_float4(pk[0], pk[1], pk[2], pk[3]);
    op[1] = make_float4(pk[4], pk[5], pk[6], pk[7]);
    oq[0] = make_float4(pq[0], pq[1], pq[2], pq[3]);
    oq[1] = make_float4(pq[4], pq[5], pq[6], pq[7]);
}

constexpr int kSC = 4;   // columns per substitution block
constexpr int kKS = 4;   // lanes sharing one dot (each takes every kKS-th term)

// Part of sum_{j0 <= j < j1} row[j] * col[j * kSC]: the terms with j = j0 + ks (mod kKS).
__device__ __forceinline__ float lds_dot_part(const float* row, const float* col, int j0, int j1, int ks) {
    float s = 0.0f;
    for (int j = j0 + ks; j < j1; j += kKS) s = fmaf(row[j], col[j * kSC], s);
    return s;
}

// The kKS parts of a dot (lanes 4 and 8 apart) added by a butterfly: every lane gets the same bits
// ((p0 + p1) + (p2 + p3), float addition being commutative).
__device__ __forceinline__ float dot_total(float s) {
    s += __shfl_xor(s, kSC, kWave);
    s += __shfl_xor(s, kSC * 2, kWave);
    return s;
}

// Dynamic LDS of the substitution kernel (floats): dv of every token (C x kSC), the current block's
// A and QK rows (16 x (C + 1) each, padded against bank conflicts), the inverses of the diagonal
// blocks (C x 16) and the block's scaled right-hand sides (16 x kSC).
size_t solve_lds_bytes(int C) {
    return sizeof(float) * (static_cast<size_t>(C) * kSC + static_cast<size_t>(kSB) * (C + 1) * 2 +
                            static_cast<size_t>(C) * kSB + kSB * kSC);
}

__global__ void __launch_bounds__(256) read_solve_kernel(ReadArgs a) {
    extern __shared__ float lds[];
    const int C = a.C;
    const int ld = C + 1;
    float* sdv = lds;                   // [C][kSC]
    float* sA = sdv + C * kSC;          // [16][ld]
    float* sQ = sA + kSB * ld;          // [16][ld]
    float* sT = sQ + kSB * ld;          // [C][16]: row t holds row (t mod 16) of its block's inverse
    float* srhs = sT + C * kSB;         // [16][kSC]
    const int tid = static_cast<int>(threadIdx.x);
    // Lanes: token in block tl (tid / 16), dot part ks, column d (tid = tl * 16 + ks * kSC + d).
    const int tl = tid / kSB;
    const int ks = (tid / kSC) % kKS;
    const int d = tid % kSC;
    // Staging and inverse lanes: row / block sr (tid / 16), lane sl (tid % 16).
    const int sr = tid / kSB, sl = tid % kSB;
    // Block b is (chunk b mod P, column group b / P): consecutive blocks go round the XCDs (8, each
    // with its own L2), so a chunk's column groups share one XCD when P is a multiple of 8 (and
    // 8 / gcd(P, 8) otherwise) and its A / QK rows are fetched from HBM once per XCD, not per block.
    const int p = static_cast<int>(blockIdx.x) % a.P;
    const int col = (static_cast<int>(blockIdx.x) / a.P) * kSC + d;
    const bool col_ok = col < a.hd;
    const int64_t c = a.chunk0 + p;
    const int tv = c >= a.first_partial ? a.valid_last : C;
    const float* A = a.a + c * C * C;
    const float* QK = a.qk + c * C * C;
    const float* beta = a.beta + c * C;
    const int64_t rbase = a.row0 + static_cast<int64_t>(p) * C;
    const int nblk = (C + kSB - 1) / kSB;

    // Inverse of every diagonal block T_b = I + diag(beta_b) A_bb (unit lower triangular): lane
    // (block sr, column sl) solves T_b x = e_sl by substitution; masked tokens have beta taken as 0.
    if (sr < nblk) {
        const int t0 = sr * kSB;
        float al[kSB][kSB];
        float bt[kSB];
#pragma unroll
        for (int i = 0; i < kSB; ++i) {
            const bool ok = t0 + i < tv;
            bt[i] = ok ? beta[t0 + i] : 0.0f;
#pragma unroll
            for (int k = 0; k < i; ++k) al[i][k] = ok ? A[static_cast<int64_t>(t0 + i) * C + t0 + k] : 0.0f;
        }
        float x[kSB];
#pragma unroll
        for (int i = 0; i < kSB; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < i; ++k) s = fmaf(al[i][k], x[k], s);
            x[i] = (i == sl ? 1.0f : 0.0f) - bt[i] * s;
            if (t0 + i < C) sT[(t0 + i) * kSB + sl] = x[i];
        }
    }

    // Staged rows of token block b (row sr, columns sl + 16u) and this lane's token values, loaded
    // two blocks ahead.
    float stA[kSB], stQ[kSB], stA2[kSB], stQ2[kSB];
    float nx_p0 = 0.0f, nx_v = 0.0f, nx_q0 = 0.0f, nx_b = 0.0f;
    float nx2_p0 = 0.0f, nx2_v = 0.0f, nx2_q0 = 0.0f, nx2_b = 0.0f;
    // Loads of block b into the second set (two blocks ahead of their use).
    auto prefetch = [&](int b) {
        const int b0 = b * kSB;
        const int tr = b0 + sr;
        const int groups = b + 1;                   // column groups of 16 up to the block's diagonal
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            const int j = sl + kSB * u;
            const bool in = tr < C && u < groups && j < C;
            stA2[u] = in ? A[static_cast<int64_t>(tr) * C + j] : 0.0f;
            stQ2[u] = in ? QK[static_cast<int64_t>(tr) * C + j] : 0.0f;
        }
        const int t = b0 + tl;
        const bool valid = t < tv && col_ok;
        nx2_p0 = valid ? a.pred[(rbase + t) * a.hd + col] : 0.0f;
        nx2_v = valid ? a.v[(rbase + t) * a.hd + col] : 0.0f;
        nx2_q0 = valid ? a.read[(rbase + t) * a.hd + col] : 0.0f;
        nx2_b = valid ? beta[t] : 0.0f;
    };
    auto shift = [&]() {   // the second set becomes the next block's
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            stA[u] = stA2[u];
            stQ[u] = stQ2[u];
        }
        nx_p0 = nx2_p0;
        nx_v = nx2_v;
        nx_q0 = nx2_q0;
        nx_b = nx2_b;
    };
    prefetch(0);
    shift();
    if (nblk > 1) prefetch(1);
    for (int b = 0; b < nblk; ++b) {
        const int b0 = b * kSB;
        const int t = b0 + tl;
        const bool valid = t < tv && col_ok;
        const int groups = b + 1;
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            if (u < groups && sl + kSB * u < C) {
                sA[sr * ld + sl + kSB * u] = stA[u];
                sQ[sr * ld + sl + kSB * u] = stQ[u];
            }
        }
        const float p0 = nx_p0, vv = nx_v, q0 = nx_q0, bt = nx_b;
        if (b + 1 < nblk) shift();
        if (b + 2 < nblk) prefetch(b + 2);
        __syncthreads();   // the block's rows (and, first time, the inverses) are in LDS
        // Scaled right-hand side: beta (v - p0 - terms of the earlier blocks).
        const float far = dot_total(lds_dot_part(sA + tl * ld, sdv + d, 0, b0, ks));
        if (ks == 0) srhs[tl * kSC + d] = valid ? bt * ((vv - p0) - far) : 0.0f;
        __syncthreads();
        // dv of the block: the inverse's row times the scaled right-hand sides.
        float x = 0.0f;
        if (t < C) {
            for (int k = 0; k <= tl; ++k) x = fmaf(sT[t * kSB + k], srhs[k * kSC + d], x);
            if (ks == 0) sdv[t * kSC + d] = valid ? x : 0.0f;
        }
        __syncthreads();
        // pred and read of the block's tokens.
        const int tt = t < C ? t : 0;
        const float near = dot_total(lds_dot_part(sA + tl * ld, sdv + d, b0, t < C ? t : b0, ks));
        const float rd = dot_total(lds_dot_part(sQ + tl * ld, sdv + d, 0, t < C ? tt + 1 : 0, ks));
        if (ks == 0 && t < C && col_ok) {
            const int64_t o = (rbase + t) * a.hd + col;
            a.dv[o] = valid ? x : 0.0f;
            a.pred[o] = valid ? (p0 + far) + near : 0.0f;
            a.read[o] = valid ? q0 + rd : 0.0f;
        }
        __syncthreads();   // the staged rows are replaced next
    }
}

}  // namespace

hipError_t read_launch(const ReadLaunch& L, hipStream_t st) {
    const sdm_read_io* io = L.io;
    ReadArgs a;
    a.bank = io->bank;
    a.rows = io->rows;
    a.k_idx = io->k_idx;
    a.q_idx = io->q_idx;
    a.k_eff = io->k_eff;
    a.q_w = io->q_w;
    a.a = io->a;
    a.qk = io->qk;
    a.v = io->v;
    a.beta = io->beta;
    a.dv = io->dv;
    a.pred = io->pred;
    a.read = io->read;
    a.chunk0 = L.ti * io->P;
    a.row0 = L.ti * io->step_rows;
    a.P = io->P;
    a.C = io->C;
    a.W = io->W;
    a.R = io->R;
    a.hd = io->hd;
    a.first_partial = io->first_partial;
    a.valid_last = io->valid_last;
    const int tok_blocks = (a.C + kGTok - 1) / kGTok;
    const int col_blocks = (a.hd + kGTeam * kGCols - 1) / (kGTeam * kGCols);
    const hipEvent_t ev[4] = {io->events ? io->events[0] : nullptr, io->events ? io->events[1] : nullptr,
                              io->events ? io->events[2] : nullptr, io->events ? io->events[3] : nullptr};
    void* kargs[] = {&a};
    const bool id64 = io->idx_bytes == 8;
    const void* g = io->bank_dtype == SDM_BF16
                        ? (id64 ? reinterpret_cast<const void*>(&read_gather_kernel<true, true>)
                                : reinterpret_cast<const void*>(&read_gather_kernel<true, false>))
                        : (id64 ? reinterpret_cast<const void*>(&read_gather_kernel<false, true>)
                                : reinterpret_cast<const void*>(&read_gather_kernel<false, false>));
    hipError_t e = hipExtLaunchKernel(g, dim3(static_cast<unsigned>(a.P * tok_blocks * col_blocks)), dim3(256), kargs, 0,
                                      st, ev[0], ev[1], 0);
    if (e != hipSuccess) return e;
    const int solve_blocks = a.P * ((a.hd + kSC - 1) / kSC);
    const size_t lds = solve_lds_bytes(a.C);
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&read_solve_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
    if (e != hipSuccess) return e;
    return hipExtLaunchKernel(reinterpret_cast<const void*>(&read_solve_kernel), dim3(static_cast<unsigned>(solve_blocks)),
                              dim3(256), kargs, lds, st, ev[2], ev[3], 0);
}

}  // namespace sdm
