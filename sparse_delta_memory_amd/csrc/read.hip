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
// per (chunk, 16 columns); the tokens are taken in blocks of 16: the A and QK rows of the block are
// staged in LDS, every thread forms its token's right-hand side from the earlier blocks' dv, 16
// threads (one per column) solve the block's unit triangle in order, then every thread adds its
// token's pred and read terms. Sums run in a fixed order: results are reproducible.
#include <hip/hip_ext.h>

#include "sdm_device.hpp"
#include "sdm_launch.hpp"

namespace sdm {
namespace {

constexpr int kGTeam = 16;          // lanes per token in the gather
constexpr int kGCols = 8;           // columns per lane
constexpr int kGTok = 256 / kGTeam; // tokens per gather block
constexpr int kGBatch = 8;          // entries whose rows are in flight together
constexpr int kSB = 16;             // tokens per substitution block and columns per solve block

struct ReadArgs {
    const void* bank;
    int64_t rows;
    const int32_t* k_idx;
    const int32_t* q_idx;
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

// sum_e w[e] M0[idx[e]] over n entries, 8 columns of one token; entries kGBatch at a time.
template <bool BF16>
__device__ __forceinline__ void gather_sum(const ReadArgs& a, const int32_t* idx, const float* w, int n, int col0,
                                           float (&acc)[kGCols]) {
    for (int e0 = 0; e0 < n; e0 += kGBatch) {
        int32_t s[kGBatch];
        float ws[kGBatch];
#pragma unroll
        for (int b = 0; b < kGBatch; ++b) {
            const int e = min(e0 + b, n - 1);
            s[b] = idx[e];
            ws[b] = e0 + b < n ? w[e] : 0.0f;
        }
        uint4 raw[kGBatch][BF16 ? 1 : 2];
#pragma unroll
        for (int b = 0; b < kGBatch; ++b) {
            // A slot outside the bank contributes nothing (its row is not read).
            const bool ok = s[b] >= 0 && static_cast<int64_t>(s[b]) < a.rows;
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

template <bool BF16>
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
        gather_sum<BF16>(a, a.k_idx + ko, a.k_eff + ko, a.W, col0, pk);
        gather_sum<BF16>(a, a.q_idx + qo, a.q_w + qo, a.R, col0, pq);
    }
    float4* op = reinterpret_cast<float4*>(a.pred + row * a.hd + col0);
    float4* oq = reinterpret_cast<float4*>(a.read + row * a.hd + col0);
    op[0] = make_float4(pk[0], pk[1], pk[2], pk[3]);
    op[1] = make_float4(pk[4], pk[5], pk[6], pk[7]);
    oq[0] = make_float4(pq[0], pq[1], pq[2], pq[3]);
    oq[1] = make_float4(pq[4], pq[5], pq[6], pq[7]);
}

__global__ void __launch_bounds__(256) read_solve_kernel(ReadArgs a) {
    __shared__ float sdv[256][kSB];        // dv of every token so far, this block's 16 columns
    __shared__ float sA[kSB][256 + 1];      // A rows of the current token block (columns 0 .. b0+15)
    __shared__ float sQ[kSB][256 + 1];      // QK rows of the current token block
    __shared__ float srhs[kSB][kSB];        // right-hand sides of the current token block
    const int col_blocks = (a.hd + kSB - 1) / kSB;
    const int p = blockIdx.x / col_blocks;
    const int d = static_cast<int>(threadIdx.x) % kSB;       // column within the block
    const int tl = static_cast<int>(threadIdx.x) / kSB;      // token within a token block
    const int col = (blockIdx.x % col_blocks) * kSB + d;
    const bool col_ok = col < a.hd;
    const int64_t c = a.chunk0 + p;
    const int C = a.C;
    const int tv = c >= a.first_partial ? a.valid_last : C;
    const float* A = a.a + c * C * C;
    const float* QK = a.qk + c * C * C;
    const int64_t rbase = a.row0 + static_cast<int64_t>(p) * C;
    for (int b0 = 0; b0 < C; b0 += kSB) {
        const int t = b0 + tl;
        const bool valid = t < tv && col_ok;
        // Stage the block's A and QK rows, columns 0 .. b0 + 15.
        const int wcols = b0 + kSB;
        for (int i = threadIdx.x; i < kSB * wcols; i += 256) {
            const int r = i / wcols, j = i - r * wcols;
            const bool in = b0 + r < C && j < C;   // the block's rows; columns past C are zero
            sA[r][j] = in ? A[static_cast<int64_t>(b0 + r) * C + j] : 0.0f;
            sQ[r][j] = in ? QK[static_cast<int64_t>(b0 + r) * C + j] : 0.0f;
        }
        __syncthreads();
        // Right-hand side: v - p0 - (terms of earlier blocks).
        float far = 0.0f;
        for (int j = 0; j < b0; ++j) far = fmaf(sA[tl][j], sdv[j][d], far);
        const float p0 = valid ? a.pred[(rbase + t) * a.hd + col] : 0.0f;
        const float vv = valid ? a.v[(rbase + t) * a.hd + col] : 0.0f;
        srhs[tl][d] = valid ? (vv - p0) - far : 0.0f;
        __syncthreads();
        // The block's unit triangle, in token order, one thread per column.
        if (tl == 0) {
            float x[kSB];
#pragma unroll
            for (int i = 0; i < kSB; ++i) {
                float s = srhs[i][d];
#pragma unroll
                for (int k = 0; k < i; ++k) s = fmaf(-sA[i][b0 + k], x[k], s);
                const bool ok = b0 + i < tv && col_ok;
                x[i] = ok ? a.beta[c * C + b0 + i] * s : 0.0f;
                if (b0 + i < C) sdv[b0 + i][d] = x[i];
            }
        }
        __syncthreads();
        // pred and read of the block's tokens.
        if (t < C && col_ok) {
            float near = 0.0f;
            for (int j = b0; j < t; ++j) near = fmaf(sA[tl][j], sdv[j][d], near);
            float rd = 0.0f;
            for (int j = 0; j <= t; ++j) rd = fmaf(sQ[tl][j], sdv[j][d], rd);
            const float q0 = valid ? a.read[(rbase + t) * a.hd + col] : 0.0f;
            const int64_t o = (rbase + t) * a.hd + col;
            a.dv[o] = sdv[t][d];
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
    const void* g = io->bank_dtype == SDM_BF16 ? reinterpret_cast<const void*>(&read_gather_kernel<true>)
                                               : reinterpret_cast<const void*>(&read_gather_kernel<false>);
    hipError_t e = hipExtLaunchKernel(g, dim3(static_cast<unsigned>(a.P * tok_blocks * col_blocks)), dim3(256), kargs, 0,
                                      st, ev[0], ev[1], 0);
    if (e != hipSuccess) return e;
    const int solve_blocks = a.P * ((a.hd + kSB - 1) / kSB);
    return hipExtLaunchKernel(reinterpret_cast<const void*>(&read_solve_kernel), dim3(static_cast<unsigned>(solve_blocks)),
                              dim3(256), kargs, 0, st, ev[2], ev[3], 0);
}

}  // namespace sdm
