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
// of four waves per (chunk, 16 columns). It first inverts every 16 x 16 diagonal block of
// I + diag(beta) A (one column of one block per lane, by substitution); then it takes the tokens in
// blocks of 16, the block's A rows staged in LDS (loaded one block ahead): the earlier blocks'
// terms A[block, :b0] dv are formed with 16 x 16 x 4 float32 matrix (MFMA) steps, shared out among
// the four waves, and wave 0 adds the four shares, forms the block's dv as its inverse times the
// scaled right-hand sides and the block's own A terms for pred. Only that chain is sequential: the
// reads QK[block, :b0+16] dv follow for every block at once, once all of dv is in LDS. Sums run in
// a fixed order: results are reproducible.
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
    const void* k_eff;   // float32, or bfloat16 when vbf
    const void* q_w;
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
    int vbf;             // 1: k_eff / q_w are bfloat16
};

// TAIL (hd not a multiple of 8): rows are only element-aligned; the lane's first nv (1..8) columns
// are read element by element and the rest are zero.
template <bool BF16, bool TAIL>
__device__ __forceinline__ void load_row8(const void* bank, int64_t slot, int hd, int col0, int nv,
                                          uint4 (&raw)[BF16 ? 1 : 2]) {
    const unsigned char* p = static_cast<const unsigned char*>(bank) + (slot * hd + col0) * (BF16 ? 2 : 4);
    if constexpr (TAIL) {
        uint32_t w[BF16 ? 4 : 8];
        if constexpr (BF16) {
            const uint16_t* q = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
            for (int e = 0; e < kGCols; e += 2) {
                const uint32_t lo = e < nv ? q[e] : 0u;
                const uint32_t hi = e + 1 < nv ? q[e + 1] : 0u;
                w[e / 2] = lo | hi << 16;
            }
            raw[0] = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
            for (int e = 0; e < kGCols; ++e) w[e] = e < nv ? q[e] : 0u;
            raw[0] = make_uint4(w[0], w[1], w[2], w[3]);
            raw[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
    } else {
        raw[0] = *reinterpret_cast<const uint4*>(p);
        if constexpr (!BF16) raw[1] = *reinterpret_cast<const uint4*>(p + 16);
    }
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
template <bool BF16, bool ID64, bool TAIL>
__device__ __forceinline__ void gather_sum(const ReadArgs& a, const void* idx, const void* w, int n, int col0, int nv,
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
            ws[b] = e0 + b < n ? load_val(w, e, a.vbf) : 0.0f;
        }
        uint4 raw[kGBatch][BF16 ? 1 : 2];
#pragma unroll
        for (int b = 0; b < kGBatch; ++b) {
            // A slot outside the bank contributes nothing (its row is not read).
            const bool ok = s[b] >= 0 && s[b] < a.rows;
            load_row8<BF16, TAIL>(a.bank, ok ? s[b] : 0, a.hd, col0, nv, raw[b]);
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

template <bool BF16, bool ID64, bool TAIL>
__global__ void __launch_bounds__(256) read_gather_kernel(ReadArgs a) {
    const int tok_blocks = (a.C + kGTok - 1) / kGTok;
    const int col_blocks = (a.hd + kGTeam * kGCols - 1) / (kGTeam * kGCols);
    const int b = blockIdx.x;
    const int p = b / (tok_blocks * col_blocks);
    const int rem = b - p * tok_blocks * col_blocks;
    const int t = (rem / col_blocks) * kGTok + static_cast<int>(threadIdx.x) / kGTeam;
    const int col0 = ((rem % col_blocks) * kGTeam + static_cast<int>(threadIdx.x) % kGTeam) * kGCols;
    if (t >= a.C || col0 >= a.hd) return;
    const int nv = TAIL ? min(kGCols, a.hd - col0) : kGCols;   // the lane's columns
    const int64_t c = a.chunk0 + p;
    const int tv = c >= a.first_partial ? a.valid_last : a.C;
    const int64_t row = a.row0 + static_cast<int64_t>(p) * a.C + t;
    float pk[kGCols], pq[kGCols];
#pragma unroll
    for (int q = 0; q < kGCols; ++q) pk[q] = pq[q] = 0.0f;
    if (t < tv) {
        const int64_t ko = (c * a.C + t) * a.W, qo = (c * a.C + t) * a.R;
        const int es = ID64 ? 8 : 4;
        const int vs = a.vbf ? 2 : 4;   // bytes per weight
        gather_sum<BF16, ID64, TAIL>(a, static_cast<const char*>(a.k_idx) + ko * es,
                                     static_cast<const char*>(a.k_eff) + ko * vs, a.W, col0, nv, pk);
        gather_sum<BF16, ID64, TAIL>(a, static_cast<const char*>(a.q_idx) + qo * es,
                                     static_cast<const char*>(a.q_w) + qo * vs, a.R, col0, nv, pq);
    }
    if constexpr (TAIL) {
#pragma unroll
        for (int q = 0; q < kGCols; ++q) {
            if (q < nv) {
                a.pred[row * a.hd + col0 + q] = pk[q];
                a.read[row * a.hd + col0 + q] = pq[q];
            }
        }
    } else {
        float4* op = reinterpret_cast<float4*>(a.pred + row * a.hd + col0);
        float4* oq = reinterpret_cast<float4*>(a.read + row * a.hd + col0);
        op[0] = make_float4(pk[0], pk[1], pk[2], pk[3]);
        op[1] = make_float4(pk[4], pk[5], pk[6], pk[7]);
        oq[0] = make_float4(pq[0], pq[1], pq[2], pq[3]);
        oq[1] = make_float4(pq[4], pq[5], pq[6], pq[7]);
    }
}

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMW = 4;    // waves per substitution block, all on the block's 16 columns
constexpr int kTLd = 20;  // row stride (floats) of the inverse, dv and partial tiles in LDS: the four
                          // lane groups of a wave (rows 4 apart) then read 64 distinct banks

// One 16 x 16 x 4 float32 matrix step: lane l gives A[l % 16][k] and B[k][l % 16] for the k its
// lane group (l / 16) stands for; D row 4 (l / 16) + r, column l % 16 is register r of lane l.
__device__ __forceinline__ floatx4 mfma4(float av, float bv, floatx4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
}

// Row stride of the staged A panels: every column a token block reaches (C rounded up to 16) plus
// 4, so that rows are 16-byte aligned and start 4 banks apart.
__host__ __device__ inline int panel_ld(int C) { return (C + kSB - 1) / kSB * kSB + 4; }

constexpr int kPanels = 3;   // A panels in LDS: block b is read while block b + 1 is written

// Dynamic LDS of the substitution kernel (floats): the inverses of the diagonal blocks and dv of
// every token for the block's 16 columns (rows x kTLd each, rows = C rounded up to 16), a ring of
// kPanels A panels (a token block's rows, 16 x panel_ld), and one 16 x 16 partial tile per wave.
size_t solve_lds_bytes(int C) {
    const size_t rows = static_cast<size_t>((C + kSB - 1) / kSB) * kSB;
    return sizeof(float) * (2 * rows * kTLd + kPanels * static_cast<size_t>(kSB) * panel_ld(C) + kMW * kSB * kTLd);
}

// The terms of earlier token block j: panel columns [16 j, 16 j + 16) times dv rows of block j, added
// to acc (lane group g takes k = 16 j + 4 g + s).
__device__ __forceinline__ floatx4 block_times_dv(const float* panel, int ld, int j, const float* sdv, int g, int m,
                                                  floatx4 acc) {
    const floatx4 av = *reinterpret_cast<const floatx4*>(panel + m * ld + j * kSB + 4 * g);   // 16-byte aligned
    const float* dcol = sdv + (j * kSB + 4 * g) * kTLd + m;
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma4(av[s], dcol[s * kTLd], acc);
    return acc;
}

// Block (chunk p, 16 columns), four waves. The substitution runs over the token blocks in order; per
// block the earlier blocks' terms A[block, :b0] dv are shared out among the waves (wave w takes the
// earlier blocks j = w mod 4, in order) and summed in wave order by wave 0, which then solves the
// block with its inverted diagonal block and writes dv and pred. A rows and token inputs are
// loaded two blocks ahead (one block's substitution is shorter than a load's round trip). The
// reads, which nothing in the substitution needs, follow for all token blocks at once (wave w
// takes blocks w mod 4): QK rows straight from global memory (VEC: C a multiple of 4, 16-byte
// loads), all of a block's in flight together, times the dv tile in LDS.
template <bool VEC>
__global__ void __launch_bounds__(256) read_solve_kernel(ReadArgs a) {
    extern __shared__ float lds[];
    const int C = a.C;
    const int nblk = (C + kSB - 1) / kSB;
    const int rows = nblk * kSB;
    const int ld = panel_ld(C);
    float* sT = lds;                       // [rows][kTLd]: row t holds row (t mod 16) of its block's inverse
    float* sdv = sT + rows * kTLd;         // [rows][kTLd]: dv of every token, the block's 16 columns
    float* sA = sdv + rows * kTLd;         // kPanels x [16][ld]: token block b's A rows in panel b mod kPanels
    float* spart = sA + kPanels * kSB * ld;   // [kMW][16][kTLd]: per wave, its share of the earlier blocks' terms
    const int tid = static_cast<int>(threadIdx.x);
    const int wv = tid / kWave, l = tid % kWave;
    const int g = l / kSB, m = l % kSB;    // lane group (k / D row quarter), lane in group
    const int sr = tid / kSB, sl = tid % kSB;   // staging / inverse lanes: row (block) sr, lane sl
    // Block b is (chunk b mod P, column group b / P): consecutive blocks go round the XCDs, so a
    // chunk's column groups share an XCD's L2 when P is a multiple of 8.
    const int p = static_cast<int>(blockIdx.x) % a.P;
    const int col = (static_cast<int>(blockIdx.x) / a.P) * kSB + m;   // this lane's column
    const bool col_ok = col < a.hd;
    const int64_t c = a.chunk0 + p;
    const int tv = c >= a.first_partial ? a.valid_last : C;
    const float* A = a.a + c * C * C;
    const float* QK = a.qk + c * C * C;
    const float* beta = a.beta + c * C;
    const int64_t rbase = a.row0 + static_cast<int64_t>(p) * C;

    // Panel rows of token block b (row sr, columns sl + 16u up to the block's diagonal; zero past
    // C or past the last block) and, for wave 0, its lanes' token inputs (D rows b0 + 4g + r).
    struct Ahead {
        float a[kSB];
        float p0[4], v[4], bt[4];
    };
    auto fetch = [&](int b, Ahead& f) {
        const int b0 = b * kSB;
        const int tr = b0 + sr;
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            const int j = sl + kSB * u;
            f.a[u] = (b < nblk && tr < C && u <= b && j < C) ? A[static_cast<int64_t>(tr) * C + j] : 0.0f;
        }
        if (wv == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = b0 + 4 * g + r;
                const bool ok = b < nblk && t < tv && col_ok;
                const int64_t o = (rbase + (ok ? t : 0)) * a.hd + (col_ok ? col : 0);
                f.p0[r] = ok ? a.pred[o] : 0.0f;
                f.v[r] = ok ? a.v[o] : 0.0f;
                f.bt[r] = ok ? beta[t] : 0.0f;
            }
        }
    };
    auto stage = [&](int b, const Ahead& f) {   // block b's panel into its ring slot
        float* pan = sA + (b % kPanels) * kSB * ld;
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            if (u <= b) pan[sr * ld + sl + kSB * u] = f.a[u];   // columns up to the block's diagonal
        }
    };
    Ahead f0, f1, f2;   // blocks b, b + 1, b + 2
    fetch(0, f0);
    fetch(1, f1);

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
            float sacc = 0.0f;
#pragma unroll
            for (int k = 0; k < i; ++k) sacc = fmaf(al[i][k], x[k], sacc);
            x[i] = (i == sl ? 1.0f : 0.0f) - bt[i] * sacc;
            sT[(t0 + i) * kTLd + sl] = t0 + i < C ? x[i] : 0.0f;
        }
    }
    stage(0, f0);

    // One token block of the substitution: cur holds block b's token inputs, nxt block b + 1's
    // panel (loaded a block ago) and nxt2 receives block b + 2's loads. The three register sets
    // rotate by unrolling (a copy between them would wait for the loads in flight).
    auto solve_block = [&](int b, const Ahead& cur, const Ahead& nxt, Ahead& nxt2) {
        const int b0 = b * kSB;
        const float* pan = sA + (b % kPanels) * kSB * ld;
        // Block b + 1's panel goes into its slot now, and block b + 2's loads are issued. Block
        // b + 1's slot last held block b - 2, read before the barriers of block b - 1.
        if (b + 1 < nblk) stage(b + 1, nxt);
        fetch(b + 2, nxt2);
        lds_barrier();   // panel b and every earlier block's dv are in LDS
        // This wave's share of A[block, :b0] dv.
        floatx4 part = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int j = wv; j < b; j += kMW) part = block_times_dv(pan, ld, j, sdv, g, m, part);
#pragma unroll
        for (int r = 0; r < 4; ++r) spart[(wv * kSB + 4 * g + r) * kTLd + m] = part[r];
        lds_barrier();   // the partial tiles are in LDS
        if (wv == 0) {
            float far[4], rhs[4];
            bool ok[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * g + r;
                far[r] = ((spart[row * kTLd + m] + spart[(kSB + row) * kTLd + m]) + spart[(2 * kSB + row) * kTLd + m]) +
                         spart[(3 * kSB + row) * kTLd + m];
                ok[r] = b0 + row < tv && col_ok;
                rhs[r] = ok[r] ? cur.bt[r] * ((cur.v[r] - cur.p0[r]) - far[r]) : 0.0f;
            }
            // dv = (block inverse) x (right-hand sides): the B operand of step s is the lane's own
            // register s (k = 4 g + s).
            floatx4 x = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) x = mfma4(sT[(b0 + m) * kTLd + 4 * g + s], rhs[s], x);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[r] = ok[r] ? x[r] : 0.0f;
                sdv[(b0 + 4 * g + r) * kTLd + m] = x[r];
            }
            // pred: the block's own A terms (B operand again the lane's registers).
            floatx4 near = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) near = mfma4(pan[m * ld + b0 + 4 * g + s], x[s], near);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = b0 + 4 * g + r;
                if (t < C && col_ok) {
                    const int64_t o = (rbase + t) * a.hd + col;
                    a.dv[o] = x[r];
                    a.pred[o] = ok[r] ? (cur.p0[r] + far[r]) + near[r] : 0.0f;
                }
            }
        }
    };
    for (int b = 0; b < nblk; b += 3) {
        solve_block(b, f0, f1, f2);
        if (b + 1 < nblk) solve_block(b + 1, f1, f2, f0);
        if (b + 2 < nblk) solve_block(b + 2, f2, f0, f1);
    }
    lds_barrier();   // dv of every token is in LDS
    // read = q0 + QK[block, :b0+16] dv, token blocks w mod 4, two blocks' QK rows and q0 in flight
    // together; each block's terms in order of the earlier blocks.
    struct QRows {
        float q[kSB][4];
        float q0[4];
    };
    auto load_q = [&](int b, QRows& f) {   // (b >= nblk: zeros, nothing loaded)
        const int b0 = b * kSB;
        const int tr = b0 + m;   // the QK row this lane gives
        const float* qrow = QK + static_cast<int64_t>(tr < C ? tr : 0) * C;
#pragma unroll
        for (int j = 0; j < kSB; ++j) {
            const int k0 = j * kSB + 4 * g;
            const bool in = b < nblk && tr < C && j <= b;
            if constexpr (VEC) {
                const floatx4 v4 = in && k0 < C ? *reinterpret_cast<const floatx4*>(qrow + k0) : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < 4; ++s) f.q[j][s] = v4[s];
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) f.q[j][s] = in && k0 + s < C ? qrow[k0 + s] : 0.0f;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = b0 + 4 * g + r;
            f.q0[r] = (b < nblk && t < C && col_ok) ? a.read[(rbase + t) * a.hd + col] : 0.0f;
        }
    };
    auto read_block = [&](int b, const QRows& f) {
        const int b0 = b * kSB;
        floatx4 rd = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < kSB; ++j) {
            if (j <= b) {   // (block-uniform)
                const float* dcol = sdv + (j * kSB + 4 * g) * kTLd + m;
#pragma unroll
                for (int s = 0; s < 4; ++s) rd = mfma4(f.q[j][s], dcol[s * kTLd], rd);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = b0 + 4 * g + r;
            if (t < C && col_ok) a.read[(rbase + t) * a.hd + col] = t < tv ? f.q0[r] + rd[r] : 0.0f;
        }
    };
    for (int b = wv; b < nblk; b += 2 * kMW) {
        QRows fa, fb;
        load_q(b, fa);
        load_q(b + kMW, fb);
        read_block(b, fa);
        if (b + kMW < nblk) read_block(b + kMW, fb);
    }
}

template <bool TAIL>
const void* gather_fn(bool bf16, bool id64) {
    return bf16 ? (id64 ? reinterpret_cast<const void*>(&read_gather_kernel<true, true, TAIL>)
                        : reinterpret_cast<const void*>(&read_gather_kernel<true, false, TAIL>))
                : (id64 ? reinterpret_cast<const void*>(&read_gather_kernel<false, true, TAIL>)
                        : reinterpret_cast<const void*>(&read_gather_kernel<false, false, TAIL>));
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
    a.vbf = io->val_bytes == 2 ? 1 : 0;
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
    const void* g = io->hd % kGCols != 0 ? gather_fn<true>(io->bank_dtype == SDM_BF16, id64)
                                         : gather_fn<false>(io->bank_dtype == SDM_BF16, id64);
    hipError_t e = hipExtLaunchKernel(g, dim3(static_cast<unsigned>(a.P * tok_blocks * col_blocks)), dim3(256), kargs, 0,
                                      st, ev[0], ev[1], 0);
    if (e != hipSuccess) return e;
    const int solve_blocks = a.P * ((a.hd + kSB - 1) / kSB);
    const size_t lds = solve_lds_bytes(a.C);
    const void* sf = a.C % 4 == 0 ? reinterpret_cast<const void*>(&read_solve_kernel<true>)
                                  : reinterpret_cast<const void*>(&read_solve_kernel<false>);
    return hipExtLaunchKernel(sf, dim3(static_cast<unsigned>(solve_blocks)), dim3(256), kargs, lds, st, ev[2], ev[3], 0);
}

int read_lds_kernels(const void** fns, int cap) {
    if (cap < 2) return 0;
    fns[0] = reinterpret_cast<const void*>(&read_solve_kernel<true>);
    fns[1] = reinterpret_cast<const void*>(&read_solve_kernel<false>);
    return 2;
}

}  // namespace sdm
